// Uncompressed decode baseline for gfx950: attention over bf16 K/V caches,
// for comparison with the compressed decode ([WD] "Os numeros que importam":
// the speed-ups the pages report are against keys kept unquantized).
//
// Same structure as the compressed split-K pass, without any decoding: the
// context is cut into splits, each workgroup runs four waves over 32-token
// tiles of one (batch, kv head) and up to 16 query heads, and a combine
// kernel merges the splits by log-sum-exp.
//
// Layouts (this library's choice, as for the compressed caches):
//   K  bf16 [rows][d], token-major (a KV head's rows are [bh * cap, bh * cap + cap)),
//   V  bf16 [rows / 32][d][32], channel-major inside each 32-row block.
// With these, both MFMA operands of a tile come straight from 16-byte loads:
// the logit product takes 8 consecutive channels of a token (K rows), the
// value product 8 consecutive tokens of a channel (V block rows).
//
// Logits: v_mfma_f32_16x16x32_bf16 as (32 tokens x channels).(channels x 16
// heads) with the query, scaled by scale * log2(e), split into bf16 hi and lo
// parts (two products), so the logits carry fp32-grade query precision.
// Softmax weights are likewise split into bf16 hi and lo parts for the value
// product (channels x tokens).(tokens x heads). Online softmax with an
// integer log2 reference (results do not depend on the split count beyond
// the order of fp32 sums). Rows past n_ctx in the last tile are ignored
// whatever they hold: their logits are masked and their V values zeroed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "turboquant.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kWaves = 4;
constexpr int kHeads = 16;  // query heads per workgroup (MFMA columns)
constexpr int kMaxSplit = 1024;
constexpr int kTargetWorkgroups = 512;  // 2 per CU on a 256-CU MI355X
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// hi and lo bf16 parts of two values, packed as (v0, v1) pairs
__device__ __forceinline__ void split_pair(float v0, float v1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h0 = bf16_bits(v0), h1 = bf16_bits(v1);
  hi = h0 | (h1 << 16);
  lo = bf16_bits(v0 - bf16_value(h0)) | (bf16_bits(v1 - bf16_value(h1)) << 16);
}

// max / sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct BArgs {
  int batch, hq, hkv, group, n_split;
  int64_t n_ctx, cap;
  float scale_l2;  // scale * log2(e)
  const void* q;
  int q_bf16;
  const uint16_t* k;
  const uint16_t* v;
  float* logits;  // [batch, hq, n_ctx] or null
  float* part;    // [batch * hq][n_split][2 + d]
};

// One 32-token tile as this lane loads it: K rows of the logit product (two
// halves of 16 tokens, 32 channels each) and V block rows of the value
// product (8 tokens of 8 channels).
struct Tile {
  u32x4 k[2][4];
  u32x4 v[kD / 16];
};

// Tile at rows row0 .. row0 + 31 of a KV head (row0 a multiple of 32). Lane
// (ln, lg): logit-product row ln <-> token 8 (ln / 4) + 4 tau + ln % 4,
// channels [32 lg, 32 lg + 32); value-product row ln of 16-channel tile u <->
// channel 16 u + ln, tokens [8 lg, 8 lg + 8).
__device__ __forceinline__ void load_tile(const BArgs& a, int64_t row0, int ln, int lg, Tile& t) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int tok = 8 * (ln >> 2) + 4 * tau + (ln & 3);
    const u32x4* p = reinterpret_cast<const u32x4*>(a.k + (row0 + tok) * kD + 32 * lg);
#pragma unroll
    for (int c = 0; c < 4; ++c) t.k[tau][c] = p[c];
  }
  const uint16_t* vb = a.v + (row0 / 32) * (int64_t)(kD * 32);
#pragma unroll
  for (int u = 0; u < kD / 16; ++u) t.v[u] = *reinterpret_cast<const u32x4*>(vb + (16 * u + ln) * 32 + 8 * lg);
}

__global__ __launch_bounds__(256, 2) void bf16_split_kernel(BArgs a) {
  constexpr int NMT = kD / 16;
  constexpr int DP = kD + 1, REG = kHeads * DP;  // merge buffer: [2][heads][d + 1]
  __shared__ float s_red[2 * REG];
  __shared__ float s_m[kWaves][kHeads];
  __shared__ float s_lw[kWaves][kHeads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int hblk = blockIdx.z;
  const int b = bh / a.hkv;
  const int kvh = bh % a.hkv;

  const int64_t N = a.n_ctx;
  const int64_t n_tiles = (N + kTile - 1) / kTile;
  const int64_t tps = (n_tiles + a.n_split - 1) / a.n_split;
  const int64_t t_begin = split * tps;
  const int64_t t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;
  const int64_t rowbase = (int64_t)bh * a.cap;

  // ---- this lane's query head (column ln) and its operands: channels
  // [32 lg + 8 c, 32 lg + 8 c + 8) of chunk c, times scale * log2(e), as bf16
  // hi and lo parts (loaded before the first tile: loads complete in order) ----
  const int hloc = hblk * kHeads + ln;
  const bool hvalid = hloc < a.group;
  const int hq = kvh * a.group + (hvalid ? hloc : 0);
  u32x4 qhi[4], qlo[4];
  {
    float qv[32];
    const int64_t q0 = ((int64_t)b * a.hq + hq) * kD + 32 * lg;
    if (a.q_bf16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + q0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 w = p[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
          qv[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.q) + q0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 w = p[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * c + e] = w[e];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hi, lo;
        split_pair(qv[8 * c + 2 * e] * a.scale_l2, qv[8 * c + 2 * e + 1] * a.scale_l2, hi, lo);
        qhi[c][e] = hvalid ? hi : 0u;
        qlo[c][e] = hvalid ? lo : 0u;
      }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NMT];
#pragma unroll
  for (int u = 0; u < NMT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Tile& t, int64_t T0) __attribute__((always_inline)) {
    const bool full = T0 + kTile <= N;
    const int nvt = full ? kTile : (int)(N - T0);  // tokens of the tile before n_ctx
    // ---- logits (log2 domain): lane (head ln, lg) gets tokens 8 lg + j ----
    float l2[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = mfma_bf16(t.k[tau][c], qhi[c], s);
        s = mfma_bf16(t.k[tau][c], qlo[c], s);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) l2[4 * tau + i] = s[i];
    }
    if (a.logits) {
      if (hvalid) {
        float* lp = a.logits + ((int64_t)b * a.hq + hq) * N + T0 + 8 * lg;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * lg + j < nvt) lp[j] = l2[j] * kLn2;
      }
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) l2[j] = 8 * lg + j < nvt ? l2[j] : -INFINITY;
    }
    // ---- online softmax (integer reference: exact power-of-two rescales) ----
    float mx = l2[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, l2[j]);
    mx = rows4_max(mx);
    const float m_new = fmaxf(m_run, ceilf(mx));
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int u = 0; u < NMT; ++u) acc[u] *= corr;
      m_run = m_new;
    }
    float p[8], psum;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(l2[j] - m_run);
      psum = j == 0 ? p[j] : psum + p[j];
    }
    l_run += psum;
    u32x4 phi, plo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t hi, lo;
      split_pair(p[2 * e], p[2 * e + 1], hi, lo);
      phi[e] = hi;
      plo[e] = lo;
    }
    // ---- V: rows past n_ctx are zeroed (they may hold anything) ----
    uint32_t vmask[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vmask[e] = (8 * lg + 2 * e < nvt ? 0x0000FFFFu : 0u) | (8 * lg + 2 * e + 1 < nvt ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int u = 0; u < NMT; ++u) {
      u32x4 va = t.v[u];
      if (!full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) va[e] &= vmask[e];
      }
      acc[u] = mfma_bf16(va, phi, acc[u]);
      acc[u] = mfma_bf16(va, plo, acc[u]);
    }
  };

  // ---- tiles: one in flight while one is computed ----
  int64_t tile = t_begin + wv;
  Tile ta, tb;
  load_tile(a, rowbase + (tile < t_end ? tile : 0) * kTile, ln, lg, ta);
  if (tile < t_end) {
    const int64_t last = t_end - 1 - ((t_end - 1 - tile) % kWaves);
    auto next = [&](int64_t t) { return t + kWaves <= last ? t + kWaves : last; };
    for (;;) {
      load_tile(a, rowbase + next(tile) * kTile, ln, lg, tb);
      compute(ta, tile * kTile);
      if (tile == last) break;
      tile += kWaves;
      load_tile(a, rowbase + next(tile) * kTile, ln, lg, ta);
      compute(tb, tile * kTile);
      if (tile == last) break;
      tile += kWaves;
    }
  }

  // ---- merge the four waves into one partial per head ----
  // region r holds waves r and r + 2, scaled to the workgroup maximum
  l_run = rows4_sum(l_run);
  if (lg == 0) s_m[wv][ln] = m_run;
  __syncthreads();
  float M = s_m[0][ln];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][ln]);
  const float e = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  if (lg == 0) s_lw[wv][ln] = l_run * e;
  float* reg = s_red + (wv & 1) * REG + ln * DP;
  if (wv < 2) {
#pragma unroll
    for (int u = 0; u < NMT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[16 * u + 4 * lg + i] = acc[u][i] * e;
  }
  __syncthreads();
  if (wv >= 2) {
#pragma unroll
    for (int u = 0; u < NMT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[16 * u + 4 * lg + i] += acc[u][i] * e;
  }
  __syncthreads();
  // partial of every valid head: [max (log2 domain), sum, acc[d]]
  const int nh = a.group - hblk * kHeads < kHeads ? a.group - hblk * kHeads : kHeads;
  for (int e2 = tid; e2 < nh * (2 + kD); e2 += 256) {
    const int h = e2 / (2 + kD), k = e2 % (2 + kD);
    float val;
    if (k < 2) {
      float Mh = s_m[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_m[w][h]);
      val = k == 0 ? Mh : s_lw[0][h] + s_lw[1][h] + s_lw[2][h] + s_lw[3][h];
    } else {
      val = s_red[h * DP + k - 2] + s_red[REG + h * DP + k - 2];
    }
    const int hq2 = kvh * a.group + hblk * kHeads + h;
    a.part[(((int64_t)b * a.hq + hq2) * a.n_split + split) * (2 + kD) + k] = val;
  }
}

// Merge of the splits of one query head per workgroup:
//   M = max_s m_s, w_s = 2^(m_s - M), out = sum_s w_s acc_s / sum_s w_s l_s.
// Threads (c, g): channel c, split group g = t / d sums the splits s = g mod 2.
__global__ __launch_bounds__(256) void bf16_combine_kernel(const float* part, int n_split, float* out) {
  constexpr int PS = 2 + kD;
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[4];
  __shared__ float s_acc[kD];
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const float* P = part + (int64_t)head * n_split * PS;
  float mx = -INFINITY;
  for (int s = t; s < n_split; s += 256) mx = fmaxf(mx, P[(int64_t)s * PS]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float lsum = 0.f;
  for (int s = t; s < n_split; s += 256) {
    const float ms = P[(int64_t)s * PS];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    s_w[s] = w;
    lsum += w * P[(int64_t)s * PS + 1];
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  if (lane == 0) s_red[wv] = lsum;
  __syncthreads();
  const float L = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const int c = t % kD, g = t / kD;
  float acc = 0.f;
#pragma unroll 8
  for (int s = g; s < n_split; s += 2) acc = fmaf(s_w[s], P[(int64_t)s * PS + 2 + c], acc);
  if (g == 1) s_acc[c] = acc;
  __syncthreads();
  if (g == 0) out[(int64_t)head * kD + c] = (acc + s_acc[c]) / L;
}

int choose_split(const tq_decode_shape* s, int n_hblk) {
  const int64_t n_tiles = (s->n_ctx + kTile - 1) / kTile;
  int64_t max_split = (n_tiles + kWaves - 1) / kWaves;  // at least one tile per wave
  if (max_split > kMaxSplit) max_split = kMaxSplit;
  if (max_split < 1) max_split = 1;
  if (s->n_split > 0) return (int)(s->n_split < max_split ? s->n_split : max_split);
  const int64_t per = (int64_t)s->batch * s->n_kv_heads * n_hblk;
  int64_t want = (kTargetWorkgroups + per - 1) / per;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

bool shape_ok(const tq_decode_shape* s) {
  if (!s) return false;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->n_q_heads < 1 || s->n_q_heads % s->n_kv_heads != 0) return false;
  if (s->n_ctx < 1 || s->cache_capacity < s->n_ctx || s->cache_capacity % 32 != 0 || s->n_split < 0) return false;
  if (s->n_q_tokens < 0) return false;
  return std::isfinite(s->scale);
}

size_t workspace_for(const tq_decode_shape* s, int n_split) {
  return (size_t)s->batch * s->n_q_heads * n_split * (2 + kD) * sizeof(float);
}

int n_hblk_of(const tq_decode_shape* s) {
  const int group = s->n_q_heads / s->n_kv_heads;
  return (group + kHeads - 1) / kHeads;
}

}  // namespace

extern "C" tq_status tq_attn_decode_bf16_workspace_bytes(const tq_decode_shape* shape, int d, size_t* bytes) {
  if (!bytes || !shape_ok(shape)) return TQ_ERR_INVALID;
  if (d != kD || shape->n_q_tokens > 1) return TQ_ERR_UNSUPPORTED;
  *bytes = workspace_for(shape, choose_split(shape, n_hblk_of(shape)));
  return TQ_OK;
}

extern "C" tq_status tq_attn_decode_bf16(const tq_decode_shape* shape, int d, const void* q, tq_dtype q_dtype,
                                         const void* k, const void* v, float* logits, float* out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (!shape_ok(shape) || !q || !k || !v || !out) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (d != kD || shape->n_q_tokens > 1) return TQ_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, out, workspace};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return TQ_ERR_INVALID;
  if (logits && reinterpret_cast<uintptr_t>(logits) % 4 != 0) return TQ_ERR_INVALID;
  const int n_hblk = n_hblk_of(shape);
  const int n_split = choose_split(shape, n_hblk);
  if (!workspace || workspace_bytes < workspace_for(shape, n_split)) return TQ_ERR_WORKSPACE;
  BArgs a{};
  a.batch = shape->batch;
  a.hq = shape->n_q_heads;
  a.hkv = shape->n_kv_heads;
  a.group = shape->n_q_heads / shape->n_kv_heads;
  a.n_split = n_split;
  a.n_ctx = shape->n_ctx;
  a.cap = shape->cache_capacity;
  a.scale_l2 = shape->scale * kLog2e;
  a.q = q;
  a.q_bf16 = q_dtype == TQ_BF16;
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.logits = logits;
  a.part = reinterpret_cast<float*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  hipLaunchKernelGGL(bf16_split_kernel, dim3((unsigned)n_split, (unsigned)(a.batch * a.hkv), (unsigned)n_hblk),
                     dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  hipLaunchKernelGGL(bf16_combine_kernel, dim3((unsigned)(a.batch * a.hq)), dim3(256), 0, st, a.part, n_split, out);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}
