// Decode-time attention over the compressed cache, for gfx950.
//
// [WD] introduction and "Os numeros que importam": the attention logits are
// computed from the compressed keys; the decode step then applies softmax
// and sums the dequantized values. [WD] "2. QJL Residual": the residual's
// 1-bit sketch corrects the inner-product bias, so each logit is the MSE
// part plus the sign-sketch part:
//   logit = scale * sum_g ( n_g <(rot q)_g, c[idx]> + alpha_g gamma_g <(sketch q)_g, z> ).
//
// Three kernels on the caller's stream:
//  1. prep:    q_rot = rot q and q_sk = sketch q per query head (fp32 sums,
//              stored as fp16 hi/lo pairs).
//  2. decode:  split-K over the context. A workgroup takes one (batch, KV head,
//              16-query-head block) and a range of 32-token tiles; its four
//              waves take alternate tiles. Per tile a wave
//              - expands the K codes through LDS pair tables (two fp16
//                centroids per lookup) and the K sign bits into fp16 +-1,
//              - forms both logit parts on v_mfma_f32_16x16x32_f16 (tokens x
//                channels times channels x heads), with centroids and
//                queries split into fp16 hi + lo parts so the products keep
//                fp32 accuracy, scales them by the token's norms, and runs
//                the online softmax,
//              - expands the V codes/signs the same way and accumulates
//                sum_t p_t n_t c[idx_t] and sum_t p_t gamma_t z_t on MFMA
//                (channels x tokens times tokens x heads): V is summed in the
//                rotated and sketch domains, never dequantized per token.
//              The MFMA output layout of the logits (lane = head, 8 tokens)
//              is exactly the operand layout the V product needs, so the
//              softmax weights never leave registers. The four waves merge
//              through LDS into one partial (max, sum, accumulators).
//  3. combine: log-sum-exp merge of the splits, then out = (rot^T acc_rot +
//              sketch^T (alpha acc_sk)) / sum: the back-transform runs once
//              per head, which is valid because dequantization is linear.
//
// Record formats: K rows are token-major (a token's codes for 8 consecutive
// channels are one 8m-bit field); V is stored in 32-token blocks where each
// octet of tokens keeps its 8 codes of a channel in one 8m-bit field. Both
// fields feed one lane's eight MFMA operand slots directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tq_internal.h"
#include "turboquant.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2))) __attribute__((aligned(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2a8 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Low parts of the split fp16 operands are stored times 2^11 (kLoScale) so
// they stay in the normal fp16 range; their products are scaled back by 2^-11.
constexpr float kLoScale = 2048.0f;
constexpr float kLoInv = 1.0f / 2048.0f;
constexpr int lowbit(int v) { return v & (-v); }
constexpr int kWaves = 4;
constexpr int kTile = 32;

struct DArgs {
  int batch, hq, hkv, group;  // group = hq / hkv
  int n_split;
  int64_t n_ctx, cap;
  float scale;
  const _Float16* qprep;  // [batch*hq][4d]: q_rot hi, q_rot lo*2^11, q_sk hi, q_sk lo*2^11
  const uint32_t* kc;
  const uint32_t* ks;
  const float* kn;
  const uint32_t* vc;
  const uint32_t* vs;
  const float* vn;
  const float* kcent;  // K centroids (concatenated over groups)
  const float* vcent;
  float* logits;  // [batch, hq, n_ctx] or null
  float* part;    // [batch*hq][n_split][2 + 2d]
};

__device__ __forceinline__ uint32_t h2bits(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 8 sign bits -> 8 fp16 values +1 (bit set) / -1 (bit clear), two per dword.
__device__ __forceinline__ u32x4 signs_to_pm1(uint32_t byte) {
  const uint32_t x = (~byte) & 0xFFu;
  const uint32_t x2 = x | (x << 16);
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // bit 2p to bit 15 of the low half, bit 2p+1 to bit 15 of the high half
    const u16x2 sh = {(uint16_t)(15 - 2 * p), (uint16_t)(14 - 2 * p)};
    const u16x2 y = __builtin_bit_cast(u16x2, x2) << sh;
    r[p] = (__builtin_bit_cast(uint32_t, y) & 0x80008000u) | 0x3C003C00u;
  }
  return r;
}

// 8 codes of M bits (one 8M-bit field, code s at bits [M s, M s + M)) ->
// 8 fp16 centroids through a pair table (entry = code_a | code_b << M).
template <int M>
__device__ __forceinline__ u32x4 codes_to_f16(uint32_t field, const uint32_t* lut) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) r[p] = lut[(field >> (2 * M * p)) & ((1u << (2 * M)) - 1u)];
  return r;
}

// Same as codes_to_f16 from a split table: entry e holds the fp16 pair of the
// centroids (hi) and the fp16 pair of their rounding remainders times 2^11
// (lo), so that hi + 2^-11 lo reproduces the fp32 centroid.
template <int M>
__device__ __forceinline__ void codes_to_f16_split(uint32_t field, const u32x2a8* lut, u32x4& hi,
                                                   u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u32x2a8 v = lut[(field >> (2 * M * p)) & ((1u << (2 * M)) - 1u)];
    hi[p] = v[0];
    lo[p] = v[1];
  }
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }

// Load NW consecutive 32-bit words starting at p, with p known to be aligned
// to ALIGN bytes.
template <int NW, int ALIGN>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t* out) {
  if constexpr (ALIGN >= 16 && NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
      out[4 * i] = v[0];
      out[4 * i + 1] = v[1];
      out[4 * i + 2] = v[2];
      out[4 * i + 3] = v[3];
    }
  } else if constexpr (ALIGN >= 8 && NW % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 2; ++i) {
      const u32x2a4 v = reinterpret_cast<const u32x2a4*>(p)[i];
      out[2 * i] = v[0];
      out[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) out[i] = p[i];
  }
}

// Norms (n_g, gamma_g) of 8 consecutive rows; p is 16-byte aligned.
template <int NG>
__device__ __forceinline__ void load_norms(const float* p, float (&out)[8][2 * NG]) {
#pragma unroll
  for (int i = 0; i < 4 * NG; ++i) {
    const f32x4 v = reinterpret_cast<const f32x4*>(p)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int flat = 4 * i + e;
      out[flat / (2 * NG)][flat % (2 * NG)] = v[e];
    }
  }
}

// bits [pos, pos + width) of a word array; pos and width are compile-time
// constants after unrolling (width <= 32)
__device__ __forceinline__ uint32_t field_at(const uint32_t* w, int pos, int width) {
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + width > 32) v |= w[wi + 1] << (32 - sh);
  if (width < 32) v &= (1u << width) - 1u;
  return v;
}

// One group's V contribution for one 32-token tile. The lane (row ln, octet
// lg) owns channels RUN ln + u, u < RUN, of the group; for each u it expands
// the 8 codes and 8 sign bits of its octet's tokens at that channel and adds
// (V tile MT0 + u) += codes^T x P'_rot and signs^T x P'_sketch.
template <int M, int RUN, int MT0, int NMT>
__device__ __forceinline__ void v_accumulate(const uint32_t* cw, const uint32_t* sw,
                                             const uint32_t* lut, u32x4 pr, u32x4 pz,
                                             f32x4 (&acc_r)[NMT], f32x4 (&acc_s)[NMT]) {
#pragma unroll
  for (int u = 0; u < RUN; ++u) {
    const uint32_t field = field_at(cw, 8 * M * u, 8 * M);
    const u32x4 av = codes_to_f16<M>(field, lut);
    const uint32_t sbyte = (sw[u >> 2] >> (8 * (u & 3))) & 0xFFu;
    const u32x4 az = signs_to_pm1(sbyte);
    acc_r[MT0 + u] = mfma16(av, pr, acc_r[MT0 + u]);
    acc_s[MT0 + u] = mfma16(az, pz, acc_s[MT0 + u]);
  }
}

// Loads the lane's V code and sign words of one group and accumulates.
template <int M, int RUN, int DG, int MT0, int NMT>
__device__ __forceinline__ void v_group(const uint32_t* cb, const uint32_t* sb, int lg, int ln,
                                        const uint32_t* lut, u32x4 pr, u32x4 pz,
                                        f32x4 (&acc_r)[NMT], f32x4 (&acc_s)[NMT]) {
  constexpr int NWC = (RUN * M) / 4;  // 8 tokens x RUN channels x M bits / 32
  constexpr int ALC = lowbit(RUN * M) < 16 ? lowbit(RUN * M) : 16;
  constexpr int NWS = RUN / 4;
  constexpr int ALS = lowbit(RUN) < 16 ? lowbit(RUN) : 16;
  uint32_t cw[NWC + 1];
  load_words<NWC, ALC>(cb + (M * (lg * DG + RUN * ln)) / 4, cw);
  cw[NWC] = 0u;
  uint32_t swv[NWS];
  load_words<NWS, ALS>(sb + (lg * DG + RUN * ln) / 4, swv);
  v_accumulate<M, RUN, MT0, NMT>(cw, swv, lut, pr, pz, acc_r, acc_s);
}

template <int D, int NG, int M0, int M1, bool WV>
__global__ __launch_bounds__(256) void decode_kernel(DArgs a) {
  constexpr int DG = D / NG;     // channels per group
  constexpr int NC = D / 32;     // 32-channel chunks of the logit product
  constexpr int CPG = NC / NG;   // chunks per group
  constexpr int NMT = D / 16;    // 16-channel tiles of the V product
  constexpr int MTPG = NMT / NG; // V tiles per group
  constexpr int RUN = DG / 16;   // channels per lane in each group (V operand)
  constexpr int MB[2] = {M0, M1};
  // token-major word offsets of each group's codes / signs
  constexpr int CW0 = (M0 * DG + 31) / 32;
  constexpr int CW = CW0 + (NG > 1 ? (M1 * DG + 31) / 32 : 0);
  constexpr int SW0 = (DG + 31) / 32;
  constexpr int SW = SW0 * NG;
  constexpr int CWOFF[2] = {0, CW0};
  constexpr int SWOFF[2] = {0, SW0};
  // block-record word offsets
  constexpr int BCW = M0 * DG + (NG > 1 ? M1 * DG : 0);
  constexpr int BCWOFF[2] = {0, M0 * DG};
  constexpr int BSW = D;
  constexpr int BSWOFF[2] = {0, DG};
  constexpr int LUT0 = 1 << (2 * M0);
  constexpr int LUT1 = NG > 1 ? 1 << (2 * M1) : 0;
  constexpr int LUTOFF[2] = {0, LUT0};

  __shared__ u32x2a8 klut[LUT0 + LUT1];
  __shared__ uint32_t vlut[WV ? LUT0 + LUT1 : 1];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[16];
  __shared__ float s_acc[WV ? 16 * 2 * D : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;  // b * hkv + kv head
  const int hblk = blockIdx.z;
  const int b = bh / a.hkv;
  const int kvh = bh % a.hkv;

  // ---- pair tables: entry e -> (c[e & (L-1)], c[e >> M]) as two fp16 ----
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int m = MB[g];
    const int L = 1 << m;
    const int coff = g == 0 ? 0 : (1 << M0);
    for (int e = tid; e < (1 << (2 * m)); e += 256) {
      const float c0 = a.kcent[coff + (e & (L - 1))], c1 = a.kcent[coff + (e >> m)];
      const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
      klut[LUTOFF[g] + e] = u32x2a8{h2bits(c0, c1),
                                    h2bits((c0 - (float)h0) * kLoScale, (c1 - (float)h1) * kLoScale)};
      if constexpr (WV) vlut[LUTOFF[g] + e] = h2bits(a.vcent[coff + (e & (L - 1))], a.vcent[coff + (e >> m)]);
    }
  }
  if constexpr (WV) {
    for (int e = tid; e < 16 * 2 * D; e += 256) s_acc[e] = 0.f;
    if (tid < 16) s_l[tid] = 0.f;
  }

  // ---- this lane's head and its query operands (B operand: channels x heads) ----
  const int hloc = hblk * 16 + ln;  // head index within the KV group
  const bool hvalid = hloc < a.group;
  const int hq = kvh * a.group + hloc;
  u32x4 qr[NC], qrl[NC], qs[NC], qsl[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (hvalid) {
      const _Float16* qp = a.qprep + ((int64_t)b * a.hq + hq) * (4 * D) + 32 * c + 8 * lg;
      qr[c] = *reinterpret_cast<const u32x4*>(qp);
      qrl[c] = *reinterpret_cast<const u32x4*>(qp + D);
      qs[c] = *reinterpret_cast<const u32x4*>(qp + 2 * D);
      qsl[c] = *reinterpret_cast<const u32x4*>(qp + 3 * D);
    } else {
      qr[c] = qrl[c] = qs[c] = qsl[c] = u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();

  const float alpha[2] = {sqrtf(0.5f * (float)M_PI) / (float)DG, sqrtf(0.5f * (float)M_PI) / (float)DG};
  const int64_t N = a.n_ctx;
  const int64_t n_tiles = (N + kTile - 1) / kTile;
  const int64_t tps = (n_tiles + a.n_split - 1) / a.n_split;
  const int64_t t_begin = split * tps;
  const int64_t t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;
  const int64_t rowbase = (int64_t)bh * a.cap;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_r[WV ? NMT : 1], acc_s[WV ? NMT : 1];
#pragma unroll
  for (int v = 0; v < (WV ? NMT : 1); ++v) {
    acc_r[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc_s[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int64_t tile = t_begin + wv; tile < t_end; tile += kWaves) {
    const int64_t T0 = tile * kTile;
    // ---------------- K: logits ----------------
    // hi and lo (x 2^11) accumulators of the MSE part and of the sketch part
    f32x4 lr[2][NG], lrl[2][NG], ls[2][NG], lsl[2][NG];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      // A operand row ln <-> token 8 (ln / 4) + 4 tau + ln % 4 of the tile
      const int64_t row = rowbase + T0 + 8 * (ln >> 2) + 4 * tau + (ln & 3);
      const uint32_t* crow = a.kc + row * CW;
      const uint32_t* srow = a.ks + row * SW;
      uint32_t sw[SW];
      load_words<SW, (SW * 4) % 16 == 0 ? 16 : 4>(srow, sw);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        lr[tau][g] = lrl[tau][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        ls[tau][g] = lsl[tau][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int g = c / CPG;
        const int m = MB[g];
        // channels 32 (c % CPG) + 8 lg .. + 7 of group g: 8m bits at this bit offset
        const int bit = 32 * CWOFF[g] + m * (32 * (c % CPG) + 8 * lg);
        const uint32_t* wp = crow + (bit >> 5);
        const int sh = bit & 31;
        uint32_t field = wp[0] >> sh;
        if (sh + 8 * m > 32) field |= wp[1] << (32 - sh);
        u32x4 ak, akl;
        if (g == 0)
          codes_to_f16_split<M0>(field, klut, ak, akl);
        else
          codes_to_f16_split<M1>(field, klut + LUT0, ak, akl);
        const uint32_t sbyte = (sw[SWOFF[g] + (c % CPG)] >> (8 * lg)) & 0xFFu;
        const u32x4 az = signs_to_pm1(sbyte);
        // c q = c_hi q_hi + 2^-11 (c_lo' q_hi + c_hi q_lo'), products exact, fp32 sums
        lr[tau][g] = mfma16(ak, qr[c], lr[tau][g]);
        lrl[tau][g] = mfma16(akl, qr[c], lrl[tau][g]);
        lrl[tau][g] = mfma16(ak, qrl[c], lrl[tau][g]);
        ls[tau][g] = mfma16(az, qs[c], ls[tau][g]);
        lsl[tau][g] = mfma16(az, qsl[c], lsl[tau][g]);
      }
    }
    // lane (head ln, lg) now holds tokens 8 lg + j, j = 4 tau + i
    const int64_t tok0 = T0 + 8 * lg;
    float kn[8][2 * NG];
    load_norms<NG>(a.kn + (rowbase + tok0) * (2 * NG), kn);
    float l2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tau = j >> 2, i = j & 3;
      float s = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g)
        s += kn[j][2 * g] * fmaf(kLoInv, lrl[tau][g][i], lr[tau][g][i]) +
             alpha[g] * kn[j][2 * g + 1] * fmaf(kLoInv, lsl[tau][g][i], ls[tau][g][i]);
      const float lg_val = a.scale * s;
      const bool ok = tok0 + j < N;
      if (a.logits && hvalid && ok)
        a.logits[((int64_t)b * a.hq + hq) * N + tok0 + j] = lg_val;
      l2[j] = ok ? lg_val * kLog2e : -INFINITY;
    }
    if constexpr (WV) {
      // ---------------- online softmax ----------------
      float mx = l2[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, l2[j]);
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2f(m_run - m_new);
      m_run = m_new;
      float p[8], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = exp2f(l2[j] - m_new);
        psum += p[j];
      }
      l_run = l_run * corr + psum;
#pragma unroll
      for (int v = 0; v < NMT; ++v) {
        acc_r[v] *= corr;
        acc_s[v] *= corr;
      }
      // B operands of the V product: slot j <-> token 8 lg + j
      float vn[8][2 * NG];
      load_norms<NG>(a.vn + (rowbase + tok0) * (2 * NG), vn);
      u32x4 pr[NG], pz[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j0 = 2 * q, j1 = 2 * q + 1;
          const bool ok0 = tok0 + j0 < N, ok1 = tok0 + j1 < N;
          const float r0 = ok0 ? p[j0] * vn[j0][2 * g] : 0.f;
          const float r1 = ok1 ? p[j1] * vn[j1][2 * g] : 0.f;
          // alpha_g is applied once per head in the combine, not here
          const float z0 = ok0 ? p[j0] * vn[j0][2 * g + 1] : 0.f;
          const float z1 = ok1 ? p[j1] * vn[j1][2 * g + 1] : 0.f;
          pr[g][q] = h2bits(r0, r1);
          pz[g][q] = h2bits(z0, z1);
        }
      }
      // ---------------- V: accumulate in the rotated / sketch domains ----------------
      const int64_t blk = (rowbase + T0) / 32;
      v_group<M0, RUN, DG, 0, NMT>(a.vc + blk * BCW + BCWOFF[0], a.vs + blk * BSW + BSWOFF[0], lg,
                                   ln, vlut, pr[0], pz[0], acc_r, acc_s);
      if constexpr (NG > 1)
        v_group<M1, RUN, DG, MTPG, NMT>(a.vc + blk * BCW + BCWOFF[1], a.vs + blk * BSW + BSWOFF[1],
                                        lg, ln, vlut + LUT0, pr[1], pz[1], acc_r, acc_s);
    }
  }

  if constexpr (WV) {
    // ---- merge the four waves into one partial ----
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (lg == 0) s_m[wv][ln] = m_run;
    __syncthreads();
    float M = s_m[0][ln];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][ln]);
    const float e = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
    if (lg == 0) atomicAdd(&s_l[ln], l_run * e);
#pragma unroll
    for (int v = 0; v < NMT; ++v) {
      const int g = v / MTPG;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // accumulator row 4 lg + i of V tile v <-> channel of group g
        const int ch = g * DG + RUN * (4 * lg + i) + (v % MTPG);
        atomicAdd(&s_acc[ln * 2 * D + ch], acc_r[v][i] * e);
        atomicAdd(&s_acc[ln * 2 * D + D + ch], acc_s[v][i] * e);
      }
    }
    __syncthreads();
    // write the partial of every valid head: [max (log2 domain), sum, acc_rot[D], acc_sk[D]]
    const int nh = a.group - hblk * 16 < 16 ? a.group - hblk * 16 : 16;
    for (int e2 = tid; e2 < nh * (2 + 2 * D); e2 += 256) {
      const int h = e2 / (2 + 2 * D), k = e2 % (2 + 2 * D);
      float Mh = s_m[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_m[w][h]);
      const float val = k == 0 ? Mh : (k == 1 ? s_l[h] : s_acc[h * 2 * D + k - 2]);
      const int hq2 = kvh * a.group + hblk * 16 + h;
      a.part[(((int64_t)b * a.hq + hq2) * a.n_split + split) * (2 + 2 * D) + k] = val;
    }
  }
}


// ---------------------------------------------------------------------------
// Query preparation: q_rot = rot q, q_sk = sketch q (fp32 sums), each stored
// as an fp16 pair (hi, (q - hi) * 2^11) so the logit products keep fp32 accuracy.
// Thread t computes output channel t % D of matrix t / D for kPrepHeads heads.
// ---------------------------------------------------------------------------
constexpr int kPrepHeads = 4;

template <int D>
__global__ __launch_bounds__(2 * D) void prep_kernel(const void* q, int q_bf16, int n_heads,
                                                     const float* rot, const float* sketch,
                                                     _Float16* qprep) {
  __shared__ float sq[kPrepHeads][D];
  const int h0 = blockIdx.x * kPrepHeads;
  const int t = threadIdx.x;
  for (int e = t; e < kPrepHeads * D; e += 2 * D) {
    const int h = h0 + e / D, k = e % D;
    float v = 0.f;
    if (h < n_heads) {
      const int64_t off = (int64_t)h * D + k;
      v = q_bf16 ? __uint_as_float(((uint32_t) reinterpret_cast<const uint16_t*>(q)[off]) << 16)
                 : reinterpret_cast<const float*>(q)[off];
    }
    sq[e / D][k] = v;
  }
  __syncthreads();
  const int half = t / D, i = t % D;
  const float* row = (half == 0 ? rot : sketch) + (int64_t)i * D;
  float acc[kPrepHeads] = {};
  for (int k = 0; k < D; ++k) {
    const float mk = row[k];
#pragma unroll
    for (int h = 0; h < kPrepHeads; ++h) acc[h] = fmaf(mk, sq[h][k], acc[h]);
  }
#pragma unroll
  for (int h = 0; h < kPrepHeads; ++h)
    if (h0 + h < n_heads) {
      const _Float16 hi = (_Float16)acc[h];
      const _Float16 lo = (_Float16)((acc[h] - (float)hi) * kLoScale);
      _Float16* dst = qprep + (int64_t)(h0 + h) * 4 * D + half * 2 * D + i;
      dst[0] = hi;
      dst[D] = lo;
    }
}

// ---------------------------------------------------------------------------
// Split merge and back-transform, one block per query head:
//   M = max_s m_s, w_s = 2^(m_s - M), L = sum_s w_s l_s, acc = sum_s w_s acc_s,
//   out = (rot^T acc_rot + sketch^T (alpha_g acc_sk)) / L.
// ---------------------------------------------------------------------------
constexpr int kMaxSplit = 1024;

template <int D>
__global__ __launch_bounds__(2 * D) void combine_kernel(const float* part, int n_split,
                                                        const float* rot, const float* sketch,
                                                        int group_dim0, float* out) {
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_acc[2 * D];
  __shared__ float s_o[2 * D];
  __shared__ float s_red[2 * D / 64];
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  constexpr int NW = 2 * D / 64;
  const float* P = part + (int64_t)head * n_split * (2 + 2 * D);
  // max over splits
  float mx = -INFINITY;
  for (int s = t; s < n_split; s += 2 * D) mx = fmaxf(mx, P[(int64_t)s * (2 + 2 * D)]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  float M = s_red[0];
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();
  // weights and the total sum
  float lsum = 0.f;
  for (int s = t; s < n_split; s += 2 * D) {
    const float ms = P[(int64_t)s * (2 + 2 * D)];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    s_w[s] = w;
    lsum += w * P[(int64_t)s * (2 + 2 * D) + 1];
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  if (lane == 0) s_red[wv] = lsum;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < NW; ++w) L += s_red[w];
  // merged accumulators; alpha_g is applied to the sketch half here
  {
    float acc = 0.f;
    for (int s = 0; s < n_split; ++s) acc = fmaf(s_w[s], P[(int64_t)s * (2 + 2 * D) + 2 + t], acc);
    if (t >= D) {
      const int j = t - D;
      const int dg = j < group_dim0 ? group_dim0 : D - group_dim0;
      acc *= sqrtf(0.5f * (float)M_PI) / (float)dg;
    }
    s_acc[t] = acc;
  }
  __syncthreads();
  // back-transform: o_half[i] = sum_j M_half[j][i] acc_half[j]
  {
    const int half = t / D, i = t % D;
    const float* mat = half == 0 ? rot : sketch;
    const float* av = s_acc + half * D;
    float o = 0.f;
    for (int j = 0; j < D; ++j) o = fmaf(mat[(int64_t)j * D + i], av[j], o);
    s_o[t] = o;
  }
  __syncthreads();
  if (t < D) out[(int64_t)head * D + t] = (s_o[t] + s_o[D + t]) / L;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kTargetWorkgroups = 512;  // 2 per CU on a 256-CU MI355X

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

bool same_layout(const tq_layout& a, const tq_layout& b) {
  if (a.d != b.d || a.n_groups != b.n_groups) return false;
  for (int g = 0; g < a.n_groups; ++g)
    if (a.group_dim[g] != b.group_dim[g] || a.mse_bits[g] != b.mse_bits[g]) return false;
  return true;
}

bool shape_valid(const tq_decode_shape* s) {
  if (!s) return false;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->n_q_heads < 1) return false;
  if (s->n_q_heads % s->n_kv_heads != 0) return false;
  if (s->n_ctx < 1 || s->cache_capacity < s->n_ctx || s->cache_capacity % 32 != 0) return false;
  if (s->n_split < 0) return false;
  if (!std::isfinite(s->scale)) return false;
  return true;
}

bool decode_supported(const tq_layout& l) {
  if (l.d != 128) return false;
  if (l.n_groups == 2 && (l.group_dim[0] != 64 || l.group_dim[1] != 64)) return false;
  return true;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t workspace_for(const tq_decode_shape* s, int d, bool with_v, int n_split) {
  const size_t heads = (size_t)s->batch * s->n_q_heads;
  size_t bytes = align256(heads * 4 * d * sizeof(_Float16));
  if (with_v) bytes += align256(heads * (size_t)n_split * (2 + 2 * d) * sizeof(float));
  return bytes;
}

template <int D, int NG, int M0, int M1, bool WV>
hipError_t launch_decode(const DArgs& a, int n_hblk, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, NG, M0, M1, WV>),
                     dim3((unsigned)a.n_split, (unsigned)(a.batch * a.hkv), (unsigned)n_hblk), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

template <int D, int NG, int M0, bool WV>
hipError_t dispatch_m1(const DArgs& a, int m1, int n_hblk, hipStream_t st) {
  switch (m1) {
    case 1: return launch_decode<D, NG, M0, 1, WV>(a, n_hblk, st);
    case 2: return launch_decode<D, NG, M0, 2, WV>(a, n_hblk, st);
    case 3: return launch_decode<D, NG, M0, 3, WV>(a, n_hblk, st);
    default: return launch_decode<D, NG, M0, 4, WV>(a, n_hblk, st);
  }
}

template <int D, int NG, bool WV>
hipError_t dispatch_m0(const DArgs& a, int m0, int m1, int n_hblk, hipStream_t st) {
  if constexpr (NG == 1) {
    switch (m0) {
      case 1: return launch_decode<D, 1, 1, 1, WV>(a, n_hblk, st);
      case 2: return launch_decode<D, 1, 2, 2, WV>(a, n_hblk, st);
      case 3: return launch_decode<D, 1, 3, 3, WV>(a, n_hblk, st);
      default: return launch_decode<D, 1, 4, 4, WV>(a, n_hblk, st);
    }
  } else {
    switch (m0) {
      case 1: return dispatch_m1<D, 2, 1, WV>(a, m1, n_hblk, st);
      case 2: return dispatch_m1<D, 2, 2, WV>(a, m1, n_hblk, st);
      case 3: return dispatch_m1<D, 2, 3, WV>(a, m1, n_hblk, st);
      default: return dispatch_m1<D, 2, 4, WV>(a, m1, n_hblk, st);
    }
  }
}

}  // namespace

extern "C" tq_status tq_attn_decode_workspace_bytes(const tq_quantizer* kq, const tq_quantizer* vq,
                                                    const tq_decode_shape* shape, size_t* bytes) {
  if (!kq || !tq::layout_valid(&kq->layout) || !shape_valid(shape) || !bytes) return TQ_ERR_INVALID;
  if (vq && !tq::layout_valid(&vq->layout)) return TQ_ERR_INVALID;
  const int n_hblk = (shape->n_q_heads / shape->n_kv_heads + 15) / 16;
  *bytes = workspace_for(shape, kq->layout.d, vq != nullptr, choose_split(shape, n_hblk));
  return TQ_OK;
}

extern "C" tq_status tq_attn_decode(const tq_quantizer* kq, const tq_quantizer* vq,
                                    const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                                    const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!tq::quantizer_pointers_valid(kq) || !shape_valid(shape)) return TQ_ERR_INVALID;
  if (vq && !tq::quantizer_pointers_valid(vq)) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (!q || reinterpret_cast<uintptr_t>(q) % 16 != 0) return TQ_ERR_INVALID;
  if (!k_cache || !k_cache->codes || !k_cache->signs || !k_cache->norms) return TQ_ERR_INVALID;
  const int64_t rows_needed = (int64_t)shape->batch * shape->n_kv_heads * shape->cache_capacity;
  if (k_cache->n_rows < rows_needed) return TQ_ERR_INVALID;
  const bool with_v = vq != nullptr;
  if (with_v) {
    if (!v_cache || !v_cache->codes || !v_cache->signs || !v_cache->norms) return TQ_ERR_INVALID;
    if (v_cache->n_rows < rows_needed || !out) return TQ_ERR_INVALID;
    if (!same_layout(kq->layout, vq->layout)) return TQ_ERR_UNSUPPORTED;
  } else {
    if (!logits || out) return TQ_ERR_INVALID;
  }
  const void* ptrs[] = {k_cache->codes, k_cache->signs, k_cache->norms, logits, out, workspace,
                        with_v ? (const void*)v_cache->codes : nullptr,
                        with_v ? (const void*)v_cache->signs : nullptr,
                        with_v ? (const void*)v_cache->norms : nullptr};
  for (const void* p : ptrs)
    if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0) return TQ_ERR_INVALID;
  if (!decode_supported(kq->layout)) return TQ_ERR_UNSUPPORTED;
  const tq_layout& l = kq->layout;
  const int group = shape->n_q_heads / shape->n_kv_heads;
  const int n_hblk = (group + 15) / 16;
  const int n_split = choose_split(shape, n_hblk);
  const size_t need = workspace_for(shape, l.d, with_v, n_split);
  if (!workspace || workspace_bytes < need) return TQ_ERR_WORKSPACE;

  constexpr int D = 128;
  const int n_heads = shape->batch * shape->n_q_heads;
  _Float16* qprep = reinterpret_cast<_Float16*>(workspace);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                         align256((size_t)n_heads * 4 * D * sizeof(_Float16)));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  hipLaunchKernelGGL((prep_kernel<D>), dim3((n_heads + kPrepHeads - 1) / kPrepHeads), dim3(2 * D), 0,
                     st, q, (int)(q_dtype == TQ_BF16), n_heads, kq->rot, kq->sketch, qprep);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;

  DArgs a{};
  a.batch = shape->batch;
  a.hq = shape->n_q_heads;
  a.hkv = shape->n_kv_heads;
  a.group = group;
  a.n_split = n_split;
  a.n_ctx = shape->n_ctx;
  a.cap = shape->cache_capacity;
  a.scale = shape->scale;
  a.qprep = qprep;
  a.kc = k_cache->codes;
  a.ks = k_cache->signs;
  a.kn = k_cache->norms;
  a.kcent = kq->centroids;
  if (with_v) {
    a.vc = v_cache->codes;
    a.vs = v_cache->signs;
    a.vn = v_cache->norms;
    a.vcent = vq->centroids;
  }
  a.logits = logits;
  a.part = part;
  hipError_t e;
  if (l.n_groups == 1)
    e = with_v ? dispatch_m0<D, 1, true>(a, l.mse_bits[0], 0, n_hblk, st)
               : dispatch_m0<D, 1, false>(a, l.mse_bits[0], 0, n_hblk, st);
  else
    e = with_v ? dispatch_m0<D, 2, true>(a, l.mse_bits[0], l.mse_bits[1], n_hblk, st)
               : dispatch_m0<D, 2, false>(a, l.mse_bits[0], l.mse_bits[1], n_hblk, st);
  if (e != hipSuccess) return TQ_ERR_DEVICE;
  if (with_v) {
    hipLaunchKernelGGL((combine_kernel<D>), dim3(n_heads), dim3(2 * D), 0, st, part, n_split, vq->rot,
                       vq->sketch, l.n_groups == 2 ? l.group_dim[0] : D, out);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}
