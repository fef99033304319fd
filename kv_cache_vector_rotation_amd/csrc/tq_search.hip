// Nearest-neighbour search over compressed vectors for gfx950.
//
// [WD] "Os numeros que importam": the same codes also serve vector search
// (recall on a word-vector benchmark above methods with large codebooks).
// Every query is scored against every database vector with the inner-product
// estimator of the attention logits (scale 1),
//   score(q, i) = n_i <Pi q, c[idx_i]> + alpha gamma_i <S q, z_i>,
// and the k best scores are kept; equal scores go to the lower index.
//
// Work decomposition. The queries are prepared once (the decode's query
// preparation with scale 1: Pi q as fp16 hi and lo parts, alpha S q as fp16,
// and the fp16 codebook scale; the search uses the hi part alone: its
// rounding moves a score by at most 2^-12 sum |q_i c_i| n, far inside the
// score tolerance, whereas the decode needs the lo part because the softmax
// amplifies logit errors). A workgroup takes 32 queries and one slice of
// the database; its four waves take 16-vector tiles of the slice in turn. Per
// tile a wave expands the codes of its 16 vectors into fp16 centroid pairs
// through a replicated LDS table (one lookup per two coordinates) and the
// sign bits into fp16 +-1 through a nibble table, and multiplies them with
// the 32 queries on v_mfma_f32_16x16x32_f16 (two products per 32
// coordinates and 16 queries: rotated and sketch), with the query operands in
// LDS in lane order. The scores of a tile then enter per-lane sorted top-k
// lists (lane (l, g) owns query l of each 16-query block and database rows
// 4 g .. 4 g + 3 of every tile, so its candidates arrive in increasing index
// order and a strict comparison keeps the lower index on ties). At the end
// the 16 lists of each query are merged in LDS into the workgroup's top k,
// and a second kernel merges the slices.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tq_internal.h"
#include "tq_prep_dev.h"
#include "turboquant.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kQB = 32;       // queries per workgroup (two MFMA column blocks)
constexpr int kTV = 16;       // database vectors per wave tile (MFMA rows)
constexpr int kWaves = 4;
constexpr int kKL = 10;       // list length; k <= kKL
constexpr int kMaxSlices = 16;
constexpr int kTargetWorkgroups = 2048;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

struct SArgs {
  int64_t n_db;
  int n_q, n_slices;
  int64_t tiles_per_slice;
  const uint32_t* codes;
  const uint32_t* signs;
  const float* norms;
  int norm_f16;  // norm pairs stored as float16 (one word per row)
  const _Float16* qprep;  // [n_q][4 D]: q_rot hi, q_rot lo * 2^11 (unused here), q_sk hi, q_sk lo (unused)
  const float* kscale;    // fp16 codebook scale s
  const float* centroids;
  float* part_score;      // [n_q][n_slices][kKL]
  int* part_idx;
};

template <int D, int M>
struct Geo {
  static constexpr int KC = (D + 31) / 32;             // 32-coordinate chunks
  static constexpr int CW = (M * D + 31) / 32;         // code words per record
  static constexpr int SW = (D + 31) / 32;             // sign words per record
  static constexpr int NPAIR = 1 << (2 * M);           // entries of the pair table
  static constexpr int B_BYTES = KC * 2 * 2 * 64 * 16; // query operands
  static constexpr int M_BYTES = 16 * kWaves * 4 * kKL * 8;   // merge lists of one column block
  static constexpr int R0 = B_BYTES > M_BYTES ? B_BYTES : M_BYTES;
  static constexpr int off_ctab = R0;                  // u32 [NPAIR][64]
  static constexpr int off_stab = off_ctab + NPAIR * 64 * 4;  // u32x2 [16][64]
  static constexpr int bytes = off_stab + 16 * 64 * 8;
};

// Inserts (x, id) into a descending list; equal scores keep the earlier entry.
__device__ __forceinline__ void list_insert(float (&sc)[kKL], int (&ix)[kKL], float x, int id) {
#pragma unroll
  for (int j = kKL - 1; j > 0; --j) {
    const bool shift = x > sc[j - 1];
    const bool here = !shift && x > sc[j];
    const float s2 = shift ? sc[j - 1] : (here ? x : sc[j]);
    const int i2 = shift ? ix[j - 1] : (here ? id : ix[j]);
    sc[j] = s2;
    ix[j] = i2;
  }
  if (x > sc[0]) {
    sc[0] = x;
    ix[0] = id;
  }
}

// H: the database stores its norms as float16 pairs
template <int D, int M, bool H>
__global__ __launch_bounds__(256, 3) void search_kernel(SArgs a) {
  using G = Geo<D, M>;
  constexpr int KC = G::KC, CW = G::CW, SW = G::SW;
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* s_b = reinterpret_cast<u32x4*>(smem);
  uint32_t* s_ctab = reinterpret_cast<uint32_t*>(smem + G::off_ctab);
  u32x2* s_stab = reinterpret_cast<u32x2*>(smem + G::off_stab);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int qb = blockIdx.x, slice = blockIdx.y;

  // ---- tables: fp16 (s c[a], s c[b]) for the code pair a | b << M, and the
  // fp16 +-1 of four sign bits (bit 1 -> +1), each entry once per lane ----
  {
    const float s = a.kscale[0];
    for (int e = tid; e < G::NPAIR * 64; e += 256) {
      const int v = e >> 6, l = e & 63;
      const int ca = v & ((1 << M) - 1), cb = v >> M;
      const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(s * a.centroids[ca]));
      const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(s * a.centroids[cb]));
      s_ctab[v * 64 + l] = lo | (hi << 16);
    }
    for (int e = tid; e < 16 * 64; e += 256) {
      const int v = e >> 6, l = e & 63;
      uint32_t h[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) h[b] = ((v >> b) & 1) ? 0x3C00u : 0xBC00u;
      s_stab[v * 64 + l] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
  }
  // ---- query operands in lane order: [chunk][part (rot hi, sketch)][column
  // block][lane], lane (l, g): query 16 cb + l, coordinates 32 c + 8 g .. + 8;
  // zero past D and past the last query ----
  for (int e = tid; e < KC * 2 * 2 * 64; e += 256) {
    const int l = e & 63, cb = (e >> 6) & 1, pt = (e >> 7) & 1, c = e >> 8;
    const int h = qb * kQB + cb * 16 + (l & 15);
    const int k = 32 * c + 8 * (l >> 4);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < a.n_q && k < D) v = *reinterpret_cast<const u32x4*>(a.qprep + (int64_t)h * 4 * D + 2 * pt * D + k);
    s_b[e] = v;
  }
  __syncthreads();

  float sc[2][kKL];
  int ix[2][kKL];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int j = 0; j < kKL; ++j) {
      sc[cb][j] = -INFINITY;
      ix[cb][j] = 0x7FFFFFFF;
    }
  const float inv_s = 1.0f / a.kscale[0];

  const int64_t n_tiles = (a.n_db + kTV - 1) / kTV;
  const int64_t t_begin = slice * a.tiles_per_slice;
  const int64_t t_end = t_begin + a.tiles_per_slice < n_tiles ? t_begin + a.tiles_per_slice : n_tiles;

  // record words of row ln of a tile, and the norms of rows 4 lg .. 4 lg + 3
  // (rows past the database read its last row; their scores are masked)
  struct Rec {
    uint32_t cw[CW];
    uint32_t sw[SW];
    u32x2 nr[4];
  };
  auto load = [&](int64_t t, Rec& r) __attribute__((always_inline)) {
    const int64_t row = t * kTV + ln < a.n_db ? t * kTV + ln : a.n_db - 1;
#pragma unroll
    for (int i = 0; i < CW; ++i) r.cw[i] = a.codes[row * CW + i];
#pragma unroll
    for (int i = 0; i < SW; ++i) r.sw[i] = a.signs[row * SW + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ri = t * kTV + 4 * lg + i < a.n_db ? t * kTV + 4 * lg + i : a.n_db - 1;
      if constexpr (H)
        r.nr[i] = u32x2{reinterpret_cast<const uint32_t*>(a.norms)[ri], 0u};
      else
        r.nr[i] = *reinterpret_cast<const u32x2*>(a.norms + ri * 2);
    }
  };

  auto compute = [&](const Rec& r, int64_t t) __attribute__((always_inline)) {
    f32x4 acc[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int p = 0; p < 2; ++p) acc[cb][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      // codes of coordinates 32 c + 8 lg .. + 8: 8 M bits from bit M (32 c + 8 lg)
      const int dw = (8 * M * lg) >> 5, sh = (8 * M * lg) & 31;
      uint32_t lo = r.cw[M * c < CW ? M * c : CW - 1];
      uint32_t hi = M * c + 1 < CW ? r.cw[M * c + 1] : 0u;
#pragma unroll
      for (int d = 1; d < M; ++d) {
        if (M * c + d < CW) lo = dw == d ? r.cw[M * c + d] : lo;
        const uint32_t h2 = M * c + d + 1 < CW ? r.cw[M * c + d + 1] : 0u;
        hi = dw == d ? h2 : hi;
      }
      const uint32_t f = __builtin_amdgcn_alignbit(hi, lo, sh);
      u32x4 arot;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t e = (f >> (2 * M * p)) & (G::NPAIR - 1);
        arot[p] = s_ctab[e * 64 + lane];
      }
      const uint32_t sb = (r.sw[c] >> (8 * lg)) & 0xFFu;
      const u32x2 s0 = s_stab[(sb & 15u) * 64 + lane], s1 = s_stab[(sb >> 4) * 64 + lane];
      u32x4 ask = u32x4{s0[0], s0[1], s1[0], s1[1]};
      if (32 * c + 8 * lg >= D) {  // coordinates past D
        arot = u32x4{0u, 0u, 0u, 0u};
        ask = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const u32x4* bp = s_b + ((c * 2) * 2 + cb) * 64 + lane;
        acc[cb][0] = mfma16(arot, bp[0], acc[cb][0]);
        acc[cb][1] = mfma16(ask, bp[2 * 64], acc[cb][1]);
      }
      // (keeps the next chunk's table and operand reads from being hoisted
      // above this one, which would hold every chunk's operands at once)
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (ln, lg): query 16 cb + ln, rows 4 lg + i of the tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = t * kTV + 4 * lg + i;
      const float n = H ? (float)__builtin_bit_cast(_Float16, (uint16_t)r.nr[i][0]) : __uint_as_float(r.nr[i][0]);
      const float gm =
          H ? (float)__builtin_bit_cast(_Float16, (uint16_t)(r.nr[i][0] >> 16)) : __uint_as_float(r.nr[i][1]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float x = fmaf(n * inv_s, acc[cb][0][i], gm * acc[cb][1][i]);
        if (row >= a.n_db) x = -INFINITY;
        if (x > sc[cb][kKL - 1]) list_insert(sc[cb], ix[cb], x, (int)row);
      }
    }
  };

  int64_t t = t_begin + wv;
  if (t < t_end) {
    Rec ra, rb;
    load(t, ra);
    for (;;) {
      const int64_t tn = t + kWaves < t_end ? t + kWaves : t;
      load(tn, rb);
      compute(ra, t);
      if (tn == t) break;
      t = tn;
      const int64_t tn2 = t + kWaves < t_end ? t + kWaves : t;
      load(tn2, ra);
      compute(rb, t);
      if (tn2 == t) break;
      t = tn2;
    }
  }

  // ---- merge the 16 lists of each query (4 lane groups x 4 waves), one
  // 16-query column block at a time ----
  float* m_sc = reinterpret_cast<float*>(smem);                      // [16][16][kKL]
  int* m_ix = reinterpret_cast<int*>(smem + 16 * 16 * kKL * 4);      // [16][16][kKL]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    __syncthreads();  // the query operands, or the previous block's lists, are no longer read
    const int li = wv * 4 + lg;
#pragma unroll
    for (int j = 0; j < kKL; ++j) {
      m_sc[(ln * 16 + li) * kKL + j] = sc[cb][j];
      m_ix[(ln * 16 + li) * kKL + j] = ix[cb][j];
    }
    __syncthreads();
    const int qg = qb * kQB + cb * 16 + tid;
    if (tid < 16 && qg < a.n_q) {
      int ptr[16];
#pragma unroll
      for (int l = 0; l < 16; ++l) ptr[l] = 0;
      float* ps = a.part_score + ((int64_t)qg * a.n_slices + slice) * kKL;
      int* pi = a.part_idx + ((int64_t)qg * a.n_slices + slice) * kKL;
      for (int j = 0; j < kKL; ++j) {
        float best = -INFINITY;
        int bi = 0x7FFFFFFF, bl = 0;
#pragma unroll
        for (int l = 0; l < 16; ++l) {
          const float v = ptr[l] < kKL ? m_sc[(tid * 16 + l) * kKL + ptr[l]] : -INFINITY;
          const int id = ptr[l] < kKL ? m_ix[(tid * 16 + l) * kKL + ptr[l]] : 0x7FFFFFFF;
          if (v > best || (v == best && id < bi)) {
            best = v;
            bi = id;
            bl = l;
          }
        }
#pragma unroll
        for (int l = 0; l < 16; ++l) ptr[l] += (l == bl) ? 1 : 0;
        ps[j] = best;
        pi[j] = bi;
      }
    }
  }
}

// The slices' lists of one query -> its k best (one thread per query).
__global__ __launch_bounds__(256) void search_merge_kernel(const float* part_score, const int* part_idx, int n_q,
                                                           int n_slices, int k, int64_t* out_idx,
                                                           float* out_score) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= n_q) return;
  const float* ps = part_score + (int64_t)q * n_slices * kKL;
  const int* pi = part_idx + (int64_t)q * n_slices * kKL;
  int ptr[kMaxSlices];
#pragma unroll
  for (int l = 0; l < kMaxSlices; ++l) ptr[l] = 0;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bi = 0x7FFFFFFF, bl = -1;
#pragma unroll
    for (int l = 0; l < kMaxSlices; ++l) {
      if (l >= n_slices || ptr[l] >= kKL) continue;
      const float v = ps[l * kKL + ptr[l]];
      const int id = pi[l * kKL + ptr[l]];
      if (bl < 0 || v > best || (v == best && id < bi)) {
        best = v;
        bi = id;
        bl = l;
      }
    }
#pragma unroll
    for (int l = 0; l < kMaxSlices; ++l) ptr[l] += (l == bl) ? 1 : 0;
    const bool valid = best > -INFINITY;
    out_idx[(int64_t)q * k + j] = valid ? (int64_t)bi : -1;
    out_score[(int64_t)q * k + j] = best;
  }
}

// Query preparation (scale 1), 256 threads per block.
template <int D>
__global__ __launch_bounds__(256) void search_prep_kernel(tqp::PrepArgs p) {
  __shared__ __align__(16) unsigned char smem[tqp::prep_lds_bytes<D>()];
  tqp::prep_block<D, 256>(p, blockIdx.x, blockIdx.y, threadIdx.x, smem);
}

struct Plan {
  int d, m, n_slices, n_qblocks;
  int64_t tiles_per_slice;
  size_t qprep_bytes, part_bytes, total;
};

bool plan_search(const tq_quantizer* qz, int64_t n_db, int64_t n_q, int k, Plan* pl) {
  if (!tq::quantizer_pointers_valid(qz)) return false;
  if (n_db < 1 || n_q < 1 || n_q > (1 << 30) || n_db > 0x7FFFFFFE || k < 1 || k > kKL) return false;
  pl->d = qz->layout.d;
  pl->m = qz->layout.mse_bits[0];
  pl->n_qblocks = (int)((n_q + kQB - 1) / kQB);
  const int64_t n_tiles = (n_db + kTV - 1) / kTV;
  int64_t ns = (kTargetWorkgroups + pl->n_qblocks - 1) / pl->n_qblocks;
  const int64_t max_ns = (n_tiles + kWaves - 1) / kWaves;  // at least one tile per wave
  if (ns > max_ns) ns = max_ns;
  if (ns > kMaxSlices) ns = kMaxSlices;
  if (ns < 1) ns = 1;
  pl->tiles_per_slice = (n_tiles + ns - 1) / ns;
  pl->n_slices = (int)((n_tiles + pl->tiles_per_slice - 1) / pl->tiles_per_slice);
  pl->qprep_bytes = ((size_t)n_q * 4 * pl->d * 2 + 255) / 256 * 256;
  pl->part_bytes = (size_t)n_q * pl->n_slices * kKL * 4;
  pl->total = pl->qprep_bytes + 256 + 2 * pl->part_bytes;
  return true;
}

template <int D, int M, bool H>
hipError_t launch_search_h(const SArgs& a, int n_qblocks, hipStream_t st) {
  using G = Geo<D, M>;
  static_assert(G::bytes <= 53 * 1024, "three workgroups per compute unit");
  static_assert(M <= 3, "pair tables of at most 64 entries");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&search_kernel<D, M, H>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, G::bytes);
  if (e != hipSuccess) return e;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  hipLaunchKernelGGL((search_kernel<D, M, H>), dim3((unsigned)n_qblocks, (unsigned)a.n_slices), dim3(256),
                     G::bytes, st, a);
  return hipGetLastError();
}

template <int D, int M>
hipError_t launch_search(const SArgs& a, int n_qblocks, hipStream_t st) {
  return a.norm_f16 ? launch_search_h<D, M, true>(a, n_qblocks, st) : launch_search_h<D, M, false>(a, n_qblocks, st);
}

}  // namespace

extern "C" tq_status tq_search_workspace_bytes(const tq_quantizer* qz, int64_t n_db, int64_t n_q, int k,
                                               size_t* bytes) {
  Plan pl;
  if (!bytes || !plan_search(qz, n_db, n_q, k, &pl)) return TQ_ERR_INVALID;
  *bytes = pl.total;
  return TQ_OK;
}

extern "C" tq_status tq_search(const tq_quantizer* qz, const tq_cache* db, int64_t n_db, const void* q,
                               tq_dtype q_dtype, int64_t n_q, int k, int64_t* out_idx, float* out_score,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  if (!plan_search(qz, n_db, n_q, k, &pl) || !db || !q || !out_idx || !out_score) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (!db->codes || !db->signs || !db->norms || db->n_rows < n_db) return TQ_ERR_INVALID;
  const tq_layout& l = qz->layout;
  if (l.n_groups != 1 || l.d % 8 != 0 || l.mse_only) return TQ_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, workspace, db->norms};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return TQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(out_idx) % 8 != 0 || reinterpret_cast<uintptr_t>(out_score) % 4 != 0)
    return TQ_ERR_INVALID;
  if (!workspace || workspace_bytes < pl.total) return TQ_ERR_WORKSPACE;
  const bool d200 = l.d == 200, d128 = l.d == 128;
  if (!(d200 || d128) || pl.m > 3) return TQ_ERR_UNSUPPORTED;

  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  _Float16* qprep = reinterpret_cast<_Float16*>(ws);
  float* kscale = reinterpret_cast<float*>(ws + pl.qprep_bytes);
  float* part_score = reinterpret_cast<float*>(ws + pl.qprep_bytes + 256);
  int* part_idx = reinterpret_cast<int*>(ws + pl.qprep_bytes + 256 + pl.part_bytes);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  // query preparation (scale 1): the decode's prep blocks
  tqp::PrepArgs pp{};
  pp.q = q;
  pp.q_bf16 = q_dtype == TQ_BF16;
  pp.n_heads = (int)n_q;
  pp.rot = qz->rot;
  pp.sketch = qz->sketch;
  pp.scale_l2 = 1.0f;
  pp.group_dim0 = l.d;
  pp.qprep = qprep;
  pp.kcent = qz->centroids;
  pp.n_groups = 1;
  pp.m0 = pl.m;
  pp.m1 = 0;
  pp.kscale = kscale;
  const unsigned prep_y = (unsigned)((n_q + tqp::kPrepHeads - 1) / tqp::kPrepHeads);
  if (prep_y > 65535u) return TQ_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  if (d200)
    hipLaunchKernelGGL(search_prep_kernel<200>, dim3(tqp::prep_blocks_x<200>(), prep_y), dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(search_prep_kernel<128>, dim3(tqp::prep_blocks_x<128>(), prep_y), dim3(256), 0, st, pp);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;

  SArgs a{};
  a.n_db = n_db;
  a.n_q = (int)n_q;
  a.n_slices = pl.n_slices;
  a.tiles_per_slice = pl.tiles_per_slice;
  a.codes = db->codes;
  a.signs = db->signs;
  a.norms = db->norms;
  a.norm_f16 = l.norm_f16;
  a.qprep = qprep;
  a.kscale = kscale;
  a.centroids = qz->centroids;
  a.part_score = part_score;
  a.part_idx = part_idx;
  hipError_t e = hipErrorInvalidValue;
  switch ((d200 ? 10 : 0) + pl.m) {
    case 1: e = launch_search<128, 1>(a, pl.n_qblocks, st); break;
    case 2: e = launch_search<128, 2>(a, pl.n_qblocks, st); break;
    case 3: e = launch_search<128, 3>(a, pl.n_qblocks, st); break;
    case 11: e = launch_search<200, 1>(a, pl.n_qblocks, st); break;
    case 12: e = launch_search<200, 2>(a, pl.n_qblocks, st); break;
    case 13: e = launch_search<200, 3>(a, pl.n_qblocks, st); break;
    default: return TQ_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return TQ_ERR_DEVICE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(search_merge_kernel, dim3((unsigned)((n_q + 255) / 256)), dim3(256), 0, st, part_score,
                     part_idx, (int)n_q, pl.n_slices, k, out_idx, out_score);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}
