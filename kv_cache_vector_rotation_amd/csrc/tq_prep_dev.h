// Query preparation of a decode step, shared by the decode entry points and
// the fused append + prep launch.
//
// q_rot = f rot q and q_sk = f alpha_g sketch q, each stored as fp16 hi and
// (q - hi) * 2^11 (about 22 bits), with f = scale * log2(e) so that the
// split pass forms log2-domain logits directly; fp32 sums in ascending k,
// scaled after the sum. A block takes kPrepRows rows of the stacked
// [rot; sketch] matrix and kPrepHeads heads; both are staged in LDS by
// coalesced 16-byte loads, then each thread forms dot products of one row
// with several heads. One extra block searches the K (and V) codebook
// scales.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace tqp {

constexpr int kPrepHeads = 64;
constexpr int kPrepRows = 16;
constexpr float kLoScale = 2048.0f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PrepArgs {
  const void* q;
  int q_bf16;
  int n_heads;
  const float* rot;
  const float* sketch;
  float scale_l2;  // scale * log2(e)
  int group_dim0;  // d_0 (= d for one group)
  _Float16* qprep;
  const float* kcent;
  int n_groups, m0, m1;
  float* kscale;  // out: one scale per K group, then (when vcent is set) one per V group at kscale + 2
  const float* vcent;  // V centroids (same layout as K), or null
  // query tokens per head (T > 1: heads are ordered (batch, q head, token)
  // while q rows are (batch, token, q head)), and the q heads per batch
  int T, hq;
};

// q row of prepared head h: the identity for T <= 1, else head
// (b hq + g) T + t reads row (b T + t) hq + g
__device__ __forceinline__ int64_t prep_q_row(const PrepArgs& p, int h) {
  if (p.T <= 1) return h;
  const int t = h % p.T, bh = h / p.T;
  return ((int64_t)(bh / p.hq) * p.T + t) * p.hq + bh % p.hq;
}

// blocks along x: the row blocks of rot, those of sketch (each matrix cut
// into blocks of kPrepRows rows, the last one partial when kPrepRows does not
// divide D), then the scale search
template <int D>
constexpr int prep_row_blocks() { return (D + kPrepRows - 1) / kPrepRows; }
template <int D>
constexpr int prep_blocks_x() { return 2 * prep_row_blocks<D>() + 1; }

// LDS bytes a prep block needs (row and head staging, or the search)
template <int D>
constexpr int prep_lds_bytes() { return (kPrepRows + kPrepHeads) * (D + 4) * 4; }

// Scale s in [1, 2) for which the fp16 roundings of s |c_k| are closest to
// exact (smallest largest relative error over the centroids; 2048
// candidates s = 1 + i / 2048, ties to the smaller i). The decode tables
// hold fp16(s c) and the logits divide by s, so the centroids enter the
// products with a few 1e-5 relative error instead of fp16's ~2.4e-4. The
// codebook is symmetric, so its upper half of magnitudes suffices.
template <int NTHR>
__device__ void search_fp16_scale(const float* cent, int L, float* out, int tid, unsigned char* smem) {
  float* s_err = reinterpret_cast<float*>(smem);
  int* s_idx = reinterpret_cast<int*>(smem + NTHR * 4);
  float mag[8], inv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int kk = L / 2 + (k < L / 2 ? k : 0);
    mag[k] = fabsf(cent[kk]);
    inv[k] = 1.0f / mag[k];
  }
  float best = INFINITY;
  int bi = 0;
  for (int i = tid; i < 2048; i += NTHR) {
    const float sc = 1.0f + (float)i * (1.0f / 2048.0f);
    float worst = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= L / 2) break;
      const float x = mag[k] * sc;
      worst = fmaxf(worst, fabsf((float)(_Float16)x - x) * inv[k]);
    }
    worst /= sc;  // relative to s |c_k|
    if (worst < best) {
      best = worst;
      bi = i;
    }
  }
  s_err[tid] = best;
  s_idx[tid] = bi;
  __syncthreads();
  for (int w = NTHR / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const float e2 = s_err[tid + w];
      const int i2 = s_idx[tid + w];
      if (e2 < s_err[tid] || (e2 == s_err[tid] && i2 < s_idx[tid])) {
        s_err[tid] = e2;
        s_idx[tid] = i2;
      }
    }
    __syncthreads();
  }
  if (tid == 0) *out = 1.0f + (float)s_idx[0] * (1.0f / 2048.0f);
  __syncthreads();
}

// Block (bx, by) of the preparation with NTHR threads.
template <int D, int NTHR>
__device__ void prep_block(const PrepArgs& p, int bx, int by, int t, unsigned char* smem) {
  constexpr int RB = prep_row_blocks<D>();
  if (bx == 2 * RB) {
    if (by == 0) {
      search_fp16_scale<NTHR>(p.kcent, 1 << p.m0, p.kscale, t, smem);
      if (p.n_groups > 1) search_fp16_scale<NTHR>(p.kcent + (1 << p.m0), 1 << p.m1, p.kscale + 1, t, smem);
      if (p.vcent) {
        search_fp16_scale<NTHR>(p.vcent, 1 << p.m0, p.kscale + 2, t, smem);
        if (p.n_groups > 1) search_fp16_scale<NTHR>(p.vcent + (1 << p.m0), 1 << p.m1, p.kscale + 3, t, smem);
      }
    }
    return;
  }
  constexpr int QS = D + 4;                            // LDS row stride (floats)
  constexpr int TPR = NTHR / kPrepRows;                // threads per row
  constexpr int HPT = kPrepHeads / TPR;                // heads per thread
  float (*sm)[QS] = reinterpret_cast<float (*)[QS]>(smem);
  float (*sq)[QS] = reinterpret_cast<float (*)[QS]>(smem + kPrepRows * QS * 4);
  const bool sk = bx >= RB;
  const int lr0 = (sk ? bx - RB : bx) * kPrepRows;  // first row of the block in its matrix
  const int r0 = lr0 + (sk ? D : 0);                // first row of [rot; sketch]
  const int h0 = by * kPrepHeads;
  const float* mat = (sk ? p.sketch : p.rot) + (int64_t)lr0 * D;
  {
    constexpr int C4 = D / 4;  // 16-byte chunks per matrix row
    constexpr int NM = (kPrepRows * C4 + NTHR - 1) / NTHR;
    f32x4 mb[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int c = t + NTHR * i;
      // (rows past the matrix read its last row; their results are dropped)
      const int cc = c < kPrepRows * C4 ? c : 0;
      const int rr = lr0 + cc / C4 < D ? cc / C4 : D - 1 - lr0;
      mb[i] = *reinterpret_cast<const f32x4*>(mat + rr * D + (cc % C4) * 4);
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int c = t + NTHR * i;
      if (c < kPrepRows * C4) *reinterpret_cast<f32x4*>(&sm[c / C4][(c % C4) * 4]) = mb[i];
    }
  }
  // (chunk counts rounded up; chunks past the block's last are skipped)
  if (p.q_bf16) {
    constexpr int C8 = D / 8;  // 16-byte chunks per bf16 query row
    constexpr int NC = (kPrepHeads * C8 + NTHR - 1) / NTHR;
    u32x4 qb[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = t + NTHR * i, cc = c < kPrepHeads * C8 ? c : 0, h = h0 + cc / C8;
      const int hc = h < p.n_heads ? h : p.n_heads - 1;
      qb[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + prep_q_row(p, hc) * D +
                                              (cc % C8) * 8);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = t + NTHR * i;
      if (c >= kPrepHeads * C8) continue;
      float* dst = &sq[c / C8][(c % C8) * 8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = __uint_as_float(qb[i][e] << 16);
        dst[2 * e + 1] = __uint_as_float(qb[i][e] & 0xFFFF0000u);
      }
    }
  } else {
    constexpr int C4 = D / 4;
    constexpr int NC = (kPrepHeads * C4 + NTHR - 1) / NTHR;
    f32x4 qb[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = t + NTHR * i, cc = c < kPrepHeads * C4 ? c : 0, h = h0 + cc / C4;
      const int hc = h < p.n_heads ? h : p.n_heads - 1;
      qb[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.q) + prep_q_row(p, hc) * D +
                                              (cc % C4) * 4);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = t + NTHR * i;
      if (c < kPrepHeads * C4) *reinterpret_cast<f32x4*>(&sq[c / C4][(c % C4) * 4]) = qb[i];
    }
  }
  __syncthreads();
  const int i = t % kPrepRows, hq = t / kPrepRows;
  float acc[HPT] = {};
#pragma unroll 4
  for (int k = 0; k < D; k += 4) {
    const f32x4 m4 = *reinterpret_cast<const f32x4*>(&sm[i][k]);
#pragma unroll
    for (int r = 0; r < HPT; ++r) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(&sq[hq + TPR * r][k]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r] = fmaf(m4[j], q4[j], acc[r]);
    }
  }
  const int row = r0 + i;
  if (lr0 + i >= D) return;  // a row past the matrix (partial last block)
  // logits in the log2 domain: both parts carry scale * log2(e); the sketch
  // part also alpha_g = sqrt(pi / 2) / d_g of the row's group
  float f = p.scale_l2;
  if (row >= D) {
    const int dg = row - D < p.group_dim0 ? p.group_dim0 : D - p.group_dim0;
    f *= 1.2533141373155003f / (float)dg;
  }
#pragma unroll
  for (int r = 0; r < HPT; ++r) {
    const int h = h0 + hq + TPR * r;
    if (h >= p.n_heads) continue;
    // [q_rot hi | q_rot lo | q_sk hi | q_sk lo], D each: row r of [rot;
    // sketch] goes to r (hi) and D + r (lo) of its half
    _Float16* dst = p.qprep + (int64_t)h * 4 * D + (row < D ? 0 : D);
    acc[r] *= f;
    const _Float16 hi = (_Float16)acc[r];
    dst[row] = hi;
    dst[D + row] = (_Float16)((acc[r] - (float)hi) * kLoScale);
  }
}

}  // namespace tqp
