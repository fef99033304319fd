// Quantize-on-append for gfx950: one fused kernel per call.
//
// [ZB] paragraph 2 and [WD] "Como o TurboQuant funciona": rotate each vector
// by a random orthogonal matrix, give every rotated coordinate its Lloyd-Max
// cell, take the residual of that MSE quantizer, keep the signs of a Gaussian
// sketch of the residual, and store codes, sign bits and the norms.
//
// Work decomposition. A workgroup owns a tile of 64 vectors at a time and
// loops over tiles (grid-stride). It has one wave per 16 output coordinates
// (d rounded up to 16), so a wave's slice of the d x d matrices stays in
// registers for the whole kernel, as the B operand of
// v_mfma_f32_16x16x4_f32. The input tile and later the rotated residual sit
// in LDS as the A operand shared by all waves. Both contractions are fp32
// MFMA with fp32 accumulation: the codes are decided by comparing rotated
// coordinates with the decision boundaries, which needs fp32-grade
// products (bf16-rounded operands would move coordinates by ~1e-4 of a
// cell). Between the two contractions each lane finishes its coordinates:
// group norms (cross-wave sums through LDS), cells, residual, residual norm.
// After the second contraction the sign bits and codes are packed from LDS
// bytes into the record format and stored.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"
#include "turboquant.h"

namespace {

constexpr int QT = 64;  // vectors per tile

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct QArgs {
  const void* x;
  int64_t n_vec;
  int64_t x_stride;
  int x_bf16;
  const float* rot;
  const float* skr;
  const float* centroids;
  const float* boundaries;
  int d;
  int n_groups;
  int gdim[2];
  int gbits[2];
  int choff[2];
  int cwoff[2];
  int swoff[2];
  int bcwoff[2];
  int bswoff[2];
  int coff[2];
  int boff[2];
  int code_words;
  int sign_words;
  int blk_code_words;
  int blk_sign_words;
  int fmt;
  const int64_t* dst_rows;
  int64_t seg_len;
  int64_t seg_stride;
  int64_t seg_offset;
  int64_t n_rows;
  uint32_t* codes;
  uint32_t* signs;
  float* norms;
};

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ int64_t dest_row(const QArgs& a, int64_t i) {
  if (a.dst_rows) return a.dst_rows[i];
  return (i / a.seg_len) * a.seg_stride + a.seg_offset + (i % a.seg_len);
}

// LDS layout (bytes), KP = padded K, NT = number of 16-wide coordinate tiles.
template <int KP, int NT>
struct Lds {
  static constexpr int XS = KP + 4;  // row stride of the fp32 tile, in floats
  static constexpr int DP = NT * 16;
  static constexpr int off_x = 0;                                   // float [QT][XS]
  static constexpr int off_code = off_x + QT * XS * 4;              // u8 [QT][DP]
  static constexpr int off_sign = off_code + QT * DP;               // u8 [QT][DP]
  static constexpr int off_npart = off_sign + QT * DP;              // float [NT][QT]
  static constexpr int off_gpart = off_npart + NT * QT * 4;         // float [NT][QT]
  static constexpr int off_nrm = off_gpart + NT * QT * 4;           // float [2][QT]
  static constexpr int off_cb = off_nrm + 2 * QT * 4;               // float [64]
  static constexpr int off_rows = off_cb + 64 * 4;                  // int64 [QT]
  static constexpr int off_flags = off_rows + QT * 8;               // int [4]
  static constexpr int bytes = off_flags + 16;
};

template <int KP, int NT>
__global__ __launch_bounds__(NT * 64) void quantize_kernel(QArgs a) {
  using L = Lds<KP, NT>;
  constexpr int XS = L::XS;
  constexpr int DP = L::DP;
  constexpr int KPG = KP / 4;  // k values per lane group
  static_assert(KP == NT * 16 && KPG % 4 == 0, "tile shape");
  extern __shared__ __align__(16) unsigned char smem[];
  float* xr = reinterpret_cast<float*>(smem + L::off_x);
  uint8_t* code_b = smem + L::off_code;
  uint8_t* sign_b = smem + L::off_sign;
  float* npart = reinterpret_cast<float*>(smem + L::off_npart);
  float* gpart = reinterpret_cast<float*>(smem + L::off_gpart);
  float* nrm = reinterpret_cast<float*>(smem + L::off_nrm);
  float* cbk = reinterpret_cast<float*>(smem + L::off_cb);  // [0,32): centroids, [32,64): boundaries
  int64_t* rows = reinterpret_cast<int64_t*>(smem + L::off_rows);
  int* flags = reinterpret_cast<int*>(smem + L::off_flags);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;  // wave = coordinate tile
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int d = a.d;

  // codebooks of both groups into LDS (centroids at their concatenated offsets)
  if (tid < 32) {
    int ncent = (1 << a.gbits[0]) + (a.n_groups > 1 ? (1 << a.gbits[1]) : 0);
    int nbnd = ((1 << a.gbits[0]) - 1) + (a.n_groups > 1 ? (1 << a.gbits[1]) - 1 : 0);
    cbk[tid] = tid < ncent ? a.centroids[tid] : 0.f;
    cbk[32 + tid] = tid < nbnd ? a.boundaries[tid] : 0.f;
  }

  // This wave's rows of rot and sketch_rot: B[k][n] = M[16 w + n][k] with the
  // lane group lg covering k in [lg*KPG, lg*KPG + KPG).
  const int ocoord = w * 16 + ln;  // output coordinate of this lane
  float brot[KPG], bskr[KPG];
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const int k = lg * KPG + kk;
    const bool ok = ocoord < d && k < d;
    brot[kk] = ok ? a.rot[(int64_t)ocoord * d + k] : 0.f;
    bskr[kk] = ok ? a.skr[(int64_t)ocoord * d + k] : 0.f;
  }
  // group of this wave's coordinates (group boundaries are multiples of 16)
  const int grp = (a.n_groups > 1 && w * 16 >= a.choff[1]) ? 1 : 0;
  const int nb = (1 << a.gbits[grp]) - 1;
  const int coff = a.coff[grp];
  const int boff = a.boff[grp];

  const int64_t n_tiles = (a.n_vec + QT - 1) / QT;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t v0 = tile * QT;
    const int nvalid = (int)((a.n_vec - v0) < QT ? (a.n_vec - v0) : QT);

    // ---- stage the input tile (fp32, zero padded) and destination rows ----
    for (int e = tid; e < QT * KP; e += NT * 64) {
      const int v = e / KP, k = e % KP;
      float val = 0.f;
      if (v < nvalid && k < d) {
        const int64_t off = (v0 + v) * a.x_stride + k;
        if (a.x_bf16) {
          const uint16_t h = reinterpret_cast<const uint16_t*>(a.x)[off];
          val = __uint_as_float(((uint32_t)h) << 16);
        } else {
          val = reinterpret_cast<const float*>(a.x)[off];
        }
      }
      xr[v * XS + k] = val;
    }
    if (tid < QT) {
      int64_t r = -1;
      if (tid < nvalid) {
        r = dest_row(a, v0 + tid);
        if (r < 0 || r >= a.n_rows) r = -1;
      }
      rows[tid] = r;
    }
    __syncthreads();

    // ---- y = rot x (fp32 MFMA), four 16-vector tiles ----
    f32x4 yacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* arow = xr + (mt * 16 + ln) * XS + lg * KPG;
#pragma unroll
      for (int q = 0; q < KPG / 4; ++q) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(arow + 4 * q);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[0], brot[4 * q + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[1], brot[4 * q + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[2], brot[4 * q + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[3], brot[4 * q + 3], acc, 0, 0, 0);
      }
      yacc[mt] = acc;
      // lane (ln, lg) holds y[vector 16 mt + 4 lg + i][coordinate 16 w + ln]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = acc[i] * acc[i];
        s += shfl_xor_f(s, 1);
        s += shfl_xor_f(s, 2);
        s += shfl_xor_f(s, 4);
        s += shfl_xor_f(s, 8);
        if (ln == 0) npart[w * QT + mt * 16 + lg * 4 + i] = s;
      }
    }
    __syncthreads();
    // group norms n_g = sqrt(sum of the partial sums of the group's waves)
    if (tid < QT * a.n_groups) {
      const int g = tid / QT, v = tid % QT;
      const int w0 = a.choff[g] / 16, w1 = (a.choff[g] + a.gdim[g] + 15) / 16;
      float s = 0.f;
      for (int ww = w0; ww < w1; ++ww) s += npart[ww * QT + v];
      nrm[g * QT + v] = sqrtf(s);
    }
    __syncthreads();

    // ---- cells, residual in the rotated domain, residual norm partials ----
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = mt * 16 + lg * 4 + i;
        const float y = yacc[mt][i];
        const float n = nrm[grp * QT + v];
        int idx;
        float r;
        if (n > 0.f) {
          const float u = y * (1.0f / n);
          idx = 0;
          float cval = cbk[coff];
          for (int k = 0; k < nb; ++k) {
            if (u > cbk[32 + boff + k]) {
              idx = k + 1;
              cval = cbk[coff + k + 1];
            }
          }
          r = fmaf(-n, cval, y);
        } else {
          idx = (nb + 1) / 2 - 1;
          r = 0.f;
        }
        if (ocoord >= d) r = 0.f;
        code_b[v * DP + ocoord] = (uint8_t)idx;
        xr[v * XS + ocoord] = r;  // A operand of the sketch product (k = rotated coordinate)
        float s = r * r;
        s += shfl_xor_f(s, 1);
        s += shfl_xor_f(s, 2);
        s += shfl_xor_f(s, 4);
        s += shfl_xor_f(s, 8);
        if (ln == 0) gpart[w * QT + v] = s;
      }
    }
    // (every k < KP is a coordinate owned by some wave, so the residual tile
    // is fully written, with zeros past d)
    __syncthreads();

    // ---- s = (S Pi^T) r (fp32 MFMA); sign bit = [s >= 0] ----
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* arow = xr + (mt * 16 + ln) * XS + lg * KPG;
#pragma unroll
      for (int q = 0; q < KPG / 4; ++q) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(arow + 4 * q);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[0], bskr[4 * q + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[1], bskr[4 * q + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[2], bskr[4 * q + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[3], bskr[4 * q + 3], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = mt * 16 + lg * 4 + i;
        sign_b[v * DP + ocoord] = acc[i] >= 0.f ? 1 : 0;
      }
    }
    // full aligned 32-row blocks of this tile (block records only)
    if (tid < 2) {
      int full = 0;
      if (a.fmt == TQ_BLOCK32) {
        const int base = tid * 32;
        const int64_t r0 = rows[base];
        full = (base + 32 <= nvalid) && r0 >= 0 && (r0 % 32 == 0);
        for (int t = 1; t < 32 && full; ++t) full = rows[base + t] == r0 + t;
      }
      flags[tid] = full;
    }
    __syncthreads();

    // ---- pack and store ----
    // norms (both formats): (n_g, gamma_g) per row
    if (tid < QT * a.n_groups) {
      const int g = tid / QT, v = tid % QT;
      const int64_t row = rows[v];
      if (row >= 0) {
        const int w0 = a.choff[g] / 16, w1 = (a.choff[g] + a.gdim[g] + 15) / 16;
        float s = 0.f;
        for (int ww = w0; ww < w1; ++ww) s += gpart[ww * QT + v];
        a.norms[row * (2 * a.n_groups) + 2 * g] = nrm[g * QT + v];
        a.norms[row * (2 * a.n_groups) + 2 * g + 1] = sqrtf(s);
      }
    }
    if (a.fmt == TQ_TOKEN_MAJOR) {
      const int cw = a.code_words;
      for (int e = tid; e < QT * cw; e += NT * 64) {
        const int v = e / cw, wd = e % cw;
        const int64_t row = rows[v];
        if (row < 0) continue;
        const int g = (a.n_groups > 1 && wd >= a.cwoff[1]) ? 1 : 0;
        const int m = a.gbits[g], dg = a.gdim[g];
        const int lw = wd - a.cwoff[g];
        const int b0 = 32 * lw;
        int j0 = b0 / m - 1;
        if (j0 < 0) j0 = 0;
        int j1 = (b0 + 31) / m;
        if (j1 > dg - 1) j1 = dg - 1;
        uint64_t acc = 0;
        for (int j = j0; j <= j1; ++j) {
          const int pos = m * j - b0;
          const uint64_t c = code_b[v * DP + a.choff[g] + j];
          if (pos >= 0)
            acc |= c << pos;
          else
            acc |= c >> (-pos);
        }
        a.codes[row * cw + wd] = (uint32_t)acc;
      }
      const int sw = a.sign_words;
      for (int e = tid; e < QT * sw; e += NT * 64) {
        const int v = e / sw, wd = e % sw;
        const int64_t row = rows[v];
        if (row < 0) continue;
        const int g = (a.n_groups > 1 && wd >= a.swoff[1]) ? 1 : 0;
        const int dg = a.gdim[g];
        const int lw = wd - a.swoff[g];
        uint32_t word = 0;
        for (int b = 0; b < 32; ++b) {
          const int j = 32 * lw + b;
          if (j < dg) word |= (uint32_t)sign_b[v * DP + a.choff[g] + j] << b;
        }
        a.signs[row * sw + wd] = word;
      }
    } else {
      // block records: whole blocks are written word by word
      for (int h = 0; h < 2; ++h) {
        if (!flags[h]) continue;
        const int64_t blk = rows[h * 32] / 32;
        const int bcw = a.blk_code_words;
        for (int wd = tid; wd < bcw; wd += NT * 64) {
          const int g = (a.n_groups > 1 && wd >= a.bcwoff[1]) ? 1 : 0;
          const int m = a.gbits[g], dg = a.gdim[g];
          const int lw = wd - a.bcwoff[g];
          const int b0 = 32 * lw;
          const int u0 = b0 / (8 * m), u1 = (b0 + 31) / (8 * m);
          uint64_t word = 0;
          for (int u = u0; u <= u1 && u < 4 * dg; ++u) {
            const int o = u / dg, j = u % dg;
            uint64_t unit = 0;
            for (int s = 0; s < 8; ++s)
              unit |= (uint64_t)code_b[(h * 32 + 8 * o + s) * DP + a.choff[g] + j] << (m * s);
            const int pos = 8 * m * u - b0;
            if (pos >= 0)
              word |= unit << pos;
            else
              word |= unit >> (-pos);
          }
          a.codes[blk * bcw + wd] = (uint32_t)word;
        }
        const int bsw = a.blk_sign_words;
        for (int wd = tid; wd < bsw; wd += NT * 64) {
          const int g = (a.n_groups > 1 && wd >= a.bswoff[1]) ? 1 : 0;
          const int dg = a.gdim[g];
          const int lw = wd - a.bswoff[g];
          uint32_t word = 0;
          for (int q = 0; q < 4; ++q) {
            const int u = 4 * lw + q;
            const int o = u / dg, j = u % dg;
            uint32_t unit = 0;
            for (int s = 0; s < 8; ++s)
              unit |= (uint32_t)sign_b[(h * 32 + 8 * o + s) * DP + a.choff[g] + j] << s;
            word |= unit << (8 * q);
          }
          a.signs[blk * bsw + wd] = word;
        }
      }
      // rows outside full blocks: update their bits in place
      for (int e = tid; e < QT * d; e += NT * 64) {
        const int v = e / d, ch = e % d;
        if (flags[v / 32]) continue;
        const int64_t row = rows[v];
        if (row < 0) continue;
        const int g = (a.n_groups > 1 && ch >= a.choff[1]) ? 1 : 0;
        const int m = a.gbits[g], dg = a.gdim[g];
        const int j = ch - a.choff[g];
        const int64_t blk = row / 32;
        const int t = (int)(row % 32), o = t / 8, s = t % 8;
        const uint32_t code = code_b[v * DP + ch];
        const int pos = 8 * m * (o * dg + j) + m * s;
        uint32_t* base = a.codes + blk * a.blk_code_words + a.bcwoff[g];
        const int wi = pos / 32, bi = pos % 32;
        const uint32_t fmask = (1u << m) - 1u;
        atomicAnd(base + wi, ~(fmask << bi));
        atomicOr(base + wi, code << bi);
        if (bi + m > 32) {
          const int spill = bi + m - 32;
          atomicAnd(base + wi + 1, ~((1u << spill) - 1u));
          atomicOr(base + wi + 1, code >> (32 - bi));
        }
        const int spos = 8 * (o * dg + j) + s;
        uint32_t* sbase = a.signs + blk * a.blk_sign_words + a.bswoff[g];
        const uint32_t sbit = sign_b[v * DP + ch];
        atomicAnd(sbase + spos / 32, ~(1u << (spos % 32)));
        atomicOr(sbase + spos / 32, sbit << (spos % 32));
      }
    }
    __syncthreads();
  }
}

template <int KP, int NT>
tq_status launch_quantize(const QArgs& a, hipStream_t stream) {
  using L = Lds<KP, NT>;
  static_assert(L::bytes <= 160 * 1024, "LDS budget");
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&quantize_kernel<KP, NT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes) != hipSuccess)
    return TQ_ERR_DEVICE;
  const int64_t n_tiles = (a.n_vec + QT - 1) / QT;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n_cu = v;
  }
  const int64_t per_cu = L::bytes <= 80 * 1024 ? 2 : 1;
  const int64_t grid = n_tiles < per_cu * n_cu ? n_tiles : per_cu * n_cu;
  hipLaunchKernelGGL((quantize_kernel<KP, NT>), dim3((unsigned)grid), dim3(NT * 64), L::bytes, stream,
                     a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

}  // namespace

extern "C" tq_status tq_quantize(const tq_quantizer* qz, tq_format fmt, const void* x,
                                 tq_dtype x_dtype, int64_t n_vec, int64_t x_row_stride,
                                 const tq_rows* rows, const tq_cache* cache, void* stream) {
  if (!tq::quantizer_pointers_valid(qz) || !rows || !cache) return TQ_ERR_INVALID;
  if (fmt != TQ_TOKEN_MAJOR && fmt != TQ_BLOCK32) return TQ_ERR_INVALID;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_INVALID;
  const tq_layout& l = qz->layout;
  if (n_vec < 0 || x_row_stride < l.d) return TQ_ERR_INVALID;
  if (!cache->codes || !cache->signs || !cache->norms || cache->n_rows < 0) return TQ_ERR_INVALID;
  if (fmt == TQ_BLOCK32 && cache->n_rows % 32 != 0) return TQ_ERR_INVALID;
  if (!rows->dst_rows) {
    if (rows->seg_len < 1 || rows->seg_stride < 0 || rows->seg_offset < 0) return TQ_ERR_INVALID;
    if (n_vec > 0) {
      // rows grow with the segment index when segments do not overlap, so the
      // largest row is the last vector's
      const int64_t last = n_vec - 1;
      const int64_t nseg = last / rows->seg_len;
      if (nseg > 0 && rows->seg_stride < rows->seg_len) return TQ_ERR_INVALID;  // overlapping rows
      const int64_t hi = nseg * rows->seg_stride + rows->seg_offset + last % rows->seg_len;
      if (hi >= cache->n_rows) return TQ_ERR_INVALID;
    }
  }
  const tq::GroupGeom geo = tq::geometry(&l);
  if (l.n_groups == 2 && l.group_dim[0] % 16 != 0) return TQ_ERR_UNSUPPORTED;
  if (fmt == TQ_BLOCK32)
    for (int g = 0; g < l.n_groups; ++g)
      if (l.group_dim[g] % 8 != 0) return TQ_ERR_UNSUPPORTED;
  if (n_vec == 0) return TQ_OK;
  if (!x || reinterpret_cast<uintptr_t>(x) % 4 != 0) return TQ_ERR_INVALID;

  QArgs a{};
  a.x = x;
  a.n_vec = n_vec;
  a.x_stride = x_row_stride;
  a.x_bf16 = x_dtype == TQ_BF16;
  a.rot = qz->rot;
  a.skr = qz->sketch_rot;
  a.centroids = qz->centroids;
  a.boundaries = qz->boundaries;
  a.d = l.d;
  a.n_groups = l.n_groups;
  for (int g = 0; g < 2; ++g) {
    a.gdim[g] = geo.dim[g];
    a.gbits[g] = geo.bits[g];
    a.choff[g] = geo.ch_off[g];
    a.cwoff[g] = geo.code_word_off[g];
    a.swoff[g] = geo.sign_word_off[g];
    a.bcwoff[g] = geo.blk_code_off[g];
    a.bswoff[g] = geo.blk_sign_off[g];
    a.coff[g] = geo.centroid_off[g];
    a.boff[g] = geo.boundary_off[g];
  }
  if (l.n_groups == 1) a.choff[1] = 1 << 30;  // never reached
  a.code_words = geo.info.code_words;
  a.sign_words = geo.info.sign_words;
  a.blk_code_words = geo.info.block_code_words;
  a.blk_sign_words = geo.info.block_sign_words;
  a.fmt = fmt;
  a.dst_rows = rows->dst_rows;
  a.seg_len = rows->seg_len < 1 ? 1 : rows->seg_len;
  a.seg_stride = rows->seg_stride;
  a.seg_offset = rows->seg_offset;
  a.n_rows = cache->n_rows;
  a.codes = cache->codes;
  a.signs = cache->signs;
  a.norms = cache->norms;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int dpad = (l.d + 15) / 16;
  if (dpad <= 4) return launch_quantize<64, 4>(a, s);
  if (dpad <= 8) return launch_quantize<128, 8>(a, s);
  if (dpad <= 13) return launch_quantize<208, 13>(a, s);
  return launch_quantize<256, 16>(a, s);
}
