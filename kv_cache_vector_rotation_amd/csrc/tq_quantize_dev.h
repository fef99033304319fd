// Quantize kernel body and argument set-up, shared by the quantize entry
// point and the fused append + query-prep launch of a decode step.
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
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"
#include "turboquant.h"

namespace tqq {


constexpr int QT = 64;  // vectors per tile

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct QArgs {
  const void* x;
  int64_t n_vec;
  int64_t x_stride;
  int x_bf16;
  int x_vec;  // rows 16-byte aligned and d a multiple of the 16-byte vector width
  int m_vec;  // rot and sketch_rot 16-byte aligned and d a multiple of 4
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
  int mse_only;  // stage one alone: no sketch, no sign bits (sign_words = 0)
  int norm_f16;  // norms stored as float16 pairs (one 32-bit word per row and group)
  int blk_code_words;
  int blk_sign_words;
  int fmt;
  const int64_t* dst_rows;
  int64_t seg_len;
  int64_t seg_stride;
  int64_t seg_offset;
  int64_t n_rows;
  // Block-owned tiling (block records, segment rows, seg_stride % 32 == 0):
  // tile = (segment, pair of 32-row blocks); the workgroup owning the tile is
  // the only writer of those blocks, so partial blocks are read-modify-written.
  int blk_owned;
  int pk_zero;  // token-major: some record word is only partly covered by the waves' fields
  int64_t pairs_per_seg;
  int64_t n_tiles;
  uint32_t* codes;
  uint32_t* signs;
  float* norms;
};

// Stores the norm pair (n_g, gamma_g) of record value pair i = row * n_groups
// + g: two float32, or two float16 (round to nearest even) in one word.
__device__ __forceinline__ void store_norms(float* norms, int f16, int64_t i, float n, float gam) {
  if (f16) {
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v h = {(_Float16)n, (_Float16)gam};
    reinterpret_cast<uint32_t*>(norms)[i] = __builtin_bit_cast(uint32_t, h);
  } else {
    norms[2 * i] = n;
    norms[2 * i + 1] = gam;
  }
}

// Sum over each row of 16 lanes, result in every lane of the row, with DPP
// lane moves (no LDS round trip): swap neighbours, swap pairs, then mirror
// within 8 and within 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t row16_or(uint32_t s) {
  s |= dpp_u<0xB1>(s);
  s |= dpp_u<0x4E>(s);
  s |= dpp_u<0x141>(s);
  s |= dpp_u<0x140>(s);
  return s;
}
__device__ __forceinline__ float row16_sum(float s) {
  s += dpp_f<0xB1>(s);   // quad_perm [1, 0, 3, 2]
  s += dpp_f<0x4E>(s);   // quad_perm [2, 3, 0, 1]
  s += dpp_f<0x141>(s);  // row_half_mirror
  s += dpp_f<0x140>(s);  // row_mirror
  return s;
}

__device__ __forceinline__ int64_t dest_row(const QArgs& a, int64_t i) {
  if (a.dst_rows) return a.dst_rows[i];
  return (i / a.seg_len) * a.seg_stride + a.seg_offset + (i % a.seg_len);
}

// acc[mt] = A[16 mt .. 16 mt + 15][:] x B for the first NMT 16-vector tiles
// (the rest are zeroed). A is the fp32 tile in LDS (row stride XS); B is this
// wave's register fragment. Step (q, j) of lane group lg takes k = 16 q + 4 lg
// + j, so a lane's four k of one q are adjacent in memory on both sides (one
// 16-byte read each) and the four lane groups of a row cover 64 contiguous
// bytes. The NMT accumulator chains are interleaved so consecutive MFMAs are
// independent.
// The same product with the B fragment read from LDS: b4 points at this
// lane's f32x4 of step q = 0; step q is 64 f32x4 further.
template <int NMT, int KPG, int XS>
__device__ __forceinline__ void mfma_tiles_lds(const float* xr, const f32x4* b4, int ln, int lg,
                                               f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < KPG / 4; ++q) {
    f32x4 a4[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      a4[mt] = *reinterpret_cast<const f32x4*>(xr + (mt * 16 + ln) * XS + 16 * q + 4 * lg);
    const f32x4 b = b4[64 * q];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[mt][j], b[j], acc[mt], 0, 0, 0);
  }
}

template <int NMT, int KPG, int XS>
__device__ __forceinline__ void mfma_tiles(const float* xr, const float (&b)[KPG], int ln, int lg,
                                           f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < KPG / 4; ++q) {
    f32x4 a4[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      a4[mt] = *reinterpret_cast<const f32x4*>(xr + (mt * 16 + ln) * XS + 16 * q + 4 * lg);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[mt][j], b[4 * q + j], acc[mt], 0, 0, 0);
  }
}

// The same product with the B fragment read from global memory (the
// row-major d x d matrix m, rows past d and entries past a row's end as
// zeros), one step ahead of its use: for d > 128 the matrix slices are not
// kept in registers (with 13 or 16 waves per workgroup they would not fit
// without spills); a wave's 16 rows stay in the caches across tiles.
template <int NMT, int KPG, int XS>
__device__ __forceinline__ void mfma_tiles_gmem(const float* xr, const float* m, int d, int m_vec, int orow, int ln,
                                                int lg, f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool row_ok = orow < d;
  const float* rowp = m + (int64_t)(row_ok ? orow : d - 1) * d;
  auto ld = [&](int q) __attribute__((always_inline)) -> f32x4 {
    const int k = 16 * q + 4 * lg;
    f32x4 v;
    if (m_vec) {
      v = *reinterpret_cast<const f32x4*>(rowp + (k < d ? k : d - 4));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = rowp[k + j < d ? k + j : d - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!row_ok || k + j >= d) v[j] = 0.f;
    return v;
  };
  f32x4 b = ld(0);
#pragma unroll 1
  for (int q = 0; q < KPG / 4; ++q) {
    const f32x4 bn = ld(q + 1 < KPG / 4 ? q + 1 : q);
    f32x4 a4[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      a4[mt] = *reinterpret_cast<const f32x4*>(xr + (mt * 16 + ln) * XS + 16 * q + 4 * lg);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[mt][j], b[j], acc[mt], 0, 0, 0);
    b = bn;
  }
}

// LDS layout (bytes), KP = padded K, NT = number of 16-wide coordinate tiles.
// H: the half-precision MFMA variant (bf16 input tile, fp16 residual parts):
// the input tile is bf16 [QT][XH]; once the rotation has read it, the same
// bytes hold the high fp16 part of the scaled residual, and off_rl its low
// part (both [QT][XH]).
template <int KP, int NT, bool H = false>
struct Lds {
  static constexpr int XS = KP + 4;  // row stride of the fp32 tile, in floats
  // row stride of the 16-bit tiles: 16 bytes of padding shift consecutive
  // rows by four banks, so the 16 rows one 16-byte operand read spans fall
  // in disjoint banks
  static constexpr int XH = KP + 8;
  // row stride of the code and sign bytes: 4 bytes of padding put the rows
  // that one byte store spans (four vectors, 4 DP bytes apart) in different
  // LDS banks
  static constexpr int DP = NT * 16 + 4;
  static constexpr int off_x = 0;                                   // float [QT][XS] (H: u16 [QT][XH])
  static constexpr int off_rl = off_x + (H ? QT * XH * 2 : 0);      // H: u16 [QT][XH]
  static constexpr int off_code = off_rl + (H ? QT * XH * 2 : QT * XS * 4);  // u8 [QT][DP]
  static constexpr int off_sign = off_code + QT * DP;               // u8 [QT][DP]
  static constexpr int off_npart = off_sign + QT * DP;              // float [NT][QT]
  static constexpr int off_gpart = off_npart + NT * QT * 4;         // float [NT][QT]
  static constexpr int off_nrm = off_gpart + NT * QT * 4;           // float [2][QT]
  static constexpr int off_cb = off_nrm + 2 * QT * 4;               // float [64]
  static constexpr int off_rows = off_cb + 64 * 4;                  // int64 [QT]
  static constexpr int off_flags = off_rows + QT * 8;               // int [4]
  // packed token-major records: codes (at most 4 bits x KP) then signs, plus
  // slack for per-group rounding and for the last wave's bits past the end
  static constexpr int PKW = KP * 4 / 32 + KP / 32 + 4;
  static constexpr int off_pk = off_flags + 16;                     // u32 [QT][PKW]
  // every wave's slice of sketch_rot, in MFMA operand order: [NT][KP/16][64 lanes]
  // f32x4 (d <= 128; larger d keeps it in registers)
  static constexpr bool SKR_LDS = KP <= 128 && !H;
  static constexpr int off_skr = (off_pk + QT * PKW * 4 + 15) / 16 * 16;
  static constexpr int bytes = off_skr + (SKR_LDS ? NT * KP * 64 : 0);
};

// Vectors of one tile: [v0, v0 + nvalid). With block-owned tiling they are
// those of one segment falling in one aligned pair of blocks, whose first row
// is rowbase; slot_lo is the first vector's position in the pair.
struct TileGeo {
  int64_t v0, rowbase;
  int nvalid, slot_lo;
};

// Geometry of `tile`; false when it holds no vector (block-owned tiling).
__device__ __forceinline__ bool tile_geo(const QArgs& a, int64_t tile, TileGeo& g) {
  g.rowbase = 0;
  g.slot_lo = 0;
  if (a.blk_owned) {
    const int64_t sg = tile / a.pairs_per_seg, pr = tile % a.pairs_per_seg;
    const int o32 = (int)(a.seg_offset % 32);
    const int64_t rem = a.n_vec - sg * a.seg_len;
    const int64_t len = rem < a.seg_len ? rem : a.seg_len;
    const int64_t lo = 64 * pr - o32 > 0 ? 64 * pr - o32 : 0;  // segment-relative
    const int64_t hi = 64 * pr + 64 - o32 < len ? 64 * pr + 64 - o32 : len;
    if (hi <= lo) return false;
    g.v0 = sg * a.seg_len + lo;
    g.nvalid = (int)(hi - lo);
    g.rowbase = sg * a.seg_stride + (a.seg_offset - o32) + 64 * pr;
    g.slot_lo = (int)(lo + o32 - 64 * pr);
  } else {
    g.v0 = tile * QT;
    g.nvalid = (int)((a.n_vec - g.v0) < QT ? (a.n_vec - g.v0) : QT);
  }
  return true;
}

// The first tile at or after `tile` (in steps of `stride`) that holds
// vectors, or n_tiles. Uniform across the workgroup.
__device__ __forceinline__ int64_t next_live_tile(const QArgs& a, int64_t tile, int64_t stride, TileGeo& g) {
  for (; tile < a.n_tiles; tile += stride)
    if (tile_geo(a, tile, g)) return tile;
  return a.n_tiles;
}

// A thread's share of one input tile (QT KP / (64 NT) = 16 values) and the
// destination row of vector tid, held in registers between the global loads
// and the LDS stores.
struct XStage {
  u32x4 v[4];
  int64_t row;
};

template <int KP, int NT>
__device__ __forceinline__ void load_x(const QArgs& a, const TileGeo& g, int tid, XStage& st) {
  static_assert(QT * KP / (NT * 64) == 16, "16 values per thread");
  const int d = a.d;
  st.row = -1;
  if (tid < g.nvalid) st.row = a.blk_owned ? g.rowbase + g.slot_lo + tid : dest_row(a, g.v0 + tid);
  if (a.x_vec) {
    // rows are 16-byte aligned and d is a multiple of the vector width:
    // 16-byte loads, 8 bf16 or 4 fp32 values each
    if (a.x_bf16) {
      constexpr int CPR = KP / 8, NCH = QT * CPR / (NT * 64);  // chunks per row, per thread
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
        st.v[i] = (v < g.nvalid && k < d)
                      ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.x) +
                                                        (g.v0 + v) * a.x_stride + k)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      constexpr int CPR = KP / 4, NCH = QT * CPR / (NT * 64);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 4;
        st.v[i] = (v < g.nvalid && k < d)
                      ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.x) +
                                                        (g.v0 + v) * a.x_stride + k)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + i * NT * 64, v = e / KP, k = e % KP;
      uint32_t val = 0u;
      if (v < g.nvalid && k < d) {
        const int64_t off = (g.v0 + v) * a.x_stride + k;
        val = a.x_bf16 ? ((uint32_t) reinterpret_cast<const uint16_t*>(a.x)[off]) << 16
                       : __float_as_uint(reinterpret_cast<const float*>(a.x)[off]);
      }
      st.v[i / 4][i % 4] = val;
    }
  }
}

// The tile as fp32 in LDS (row stride XS), zero padded.
template <int KP, int NT, int XS>
__device__ __forceinline__ void store_x(const QArgs& a, const XStage& st, int tid, float* xr) {
  if (a.x_vec) {
    if (a.x_bf16) {
      constexpr int CPR = KP / 8, NCH = QT * CPR / (NT * 64);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = st.v[i][e];
          const float f0 = __uint_as_float(w << 16), f1 = __uint_as_float(w & 0xFFFF0000u);
          if (e < 2) {
            lo[2 * e] = f0;
            lo[2 * e + 1] = f1;
          } else {
            hi[2 * e - 4] = f0;
            hi[2 * e - 3] = f1;
          }
        }
        *reinterpret_cast<f32x4*>(xr + v * XS + k) = lo;
        *reinterpret_cast<f32x4*>(xr + v * XS + k + 4) = hi;
      }
    } else {
      constexpr int CPR = KP / 4, NCH = QT * CPR / (NT * 64);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 4;
        const u32x4 w = st.v[i];
        *reinterpret_cast<f32x4*>(xr + v * XS + k) =
            f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + i * NT * 64;
      xr[(e / KP) * XS + e % KP] = __uint_as_float(st.v[i / 4][i % 4]);
    }
  }
}

// The tile as bf16 in LDS (row stride XH, 16-bit units), zero padded: the
// half-precision variant takes bf16 rows that load_x read as 16-byte chunks.
template <int KP, int NT, int XH>
__device__ __forceinline__ void store_xh(const XStage& st, int tid, uint16_t* xh) {
  constexpr int CPR = KP / 8, NCH = QT * CPR / (NT * 64);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
    *reinterpret_cast<u32x4*>(xh + v * XH + k) = st.v[i];
  }
}

// Round to nearest even of an fp32 value to bf16, as the bits of the bf16
// value (finite inputs), and the fp32 value of bf16 bits.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// acc[mt] = A[16 mt .. 16 mt + 15][:] x B on v_mfma_f32_16x16x32_bf16 for the
// first NMT 16-vector tiles, B = BH + BM + BL (three bf16 parts of an fp32
// matrix). A is the bf16 tile in LDS (row stride XH). Step s of lane group lg
// takes k = 32 s + 8 lg + j, j = 0 .. 7: one 16-byte read per operand. The
// small parts go first in each step.
template <int NMT, int KS, int XH>
__device__ __forceinline__ void mfma_tiles_bf16x3(const uint16_t* xh, const u32x4 (&bh)[KS], const u32x4 (&bm)[KS],
                                                  const u32x4 (&bl)[KS], int ln, int lg, f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 a[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      a[mt] = *reinterpret_cast<const u32x4*>(xh + (mt * 16 + ln) * XH + 32 * s + 8 * lg);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(a[mt], bl[s], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(a[mt], bm[s], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(a[mt], bh[s], acc[mt]);
  }
}

// The same shape on v_mfma_f32_16x16x32_f16 with both operands in two fp16
// parts, A = AH + AL (tiles ah, al in LDS) and B = BH + BL: the products
// AL BH, AH BL and AH BH (AL BL, below 2^-22 of a term, is dropped).
template <int NMT, int KS, int XH>
__device__ __forceinline__ void mfma_tiles_f16x2(const uint16_t* ah, const uint16_t* al, const u32x4 (&bh)[KS],
                                                 const u32x4 (&bl)[KS], int ln, int lg, f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 a_h[NMT], a_l[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int off = (mt * 16 + ln) * XH + 32 * s + 8 * lg;
      a_h[mt] = *reinterpret_cast<const u32x4*>(ah + off);
      a_l[mt] = *reinterpret_cast<const u32x4*>(al + off);
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(a_l[mt], bh[s], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(a_h[mt], bl[s], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(a_h[mt], bh[s], acc[mt]);
  }
}

// Code word wd of block blk = block h of a block-owned tile's pair: the
// fields of the pair's rows [vlo, vhi) (row t is the tile's vector
// t - slot_lo; its codes are LDS bytes [vector][DP]). A word that also holds
// rows outside the tile has the tile's bits cleared and then set by two
// atomics, which need no read round trip (no other workgroup writes these
// blocks in the call).
template <int DP>
__device__ __forceinline__ void store_blk_code_word(const QArgs& a, const uint8_t* code_b, int64_t blk, int wd,
                                                    int h, int vlo, int vhi, int slot_lo) {
  const int g = (a.n_groups > 1 && wd >= a.bcwoff[1]) ? 1 : 0;
  const int m = a.gbits[g], dg = a.gdim[g];
  const int lw = wd - a.bcwoff[g];
  const int b0 = 32 * lw;
  const int u0 = b0 / (8 * m), u1 = (b0 + 31) / (8 * m);
  const uint64_t fm = (1u << m) - 1u;
  uint64_t word = 0, mask = 0;
  for (int u = u0; u <= u1 && u < 4 * dg; ++u) {
    const int o = u / dg, j = u % dg;
    uint64_t unit = 0, umask = 0;
    const int base = 32 * h + 8 * o;  // row of slot 0 of the unit
    const int s0 = vlo > base ? vlo - base : 0, s1 = vhi < base + 8 ? vhi - base : 8;
    for (int sl = s0; sl < s1; ++sl) {
      unit |= (uint64_t)code_b[(base + sl - slot_lo) * DP + a.choff[g] + j] << (m * sl);
      umask |= fm << (m * sl);
    }
    const int pos = 8 * m * u - b0;
    word |= pos >= 0 ? unit << pos : unit >> (-pos);
    mask |= pos >= 0 ? umask << pos : umask >> (-pos);
  }
  uint32_t* dst = a.codes + blk * a.blk_code_words + wd;
  const uint32_t m32 = (uint32_t)mask;
  if (m32 == 0xFFFFFFFFu) {
    *dst = (uint32_t)word;
  } else if (m32 != 0) {
    atomicAnd(dst, ~m32);
    atomicOr(dst, (uint32_t)word & m32);
  }
}

// Sign word wd of the same block, from the LDS sign bytes.
template <int DP>
__device__ __forceinline__ void store_blk_sign_word(const QArgs& a, const uint8_t* sign_b, int64_t blk, int wd,
                                                    int h, int vlo, int vhi, int slot_lo) {
  const int g = (a.n_groups > 1 && wd >= a.bswoff[1]) ? 1 : 0;
  const int dg = a.gdim[g];
  const int lw = wd - a.bswoff[g];
  uint32_t word = 0, mask = 0;
  for (int q = 0; q < 4; ++q) {
    const int u = 4 * lw + q;
    const int o = u / dg, j = u % dg;
    const int base = 32 * h + 8 * o;
    const int s0 = vlo > base ? vlo - base : 0, s1 = vhi < base + 8 ? vhi - base : 8;
    for (int sl = s0; sl < s1; ++sl) {
      word |= (uint32_t)sign_b[(base + sl - slot_lo) * DP + a.choff[g] + j] << (8 * q + sl);
      mask |= 1u << (8 * q + sl);
    }
  }
  uint32_t* dst = a.signs + blk * a.blk_sign_words + wd;
  if (mask == 0xFFFFFFFFu) {
    *dst = word;
  } else if (mask != 0) {
    atomicAnd(dst, ~mask);
    atomicOr(dst, word & mask);
  }
}

// The kernel body: this workgroup quantizes tiles first_tile,
// first_tile + tile_stride, ... of `a`, with NT * 64 threads and the dynamic
// LDS block `smem` (Lds<KP, NT, H>::bytes).
//
// H selects the half-precision MFMA variant (bf16 inputs with 16-byte rows,
// d a multiple of 8, KP <= 128; h_path_ok). Both products still reach
// fp32-grade results:
//  - y = rot x: x is exact in bf16 and rot = RH + RM + RL (three bf16 parts,
//    together within 2^-27 of rot), so the three v_mfma_f32_16x16x32_bf16
//    products are exact term by term and only the fp32 accumulation rounds.
//  - s = sketch_rot r: the sign of s is what is kept, and it does not change
//    when a row of sketch_rot or the residual of one (vector, group) is
//    scaled by a power of two. Each row of sketch_rot is scaled so that its
//    largest entry lies in [2^13, 2^14), each residual so that its group
//    norm lies in [2^9, 2^10) (|r_k| < 2 n_g, so every scaled value fits
//    fp16), and both are split into fp16 high and low parts (22 bits); the
//    products AL BH + AH BL + AH BH on v_mfma_f32_16x16x32_f16 leave out
//    AL BL, below 2^-22 of each term.
template <int KP, int NT, bool H = false>
__device__ __forceinline__ void quantize_tiles(const QArgs& a, int64_t first_tile, int64_t tile_stride,
                                               unsigned char* smem) {
  using L = Lds<KP, NT, H>;
  constexpr int XS = L::XS;
  constexpr int XH = L::XH;
  constexpr int DP = L::DP;
  constexpr int KPG = KP / 4;  // k values per lane group
  constexpr int KS = KP / 32;  // k steps of the half-precision products
  static_assert(KP == NT * 16 && KPG % 4 == 0, "tile shape");
  static_assert(!H || (KP % 32 == 0 && KP <= 128), "half-precision variant: KP in {64, 128}");
  float* xr = reinterpret_cast<float*>(smem + L::off_x);
  uint16_t* xh = reinterpret_cast<uint16_t*>(smem + L::off_x);   // H: bf16 tile, then the residual's high part
  uint16_t* rl = reinterpret_cast<uint16_t*>(smem + L::off_rl);  // H: the residual's low part
  uint8_t* code_b = smem + L::off_code;
  uint8_t* sign_b = smem + L::off_sign;
  float* npart = reinterpret_cast<float*>(smem + L::off_npart);
  float* gpart = reinterpret_cast<float*>(smem + L::off_gpart);
  float* nrm = reinterpret_cast<float*>(smem + L::off_nrm);
  float* cbk = reinterpret_cast<float*>(smem + L::off_cb);  // [0,32): centroids, [32,64): boundaries
  int64_t* rows = reinterpret_cast<int64_t*>(smem + L::off_rows);
  int* flags = reinterpret_cast<int*>(smem + L::off_flags);
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem + L::off_pk);
  uint16_t* pk16 = reinterpret_cast<uint16_t*>(smem + L::off_pk);
  constexpr int PKW = L::PKW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;  // wave = coordinate tile
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int d = a.d;

  // Every global load of the prologue and of the first tile is issued before
  // the first wait, so the kernel pays one memory latency up front.
  // Centroids of both groups (concatenated), kept in a register until the
  // tile's LDS stores.
  float cent_reg = 0.f;
  {
    const int ncent = (1 << a.gbits[0]) + (a.n_groups > 1 ? (1 << a.gbits[1]) : 0);
    cent_reg = a.centroids[tid < ncent ? tid : ncent - 1];
  }
  // the first tile's vectors and destination rows (the next tile's are
  // loaded at the end of each pass)
  TileGeo g;
  int64_t tile = next_live_tile(a, first_tile, tile_stride, g);
  XStage st;
  if (tile < a.n_tiles) load_x<KP, NT>(a, g, tid, st);

  // This wave's rows of rot and sketch_rot: B[k][n] = M[16 w + n][k], with k
  // assigned to steps as in mfma_tiles. The loads are unconditional (indices
  // clamped into the matrix) so they issue back to back; out-of-range entries
  // are zeroed afterwards.
  const int ocoord = w * 16 + ln;  // output coordinate of this lane
  constexpr bool SKR_LDS = L::SKR_LDS;
  // For d <= 128 the sketch slice lives in LDS (read once per product), which
  // leaves the register file to the rotation slice and the tile's values;
  // larger d keeps both slices in registers.
  // (for KP > 128 both slices are read from global memory in the products)
  constexpr bool GMEM = KP > 128 && !H;
  float brot[H || GMEM ? 1 : KPG];
  constexpr bool SKR_GMEM = GMEM;
  static_assert(SKR_LDS || H || GMEM, "the sketch slice is in LDS, registers or global memory");
  f32x4* skr_lds = reinterpret_cast<f32x4*>(smem + L::off_skr);
  // H: the same slices as B operands of the 16x16x32 products, lane (ln, lg)
  // holding M[16 w + ln][32 s + 8 lg + j], j = 0 .. 7, as 16-bit pairs:
  // rot in three bf16 parts, sketch_rot (row-scaled) in two fp16 parts
  u32x4 rh[H ? KS : 1], rm[H ? KS : 1], rlo[H ? KS : 1], sh[H ? KS : 1], sl[H ? KS : 1];
  if constexpr (H) {
    const bool row_ok = ocoord < a.d;
    const int64_t rb = (int64_t)(row_ok ? ocoord : a.d - 1) * a.d;
    f32x4 mr[KS][2], ms[KS][2];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        // (d is a multiple of 8: a lane's 8 entries are all inside the row or all past it)
        const int k = 32 * s2 + 8 * lg + 4 * hlf;
        const int kc = k < a.d ? k : 0;
        mr[s2][hlf] = *reinterpret_cast<const f32x4*>(a.rot + rb + kc);
        ms[s2][hlf] = *reinterpret_cast<const f32x4*>(a.skr + rb + kc);
        if (!row_ok || 32 * s2 + 8 * lg >= a.d) {
          mr[s2][hlf] = f32x4{0.f, 0.f, 0.f, 0.f};
          ms[s2][hlf] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    // largest |entry| of the sketch row: the lane's 8 KS entries, then the
    // four lane groups of the row
    float mx = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(ms[s2][e / 4][e % 4]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float ssc = mx > 0.f ? __builtin_amdgcn_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(mx)) : 1.0f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      uint32_t wh[4], wm[4], wl[4], vh[4], vl[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h2[2], m2[2], l2[2];
        f16x2 sh2, sl2;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v = mr[s2][p / 2][2 * (p % 2) + e];
          h2[e] = bf16_rne(v);
          const float r1 = v - bf16_val(h2[e]);
          m2[e] = bf16_rne(r1);
          l2[e] = bf16_rne(r1 - bf16_val(m2[e]));
          const float u = ms[s2][p / 2][2 * (p % 2) + e] * ssc;
          const _Float16 uh = (_Float16)u;
          sh2[e] = uh;
          sl2[e] = (_Float16)(u - (float)uh);
        }
        wh[p] = h2[0] | (h2[1] << 16);
        wm[p] = m2[0] | (m2[1] << 16);
        wl[p] = l2[0] | (l2[1] << 16);
        vh[p] = __builtin_bit_cast(uint32_t, sh2);
        vl[p] = __builtin_bit_cast(uint32_t, sl2);
      }
      rh[s2] = u32x4{wh[0], wh[1], wh[2], wh[3]};
      rm[s2] = u32x4{wm[0], wm[1], wm[2], wm[3]};
      rlo[s2] = u32x4{wl[0], wl[1], wl[2], wl[3]};
      sh[s2] = u32x4{vh[0], vh[1], vh[2], vh[3]};
      sl[s2] = u32x4{vl[0], vl[1], vl[2], vl[3]};
    }
  } else if constexpr (!GMEM) {
    float bs[SKR_LDS ? KPG : 1];
    const int64_t rb = (int64_t)(ocoord < d ? ocoord : d - 1) * d;
    if (a.m_vec) {
      // d is a multiple of 4 and the matrices are 16-byte aligned
#pragma unroll
      for (int q = 0; q < KPG / 4; ++q) {
        const int k = 16 * q + 4 * lg;
        const int kc = k < d ? k : d - 4;
        const f32x4 r4 = *reinterpret_cast<const f32x4*>(a.rot + rb + kc);
#pragma unroll
        for (int j = 0; j < 4; ++j) brot[4 * q + j] = r4[j];
        if constexpr (SKR_LDS) {
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(a.skr + rb + kc);
#pragma unroll
          for (int j = 0; j < 4; ++j) bs[4 * q + j] = s4[j];
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        const int k = 16 * (kk / 4) + 4 * lg + kk % 4;
        const int kc = k < d ? k : d - 1;
        brot[kk] = a.rot[rb + kc];
        if constexpr (SKR_LDS) bs[kk] = a.skr[rb + kc];
      }
    }
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const bool ok = ocoord < d && 16 * (kk / 4) + 4 * lg + kk % 4 < d;
      brot[kk] = ok ? brot[kk] : 0.f;
      if constexpr (SKR_LDS) bs[kk] = ok ? bs[kk] : 0.f;
    }
    if constexpr (SKR_LDS) {
#pragma unroll
      for (int q = 0; q < KPG / 4; ++q)
        skr_lds[(w * (KPG / 4) + q) * 64 + lane] = f32x4{bs[4 * q], bs[4 * q + 1], bs[4 * q + 2], bs[4 * q + 3]};
    }
  }
  // group of this wave's coordinates (group boundaries are multiples of 16);
  // everything derived from it is wave-uniform
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int grp = (a.n_groups > 1 && wu * 16 >= a.choff[1]) ? 1 : 0;
  const int nb = (1 << a.gbits[grp]) - 1;
  const int coff = a.coff[grp];
  const int boff = a.boff[grp];
  const int mg = a.gbits[grp];
  const int wig = wu - a.choff[grp] / 16;  // wave index within its group
  // halfword offsets, in a packed token-major row, of this wave's 16 codes
  // (2 mg bytes) and of its 16 sign bits
  const int pk_code_h = 2 * a.cwoff[grp] + mg * wig;
  const int pk_sign_h = 2 * (a.code_words + a.swoff[grp]) + wig;
  const bool tok = a.fmt == TQ_TOKEN_MAJOR;
  // decision boundaries of both groups (concatenated), like the centroids
  float bnd_reg = 0.f;
  {
    const int nbt = ((1 << a.gbits[0]) - 1) + (a.n_groups > 1 ? (1 << a.gbits[1]) - 1 : 0);
    bnd_reg = a.boundaries[tid < nbt ? tid : nbt - 1];
  }

  while (tile < a.n_tiles) {
    const int64_t rowbase = g.rowbase;
    const int nvalid = g.nvalid, slot_lo = g.slot_lo;

    // ---- stage the input tile (fp32, zero padded) and destination rows ----
    if (tok && a.pk_zero)
      for (int e = tid; e < QT * PKW; e += NT * 64) pk[e] = 0u;
    if constexpr (H)
      store_xh<KP, NT, XH>(st, tid, xh);
    else
      store_x<KP, NT, XS>(a, st, tid, xr);
    if (tid < QT) rows[tid] = (st.row < 0 || st.row >= a.n_rows) ? -1 : st.row;
    if (tid < 32) {
      cbk[tid] = cent_reg;
      cbk[32 + tid] = bnd_reg;
    }
    __syncthreads();

    // ---- y = rot x (fp32 MFMA), four 16-vector tiles ----
    // (a tile with at most 16 vectors, e.g. an append, runs only its first
    // 16-vector tile)
    const int n_mt = (nvalid + 15) / 16;
    f32x4 yacc[4];
    if constexpr (H) {
      if (n_mt == 1)
        mfma_tiles_bf16x3<1, KS, XH>(xh, rh, rm, rlo, ln, lg, yacc);
      else
        mfma_tiles_bf16x3<4, KS, XH>(xh, rh, rm, rlo, ln, lg, yacc);
    } else if constexpr (GMEM) {
      if (n_mt == 1)
        mfma_tiles_gmem<1, KPG, XS>(xr, a.rot, d, a.m_vec, ocoord, ln, lg, yacc);
      else
        mfma_tiles_gmem<4, KPG, XS>(xr, a.rot, d, a.m_vec, ocoord, ln, lg, yacc);
    } else {
      if (n_mt == 1)
        mfma_tiles<1, KPG, XS>(xr, brot, ln, lg, yacc);
      else
        mfma_tiles<4, KPG, XS>(xr, brot, ln, lg, yacc);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= n_mt) break;
      // lane (ln, lg) holds y[vector 16 mt + 4 lg + i][coordinate 16 w + ln]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = yacc[mt][i] * yacc[mt][i];
        s = row16_sum(s);
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
    // (this group's boundaries, wave-uniform LDS reads; +inf past the last)
    float tb[15];
#pragma unroll
    for (int k = 0; k < 15; ++k)
      tb[k] = k < nb ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cbk[32 + boff + k])))
                     : INFINITY;
    // In phases over a lane's four vectors of a 16-vector tile: LDS reads,
    // arithmetic, then LDS stores and row reductions, so no store sits
    // between two reads (the reads of one phase are in flight together).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= n_mt) break;  // tiles past the last vector: their rows stay zero
      float nv[4], cv[4], rr[4];
      int idx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) nv[i] = nrm[grp * QT + mt * 16 + lg * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // cell = number of boundaries below u (the +inf entries past the
        // group's count never are); fully unrolled so tb stays in SGPRs.
        // A zero vector takes the middle cell and a zero residual.
        const float u = yacc[mt][i] * __builtin_amdgcn_rcpf(nv[i]);
        int c = 0;
#pragma unroll
        for (int k = 0; k < 15; ++k) c += u > tb[k] ? 1 : 0;
        idx[i] = nv[i] > 0.f ? c : (nb + 1) / 2 - 1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) cv[i] = cbk[coff + idx[i]];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rr[i] = nv[i] > 0.f ? fmaf(-nv[i], cv[i], yacc[mt][i]) : 0.f;
        if (ocoord >= d) {
          rr[i] = 0.f;
          idx[i] = 0;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = mt * 16 + lg * 4 + i;
        code_b[v * DP + ocoord] = (uint8_t)idx[i];
        // A operand of the sketch product (k = rotated coordinate)
        if constexpr (H) {
          // scaled so that the group norm lies in [2^9, 2^10), in two fp16 parts
          const float sc = nv[i] > 0.f ? __builtin_amdgcn_ldexpf(1.0f, 10 - __builtin_amdgcn_frexp_expf(nv[i])) : 1.0f;
          const float u = rr[i] * sc;
          const _Float16 uh = (_Float16)u;
          xh[v * XH + ocoord] = __builtin_bit_cast(uint16_t, uh);
          rl[v * XH + ocoord] = __builtin_bit_cast(uint16_t, (_Float16)(u - (float)uh));
        } else {
          xr[v * XS + ocoord] = rr[i];
        }
      }
      if (tok) {
        // the row's 16 codes of this wave, OR-combined across the row of
        // lanes, are 2 mg bytes of the packed record
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t f = (uint64_t)(uint32_t)idx[i] << (mg * ln);
          lo[i] = row16_or((uint32_t)f);
          hi[i] = mg > 2 ? row16_or((uint32_t)(f >> 32)) : 0u;
        }
        if (ln == 0) {
          // (one base address; the vector and halfword offsets are constants)
          uint16_t* row = pk16 + lg * 4 * 2 * PKW + pk_code_h;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (k < mg) row[(mt * 16 + i) * 2 * PKW + k] = (uint16_t)((k < 2 ? lo[i] : hi[i]) >> (16 * (k & 1)));
        }
      }
      float ss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ss[i] = row16_sum(rr[i] * rr[i]);
      if (ln == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gpart[w * QT + mt * 16 + lg * 4 + i] = ss[i];
      }
    }
    // (every k < KP is a coordinate owned by some wave, so the residual tile
    // is fully written, with zeros past d)
    __syncthreads();

    // ---- s = (S Pi^T) r (fp32 MFMA); sign bit = [s >= 0] (not for MSE-only records) ----
    if (!a.mse_only) {
      f32x4 sacc[4];
      if constexpr (H) {
        if (n_mt == 1)
          mfma_tiles_f16x2<1, KS, XH>(xh, rl, sh, sl, ln, lg, sacc);
        else
          mfma_tiles_f16x2<4, KS, XH>(xh, rl, sh, sl, ln, lg, sacc);
      } else if constexpr (SKR_LDS) {
        if (n_mt == 1)
          mfma_tiles_lds<1, KPG, XS>(xr, skr_lds + w * (KPG / 4) * 64 + lane, ln, lg, sacc);
        else
          mfma_tiles_lds<4, KPG, XS>(xr, skr_lds + w * (KPG / 4) * 64 + lane, ln, lg, sacc);
      } else {
        if (n_mt == 1)
          mfma_tiles_gmem<1, KPG, XS>(xr, a.skr, d, a.m_vec, ocoord, ln, lg, sacc);
        else
          mfma_tiles_gmem<4, KPG, XS>(xr, a.skr, d, a.m_vec, ocoord, ln, lg, sacc);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt >= n_mt) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = mt * 16 + lg * 4 + i;
          const bool bit = sacc[mt][i] >= 0.f && ocoord < d;
          sign_b[v * DP + ocoord] = bit ? 1 : 0;
          // the wave's 16 channels for vector 16 mt + 4 q + i are ballot bits [16 q, 16 q + 16)
          const uint64_t bal = __builtin_amdgcn_ballot_w64(bit);
          if (tok && lane < 4)
            pk16[(mt * 16 + lane * 4 + i) * 2 * PKW + pk_sign_h] = (uint16_t)(bal >> (16 * lane));
        }
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
        store_norms(a.norms, a.norm_f16, row * a.n_groups + g, nrm[g * QT + v], sqrtf(s));
      }
    }
    if (tok) {
      // packed records: code words then sign words, copied word by word
      const int cw = a.code_words, sw = a.sign_words, rw = cw + sw;
      for (int e = tid; e < QT * rw; e += NT * 64) {
        const int v = e / rw, wd = e % rw;
        const int64_t row = rows[v];
        if (row < 0) continue;
        if (wd < cw)
          a.codes[row * cw + wd] = pk[v * PKW + wd];
        else
          a.signs[row * sw + wd - cw] = pk[v * PKW + wd];
      }
    } else if (a.blk_owned) {
      // block records, tile = one aligned pair of blocks owned by this
      // workgroup: each word is assembled from the tile's fields; in a word
      // that also holds rows outside the tile, the tile's bits are cleared
      // and then set by two atomics, which need no read round trip (no other
      // workgroup writes these blocks in this call)
      for (int h = 0; h < 2; ++h) {
        const int vlo = slot_lo > 32 * h ? slot_lo : 32 * h;
        const int vhi = slot_lo + nvalid < 32 * h + 32 ? slot_lo + nvalid : 32 * h + 32;
        if (vhi <= vlo) continue;
        const int64_t blk = rowbase / 32 + h;
        for (int wd = tid; wd < a.blk_code_words; wd += NT * 64)
          store_blk_code_word<DP>(a, code_b, blk, wd, h, vlo, vhi, slot_lo);
        for (int wd = tid; wd < a.blk_sign_words; wd += NT * 64)
          store_blk_sign_word<DP>(a, sign_b, blk, wd, h, vlo, vhi, slot_lo);
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
        if (a.mse_only) continue;
        const int spos = 8 * (o * dg + j) + s;
        uint32_t* sbase = a.signs + blk * a.blk_sign_words + a.bswoff[g];
        const uint32_t sbit = sign_b[v * DP + ch];
        atomicAnd(sbase + spos / 32, ~(1u << (spos % 32)));
        atomicOr(sbase + spos / 32, sbit << (spos % 32));
      }
    }
    __syncthreads();
    tile = next_live_tile(a, tile + tile_stride, tile_stride, g);
    if (tile < a.n_tiles) load_x<KP, NT>(a, g, tid, st);
  }
}

// ---------------------------------------------------------------------------
// Latency path for a few vectors (the appends of a decode step): one
// workgroup of 512 threads per vector and no tiles. Thread t owns output
// coordinate o = t / 4 and a quarter of the inner index (h = t % 4: the
// 16-byte chunks 16 i + 4 h). Its pieces of rot and sketch_rot (8 x 16
// bytes each) and the matching entries of the vector are loaded at once,
// each product is four fp32 FMA chains summed within the lane quad, and
// three barriers separate the group norms, the cells and residual, and the
// sign bits. Codes and signs are
// assembled into record words in LDS. A token-major record belongs to its
// row alone and is stored word by word; a block record shares its words with
// the block's other tokens (possibly written by other workgroups of the same
// call), so each touched word takes this vector's bits by an atomic AND
// (clear) and an atomic OR (set) on exactly those bits.
// ---------------------------------------------------------------------------
constexpr int kSmallMaxVec = 512;   // calls with at most this many vectors take this path
constexpr int kSmallThreads = 512;
constexpr int kSmallWords = 768;    // record words assembled in LDS

template <int NTHR>
struct SmallLds {
  static constexpr int off_np = 0;                        // float [8]: per-wave sums of y^2
  static constexpr int off_gp = off_np + 8 * 4;           // float [8]: per-wave sums of r^2
  static constexpr int off_r = off_gp + 8 * 4;            // float [128]: rotated residual
  static constexpr int off_bits = off_r + 128 * 4;        // u32 [kSmallWords]
  static constexpr int off_mask = off_bits + kSmallWords * 4;
  static constexpr int bytes = off_mask + kSmallWords * 4;
};

// Whether a call (already validated by make_qargs) takes the latency path.
inline bool small_path_ok(const QArgs& a) {
  const int words = a.fmt == TQ_TOKEN_MAJOR ? a.code_words + a.sign_words : a.blk_code_words + a.blk_sign_words;
  return a.n_vec <= kSmallMaxVec && a.d <= 128 && a.d >= 4 && a.m_vec && words <= kSmallWords;
}

// Sum over the whole wave, the same value in every lane (lane moves only:
// DPP within rows of 16, then swaps of the 32-lane halves and of the 16-lane
// rows inside each half).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum of the per-wave partials p[w0 .. w1) (in that order) from LDS, read as
// two 16-byte words.
__device__ __forceinline__ float wave_range_sum(const float* p, int w0, int w1) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += (k >= w0 && k < w1) ? v[k] : 0.f;
  return s;
}

// ORs an m-bit field at bit position pos of the LDS words into bits / mask.
__device__ __forceinline__ void or_field(uint32_t* bits, uint32_t* mask, int pos, uint32_t val, int m) {
  const int wi = pos >> 5, bi = pos & 31;
  const uint32_t fm = (1u << m) - 1u;
  atomicOr(bits + wi, val << bi);
  atomicOr(mask + wi, fm << bi);
  if (bi + m > 32) {
    atomicOr(bits + wi + 1, val >> (32 - bi));
    atomicOr(mask + wi + 1, fm >> (32 - bi));
  }
}

template <int NTHR>
__device__ __forceinline__ void quantize_small(const QArgs& a, int64_t vec, unsigned char* smem) {
  static_assert(NTHR == 512, "four threads per output coordinate, d <= 128");
  using L = SmallLds<NTHR>;
  float* s_np = reinterpret_cast<float*>(smem + L::off_np);
  float* s_gp = reinterpret_cast<float*>(smem + L::off_gp);
  float* s_r = reinterpret_cast<float*>(smem + L::off_r);
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(smem + L::off_bits);
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem + L::off_mask);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int o = tid >> 2, h = tid & 3;
  const int d = a.d;
  const bool tok = a.fmt == TQ_TOKEN_MAJOR;

  // ---- loads, all issued before the first use: rows o of rot and
  // sketch_rot (indices clamped into the matrix, out-of-range entries zeroed
  // afterwards), the matching entries of the vector, the codebook (lane k of
  // every 16 holds centroid k and boundary k). Thread h of a coordinate takes
  // the 16-byte chunks k = 16 i + 4 h, i = 0 .. 7, so the four threads of a
  // row read 64 contiguous bytes per load instruction ----
  const int oc = o < d ? o : d - 1;
  f32x4 rq[8], sq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = 16 * i + 4 * h, kc = k < d ? k : d - 4;
    rq[i] = *reinterpret_cast<const f32x4*>(a.rot + (int64_t)oc * d + kc);
    sq[i] = *reinterpret_cast<const f32x4*>(a.skr + (int64_t)oc * d + kc);
  }
  float xv[32];  // xv[4 i + e] = x[16 i + 4 h + e]
  if (a.x_vec && a.x_bf16) {
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(a.x) + vec * a.x_stride;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 16 * i + 4 * h, kc = k < d ? k : d - 4;
      const uint2 v = *reinterpret_cast<const uint2*>(xp + kc);
      xv[4 * i] = __uint_as_float(v.x << 16);
      xv[4 * i + 1] = __uint_as_float(v.x & 0xFFFF0000u);
      xv[4 * i + 2] = __uint_as_float(v.y << 16);
      xv[4 * i + 3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
  } else if (a.x_vec) {
    const float* xp = reinterpret_cast<const float*>(a.x) + vec * a.x_stride;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 16 * i + 4 * h, kc = k < d ? k : d - 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(xp + kc);
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[4 * i + e] = v[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int k = 16 * (i / 4) + 4 * h + i % 4, kc = k < d ? k : d - 1;
      xv[i] = a.x_bf16 ? __uint_as_float((uint32_t) reinterpret_cast<const uint16_t*>(a.x)[vec * a.x_stride + kc]
                                         << 16)
                       : reinterpret_cast<const float*>(a.x)[vec * a.x_stride + kc];
    }
  }
  // The group of this wave's 16 coordinates (group boundaries are multiples
  // of 16) and its parameters, chosen by selects rather than indexed reads of
  // the argument block, and the destination row (a row index list is read
  // through an always-valid address): every scalar argument is fetched here,
  // in one round trip, instead of at its first use further down.
  const int grp = (a.n_groups > 1 && 16 * w >= a.choff[1]) ? 1 : 0;
  int mg = grp ? a.gbits[1] : a.gbits[0];
  int choff = grp ? a.choff[1] : a.choff[0];
  int gdim = grp ? a.gdim[1] : a.gdim[0];
  int coff = grp ? a.coff[1] : a.coff[0];
  int boff = grp ? a.boff[1] : a.boff[0];
  int code_pos = tok ? 32 * (grp ? a.cwoff[1] : a.cwoff[0]) : 32 * (grp ? a.bcwoff[1] : a.bcwoff[0]);
  int sign_pos = tok ? 32 * (a.code_words + (grp ? a.swoff[1] : a.swoff[0]))
                     : 32 * (a.blk_code_words + (grp ? a.bswoff[1] : a.bswoff[0]));
  int n_words = tok ? a.code_words + a.sign_words : a.blk_code_words + a.blk_sign_words;
  int n_groups = a.n_groups, cw = a.code_words, sw = a.sign_words, bcw = a.blk_code_words,
      bsw = a.blk_sign_words;
  int c0 = a.choff[0], c1 = a.choff[1], g0 = a.gdim[0], g1 = a.gdim[1];
  int64_t seg_len = a.seg_len, seg_stride = a.seg_stride, seg_offset = a.seg_offset, n_rows = a.n_rows;
  uint32_t* codes = a.codes;
  uint32_t* signs = a.signs;
  float* norms = a.norms;
  const int64_t* dst_rows = a.dst_rows;
  int64_t row_listed = *(dst_rows ? dst_rows + vec : reinterpret_cast<const int64_t*>(a.rot));
  // (opaque to the compiler from here on, so it keeps them in registers
  // rather than reading the argument block again at each use)
  asm volatile("" : "+s"(mg), "+s"(choff), "+s"(gdim), "+s"(coff), "+s"(boff), "+s"(code_pos), "+s"(sign_pos),
               "+s"(n_words), "+s"(n_groups), "+s"(cw), "+s"(sw), "+s"(bcw), "+s"(bsw));
  asm volatile("" : "+s"(c0), "+s"(c1), "+s"(g0), "+s"(g1), "+s"(seg_len), "+s"(seg_stride), "+s"(seg_offset),
               "+s"(n_rows), "+s"(codes), "+s"(signs), "+s"(norms), "+s"(dst_rows));
  const int nb = (1 << mg) - 1;
  const int kc = (lane & 15) < nb ? (lane & 15) : nb - 1;
  const float bnd_l = a.boundaries[boff + kc];
  const float cen_l = a.centroids[coff + kc + ((lane & 15) == nb ? 1 : 0)];
  for (int e = tid; e < n_words; e += NTHR) {
    s_bits[e] = 0u;
    s_mask[e] = 0u;
  }
  const bool live = o < d;
  if (d < 128) {  // (uniform) entries past d were loaded from clamped indices
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = live && 16 * i + 4 * h < d;
      if (!ok) {
        rq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        sq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (16 * (i / 4) + 4 * h + i % 4 >= d) xv[i] = 0.f;
  }

  // ---- y_o = rot[o] . x: four FMA chains, then the lane quad ----
  float y;
  {
    float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) c4[j] = fmaf(rq[i][j], xv[4 * i + j], c4[j]);
    y = (c4[0] + c4[1]) + (c4[2] + c4[3]);
    y += dpp_f<0xB1>(y);
    y += dpp_f<0x4E>(y);
  }
  {
    const float t = wave_sum(h == 0 ? y * y : 0.f);
    if (lane == 0) s_np[w] = t;
  }
  __syncthreads();

  // ---- group norm, cell, residual (rotated domain), code field ----
  // (the destination row is formed here, off the path of the loads; a row
  // outside the cache, the same for the whole workgroup, stores nothing)
  // (vec < kSmallMaxVec here, so a segment length clamped to kSmallMaxVec
  // gives the same quotient and remainder in 32-bit arithmetic)
  const int seg = seg_len < kSmallMaxVec ? (int)seg_len : kSmallMaxVec;
  const int64_t row = dst_rows ? row_listed : (int64_t)((int)vec / seg) * seg_stride + seg_offset + (int)vec % seg;
  const bool row_ok = row >= 0 && row < n_rows;
  const int w0 = choff / 16, w1 = (choff + gdim + 15) / 16;
  const float nv = sqrtf(wave_range_sum(s_np, w0, w1));
  int idx;
  {
    const float u = y * __builtin_amdgcn_rcpf(nv);
    int c = 0;
#pragma unroll
    for (int k = 0; k < 15; ++k) {
      const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bnd_l), k));
      c += (k < nb && u > b) ? 1 : 0;
    }
    idx = nv > 0.f ? c : (nb + 1) / 2 - 1;
  }
  const float cv = __shfl(cen_l, idx, 64);  // centroid idx (lanes 0 .. 15 hold them)
  float rr = nv > 0.f ? fmaf(-nv, cv, y) : 0.f;
  if (!live) {
    rr = 0.f;
    idx = 0;
  }
  if (h == 0) s_r[o] = rr;
  {
    const float t = wave_sum(h == 0 ? rr * rr : 0.f);
    if (lane == 0) s_gp[w] = t;
  }
  const int j = o - choff;  // channel within the group
  const int slot = (int)(row & 31), quarter = slot >> 3, sl = slot & 7;
  if (h == 0 && live && row_ok) {
    const int pos = tok ? code_pos + mg * j : code_pos + 8 * mg * (quarter * gdim + j) + mg * sl;
    or_field(s_bits, s_mask, pos, (uint32_t)idx, mg);
  }
  __syncthreads();

  // ---- s_o = sketch_rot[o] . r; sign bit = [s >= 0] (not for MSE-only records) ----
  if (!a.mse_only) {
    float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 r4 = *reinterpret_cast<const f32x4*>(s_r + 16 * i + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) c4[e] = fmaf(sq[i][e], r4[e], c4[e]);
    }
    float sv = (c4[0] + c4[1]) + (c4[2] + c4[3]);
    sv += dpp_f<0xB1>(sv);
    sv += dpp_f<0x4E>(sv);
    if (h == 0 && live && row_ok) {
      const int pos = tok ? sign_pos + j : sign_pos + 8 * (quarter * gdim + j) + sl;
      or_field(s_bits, s_mask, pos, sv >= 0.f ? 1u : 0u, 1);
    }
  }
  __syncthreads();

  // ---- store: norms (n_g, gamma_g), then the record words ----
  if (!row_ok) return;
  if (tid < n_groups) {
    const int g = tid;
    const int cg = g ? c1 : c0, dg = g ? g1 : g0;
    const int v0 = cg / 16, v1 = (cg + dg + 15) / 16;
    const float nv = sqrtf(wave_range_sum(s_np, v0, v1));
    store_norms(norms, a.norm_f16, row * n_groups + g, nv, sqrtf(wave_range_sum(s_gp, v0, v1)));
  }
  if (tok) {
    for (int e = tid; e < n_words; e += NTHR) {
      if (e < cw)
        codes[row * cw + e] = s_bits[e];
      else
        signs[row * sw + e - cw] = s_bits[e];
    }
  } else {
    const int64_t blk = row >> 5;
    for (int e = tid; e < n_words; e += NTHR) {
      const uint32_t m = s_mask[e];
      if (m == 0u) continue;
      uint32_t* dst = e < bcw ? codes + blk * bcw + e : signs + blk * bsw + (e - bcw);
      atomicAnd(dst, ~m);
      atomicOr(dst, s_bits[e] & m);
    }
  }
}

// Validates the arguments of one quantize call and fills its kernel
// arguments. Returns TQ_OK with *empty = true for n_vec == 0.
inline tq_status make_qargs(const tq_quantizer* qz, tq_format fmt, const void* x, tq_dtype x_dtype,
                            int64_t n_vec, int64_t x_row_stride, const tq_rows* rows,
                            const tq_cache* cache, QArgs* out, bool* empty) {
  *empty = false;
  if (!tq::quantizer_pointers_valid(qz) || !rows || !cache) return TQ_ERR_INVALID;
  if (fmt != TQ_TOKEN_MAJOR && fmt != TQ_BLOCK32) return TQ_ERR_INVALID;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_INVALID;
  const tq_layout& l = qz->layout;
  if (n_vec < 0 || x_row_stride < l.d) return TQ_ERR_INVALID;
  // (MSE-only records have no sign words: their sign pointer is not read and may be null)
  if (!cache->codes || (!cache->signs && !l.mse_only) || !cache->norms || cache->n_rows < 0) return TQ_ERR_INVALID;
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
  if (n_vec == 0) {
    *empty = true;
    return TQ_OK;
  }
  if (!x || reinterpret_cast<uintptr_t>(x) % 4 != 0) return TQ_ERR_INVALID;

  QArgs& a = *out;
  a = QArgs{};
  a.x = x;
  a.n_vec = n_vec;
  a.x_stride = x_row_stride;
  a.x_bf16 = x_dtype == TQ_BF16;
  {
    const int64_t esz = a.x_bf16 ? 2 : 4, per = 16 / esz;
    a.x_vec = reinterpret_cast<uintptr_t>(x) % 16 == 0 && (x_row_stride * esz) % 16 == 0 && l.d % per == 0;
  }
  a.rot = qz->rot;
  a.skr = qz->sketch_rot;
  a.m_vec = l.d % 4 == 0 && reinterpret_cast<uintptr_t>(qz->rot) % 16 == 0 &&
            reinterpret_cast<uintptr_t>(qz->sketch_rot) % 16 == 0;
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
  a.mse_only = l.mse_only;
  a.norm_f16 = l.norm_f16;
  a.blk_code_words = geo.info.block_code_words;
  a.blk_sign_words = geo.info.block_sign_words;
  a.fmt = fmt;
  a.dst_rows = rows->dst_rows;
  a.seg_len = rows->seg_len < 1 ? 1 : rows->seg_len;
  a.seg_stride = rows->seg_stride;
  a.seg_offset = rows->seg_offset;
  a.n_rows = cache->n_rows;
  a.pk_zero = 0;
  for (int g = 0; g < l.n_groups; ++g) {
    const int waves = (geo.dim[g] + 15) / 16;
    if ((waves * geo.bits[g]) % 2 != 0 || waves % 2 != 0) a.pk_zero = 1;
  }
  a.blk_owned = fmt == TQ_BLOCK32 && !rows->dst_rows &&
                (n_vec <= rows->seg_len || rows->seg_stride % 32 == 0);
  if (a.blk_owned) {
    const int64_t n_seg = (n_vec + a.seg_len - 1) / a.seg_len;
    a.pairs_per_seg = (a.seg_offset % 32 + a.seg_len + 63) / 64;
    a.n_tiles = n_seg * a.pairs_per_seg;
  } else {
    a.pairs_per_seg = 1;
    a.n_tiles = (n_vec + QT - 1) / QT;
  }
  a.codes = cache->codes;
  a.signs = cache->signs;
  a.norms = cache->norms;
  return TQ_OK;
}

// Whether a call (already validated by make_qargs) can take the
// half-precision MFMA variant of the tile path: bf16 rows read as 16-byte
// chunks (so d is a multiple of 8), 16-byte aligned matrices, d <= 128.
inline bool h_path_ok(const QArgs& a) {
  return a.x_bf16 && a.x_vec && a.m_vec && a.d % 8 == 0 && a.d <= 128;
}

// Kernel shape for a dimension: KP = d rounded up to 16, NT = KP / 16 waves.
inline int quantize_kp(int d) {
  const int dpad = (d + 15) / 16;
  return dpad <= 4 ? 64 : dpad <= 8 ? 128 : dpad <= 13 ? 208 : 256;
}

}  // namespace tqq
