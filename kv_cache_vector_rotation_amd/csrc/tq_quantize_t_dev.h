// Transposed tile path of the quantize kernel: bf16 inputs, d <= 128.
//
// [ZB] paragraph 2 and [WD] "Como o TurboQuant funciona": rotate each vector,
// give every rotated coordinate its Lloyd-Max cell, take the residual of that
// MSE quantizer, keep the signs of a Gaussian sketch of the residual, store
// codes, sign bits and the norms. The values this path produces follow the
// same rules as the general tile path; only the work layout differs.
//
// Both products are formed as (matrix slice) x (tile)^T: a wave's 16 rows of
// the d x d matrix are the A operand of v_mfma_f32_16x16x32_{bf16,f16} (held
// in registers for the whole kernel) and 16 vectors of the tile in LDS are
// the B operand. The result lane (ln, lg) of 16-vector tile mt then holds
// coordinates 16 w + 4 lg + i (i = 0 .. 3) of the single vector 16 mt + ln,
// so every per-vector quantity (norm, its reciprocal, the residual scale) is
// one value per lane, sums over a wave's 16 coordinates take one in-lane sum
// and two lane swaps, and the four codes, residual values and sign bits of a
// lane are adjacent in every output layout (8-byte LDS stores of the
// residual parts, packed code and sign fields).
//
// Precision is that of the general path's half-precision variant:
//  - y = rot x: x is exact in bf16 and rot = RH + RM + RL (three bf16 parts
//    within 2^-27 of rot), so the products are exact term by term and only
//    the fp32 accumulation rounds.
//  - s = sketch_rot r: only the sign of s is kept, and it does not change when
//    a row of sketch_rot or the residual of one (vector, group) is scaled by a
//    power of two: rows are scaled so their largest entry lies in
//    [2^13, 2^14), residuals so their group norm lies in [2^9, 2^10)
//    (|r_k| < 2 n_g, so every scaled value fits fp16), both are split into
//    fp16 high and low parts, and AL BH + AH BL + AH BH leaves out AL BL,
//    below 2^-22 of each term.
//
// Tiles: token-major records take 64 consecutive vectors; block records
// take one aligned pair of 32-row blocks of one segment (block-owned tiling)
// with tile row = slot in the pair, so the 8 tokens of an octet field sit in
// 8 adjacent lanes. The next tile's input is loaded while the current one is
// processed.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_quantize_dev.h"

namespace tqq {

template <int KP, int NT>
struct LdsT {
  static constexpr int XH = KP + 8;  // row stride (16-bit units) of the bf16 tile and the residual parts
  static constexpr int off_x = 0;                             // u16 [QT][XH]: bf16 tile, then the residual's high part
  static constexpr int off_rl = off_x + QT * XH * 2;          // u16 [QT][XH]: the residual's low part
  static constexpr int off_npart = off_rl + QT * XH * 2;      // float [NT][QT]: sums of y^2 per wave
  static constexpr int off_gpart = off_npart + NT * QT * 4;   // float [NT][QT]: sums of r^2 per wave
  static constexpr int off_nrm = off_gpart + NT * QT * 4;     // float [2][QT]: group norms n_g
  static constexpr int off_cb = off_nrm + 2 * QT * 4;         // float [64]: centroids [0, 32), boundaries [32, 64)
  static constexpr int off_rows = off_cb + 64 * 4;            // int64 [QT]: destination rows (token-major)
  static constexpr int PKW = (KP * 4 / 32 + KP / 32 + 4 + 3) / 4 * 4;  // token-major staging row, words (16-byte rows)
  static constexpr int BKW = KP * 5;                          // block staging: code + sign words of one block
  static constexpr int off_pk = off_rows + QT * 8;            // u32: token-major [QT][PKW]; block [2][BKW] + masks [2][BKW]
  static constexpr int PK_WORDS = QT * PKW > 4 * BKW ? QT * PKW : 4 * BKW;
  static constexpr int bytes = off_pk + PK_WORDS * 4;
};

// Whether a call (validated by make_qargs) takes the transposed tile path.
inline bool t_path_ok(const QArgs& a) {
  return h_path_ok(a) && (a.fmt == TQ_TOKEN_MAJOR || a.blk_owned);
}

// Reduce-scatter over the four lane groups: given one value per 16-vector
// tile mt, lane group lg returns the sum (OR) over the four lane groups of
// the value of tile lg. The 32-lane swap pairs tiles (0, 2) and (1, 3), the
// 16-lane swap then pairs the two partial results.
__device__ __forceinline__ float lg_sum4(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
__device__ __forceinline__ uint32_t lg_or4(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0] | a[1], b[0] | b[1], false, false);
  return c[0] | c[1];
}

// All-gather over the four lane groups: out[mt] = the value of lane
// (ln, mt). The 16-lane swap gives every row the values of its row pair, the
// 32-lane swaps of those give rows 0 and 2, then rows 1 and 3.
__device__ __forceinline__ void lg_gather4(float v, float (&out)[4]) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto e = __builtin_amdgcn_permlane32_swap(p[0], p[0], false, false);
  const auto o = __builtin_amdgcn_permlane32_swap(p[1], p[1], false, false);
  out[0] = __uint_as_float(e[0]);
  out[1] = __uint_as_float(o[0]);
  out[2] = __uint_as_float(e[1]);
  out[3] = __uint_as_float(o[1]);
}

// OR over each aligned group of 8 lanes, the result in all 8.
__device__ __forceinline__ uint32_t oct_or(uint32_t s) {
  s |= dpp_u<0xB1>(s);   // quad_perm [1, 0, 3, 2]
  s |= dpp_u<0x4E>(s);   // quad_perm [2, 3, 0, 1]
  s |= dpp_u<0x141>(s);  // row_half_mirror
  return s;
}

// acc[mt] = (B = RH + RM + RL slice) x (tile rows 16 mt .. 16 mt + 15)^T for
// the first NMT 16-vector tiles (the rest zero): the matrix parts are the A
// operand, the bf16 tile (row stride XH) the B operand. Step s of lane group
// lg takes k = 32 s + 8 lg + j, j = 0 .. 7; the small parts go first.
template <int NMT, int KS, int XH>
__device__ __forceinline__ void mfma_t_bf16x3(const uint16_t* xh, const u32x4 (&mh)[KS], const u32x4 (&mm)[KS],
                                              const u32x4 (&ml)[KS], int ln, int lg, f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 b[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      b[mt] = *reinterpret_cast<const u32x4*>(xh + (mt * 16 + ln) * XH + 32 * s + 8 * lg);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(ml[s], b[mt], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(mm[s], b[mt], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_bf16(mh[s], b[mt], acc[mt]);
  }
}

// The same with two fp16 parts on both sides: (SL RH^T) + (SH RL^T) + (SH RH^T).
template <int NMT, int KS, int XH>
__device__ __forceinline__ void mfma_t_f16x2(const uint16_t* rh, const uint16_t* rl, const u32x4 (&sh)[KS],
                                             const u32x4 (&sl)[KS], int ln, int lg, f32x4 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 bh[NMT], bl[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int off = (mt * 16 + ln) * XH + 32 * s + 8 * lg;
      bh[mt] = *reinterpret_cast<const u32x4*>(rh + off);
      bl[mt] = *reinterpret_cast<const u32x4*>(rl + off);
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(sl[s], bh[mt], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(sh[s], bl[mt], acc[mt]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma_f16(sh[s], bh[mt], acc[mt]);
  }
}

// Cells of four unit coordinates: the number of the NB boundaries below each,
// plus corr. b_k - u has its sign bit set exactly when u > b_k (a difference
// of zero is +0 unless b_k = -0 and u = +0, a tie that either cell may take),
// so the count is a sum of sign bits (no lane masks).
template <int NB>
__device__ __forceinline__ void cells4(const float (&u)[4], const float (&tb)[15], int corr, int (&c)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t n = (uint32_t)corr;
#pragma unroll
    for (int k = 0; k < NB; ++k) n += __float_as_uint(tb[k] - u[i]) >> 31;
    c[i] = (int)n;
  }
}

// The tile's bf16 input, two 16-byte chunks per thread, held in registers
// from the load to the LDS store (one tile ahead).
struct TStage {
  u32x4 c[2];
};

// Chunk i of thread tid: tile row v = c / (KP / 8), columns k .. k + 7. A
// block tile's row is the slot in its block pair: slot t holds vector
// v0 + t - slot_lo when that lies in [0, nvalid), else zeros.
template <int KP, int NT>
__device__ __forceinline__ void load_t(const QArgs& a, const TileGeo& g, bool blk, int tid, TStage& st) {
  constexpr int CPR = KP / 8;
  static_assert(QT * CPR == 2 * NT * 64, "two chunks per thread");
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
    const int src = blk ? v - g.slot_lo : v;
    st.c[i] = (src >= 0 && src < g.nvalid && k < a.d)
                  ? *reinterpret_cast<const u32x4*>(x + (g.v0 + src) * a.x_stride + k)
                  : u32x4{0u, 0u, 0u, 0u};
  }
}

// The octet-field words of a lane's four channels: code idx[i] of channel i
// (token s of the octet) at bit 8 MG i + MG s of an MG-word string. The word
// of each channel is a constant; MG = 3 fields may straddle two words.
template <int MG>
__device__ __forceinline__ void octet_words(const int (&idx)[4], int s, uint32_t (&wv)[4]) {
  wv[0] = wv[1] = wv[2] = wv[3] = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bit0 = 8 * MG * i;  // (a constant once unrolled)
    const int wi = bit0 >> 5;
    const uint64_t f = (uint64_t)(uint32_t)idx[i] << ((bit0 & 31) + MG * s);
    wv[wi] |= (uint32_t)f;
    if (wi + 1 < MG) wv[wi + 1] |= (uint32_t)(f >> 32);
  }
}
template <int MG>
__device__ __forceinline__ void octet_or_words(const int (&idx)[4], int s, uint32_t (&wv)[4]) {
  octet_words<MG>(idx, s, wv);
#pragma unroll
  for (int q = 0; q < MG; ++q) wv[q] = oct_or(wv[q]);
}


// This wave's rows of rot (three bf16 parts) and sketch_rot (row-scaled,
// two fp16 parts), lane (ln, lg) holding M[16 w + ln][32 s + 8 lg + j]
// (rows and columns past d are zero).
template <int KS>
__device__ __forceinline__ void t_matrix_regs(const QArgs& a, int w, int ln, int lg, u32x4 (&rh)[KS], u32x4 (&rm)[KS],
                                              u32x4 (&rl3)[KS], u32x4 (&sh)[KS], u32x4 (&sl)[KS]) {
  const int d = a.d;
  const int orow = 16 * w + ln;
  const bool row_ok = orow < d;
  const int64_t rb = (int64_t)(row_ok ? orow : d - 1) * d;
  f32x4 mr[KS][2], ms[KS][2];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      // (d is a multiple of 8: a lane's 8 entries are all inside the row or all past it)
      const int k = 32 * s2 + 8 * lg + 4 * hlf;
      const int kc = k < d ? k : 0;
      mr[s2][hlf] = *reinterpret_cast<const f32x4*>(a.rot + rb + kc);
      ms[s2][hlf] = *reinterpret_cast<const f32x4*>(a.skr + rb + kc);
      if (!row_ok || 32 * s2 + 8 * lg >= d) {
        mr[s2][hlf] = f32x4{0.f, 0.f, 0.f, 0.f};
        ms[s2][hlf] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
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
    rl3[s2] = u32x4{wl[0], wl[1], wl[2], wl[3]};
    sh[s2] = u32x4{vh[0], vh[1], vh[2], vh[3]};
    sl[s2] = u32x4{vl[0], vl[1], vl[2], vl[3]};
  }
}

// Destination row of vector tid (< QT) of a token-major tile (-1: past the
// tile or outside the cache), stored to rows[tid].
__device__ __forceinline__ void t_tile_rows(const QArgs& a, const TileGeo& cg, int tid, int64_t* rows) {
  // destination rows: vector v0 + t of the call (segments of seg_len rows)
  int64_t row = -1;
  if (tid < cg.nvalid) {
    if (a.dst_rows) {
      row = a.dst_rows[cg.v0 + tid];
    } else {
      const int64_t q0 = cg.v0 / a.seg_len, r0 = cg.v0 - q0 * a.seg_len;  // (uniform)
      int64_t q = q0, r = r0 + tid;
      if (a.seg_len >= QT) {
        if (r >= a.seg_len) {
          q += 1;
          r -= a.seg_len;
        }
      } else {
        const uint32_t sl = (uint32_t)a.seg_len, rr32 = (uint32_t)r, dq = rr32 / sl;
        q += dq;
        r = rr32 - dq * sl;
      }
      row = q * a.seg_stride + a.seg_offset + r;
    }
    if (row < 0 || row >= a.n_rows) row = -1;
  }
  rows[tid] = row;
}

// Store phase of a tile: the norms of its vectors (n_g staged in nrmv
// [group][QT], gamma_g from the per-wave residual sums gpart [wave][QT]),
// then the staged records pk (token-major rows of PKW words at the
// destination rows `rows`; block records: the two blocks' words, with
// per-word masks for partial blocks).
template <int KP, int NT, bool BLK>
__device__ __forceinline__ void t_store_tile(const QArgs& a, const TileGeo& cg, const int64_t* rows,
                                             const float* nrmv, const float* gpart, const uint32_t* pk,
                                             bool partial, bool vec_out, int tid) {
  using L = LdsT<KP, NT>;
  constexpr int PKW = L::PKW;
  constexpr int BKW = L::BKW;
  constexpr bool tok = !BLK;
  const int bcw = a.blk_code_words, bsw = a.blk_sign_words;
  const bool signs_on = !a.mse_only;
  if (tid < QT * a.n_groups) {
    const int gg = tid / QT, v = tid % QT;
    int64_t row = -1;
    if (tok)
      row = rows[v];
    else if (v >= cg.slot_lo && v < cg.slot_lo + cg.nvalid)
      row = cg.rowbase + v;
    if (row >= 0) {
      const int w0 = a.choff[gg] / 16, w1 = (a.choff[gg] + a.gdim[gg] + 15) / 16;
      float s = 0.f;
      for (int ww = w0; ww < w1; ++ww) s += gpart[ww * QT + v];
      store_norms(a.norms, a.norm_f16, row * a.n_groups + gg, nrmv[gg * QT + v], sqrtf(s));
    }
  }
  if (tok) {
    const int cw = a.code_words, sw = a.sign_words;
    if (vec_out) {
      // 8 threads per row: 16-byte chunks, the row's code chunks then its sign chunks
      const int v = tid >> 3, c = tid & 7, cc = cw / 4, sc4 = sw / 4;
      for (int vv = v; vv < cg.nvalid; vv += NT * 8) {
        const int64_t row = rows[vv];
        if (row < 0 || c >= cc + sc4) continue;
        const u32x4 val = *reinterpret_cast<const u32x4*>(pk + vv * PKW + 4 * c);
        if (c < cc)
          *reinterpret_cast<u32x4*>(a.codes + row * cw + 4 * c) = val;
        else
          *reinterpret_cast<u32x4*>(a.signs + row * sw + 4 * (c - cc)) = val;
      }
    } else {
      // 16 threads per row, word by word
      const int rw = cw + sw;
      for (int v = tid >> 4; v < cg.nvalid; v += NT * 4) {
        const int64_t row = rows[v];
        if (row < 0) continue;
        for (int wd = tid & 15; wd < rw; wd += 16) {
          const uint32_t val = pk[v * PKW + wd];
          if (wd < cw)
            a.codes[row * cw + wd] = val;
          else
            a.signs[row * sw + wd - cw] = val;
        }
      }
    }
  } else {
    const int nw = bcw + (signs_on ? bsw : 0);
    if (!partial && vec_out) {
      // both blocks whole: 16-byte chunks
      const int nc = nw / 4;
      for (int e = tid; e < 2 * nc; e += NT * 64) {
        const int h = e >= nc ? 1 : 0, c = e - h * nc;
        const int64_t blkrow = cg.rowbase / 32 + h;
        const u32x4 val = *reinterpret_cast<const u32x4*>(pk + h * BKW + 4 * c);
        uint32_t* dst = 4 * c < bcw ? a.codes + blkrow * bcw + 4 * c : a.signs + blkrow * bsw + (4 * c - bcw);
        *reinterpret_cast<u32x4*>(dst) = val;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int vlo = cg.slot_lo > 32 * h ? cg.slot_lo : 32 * h;
        const int vhi = cg.slot_lo + cg.nvalid < 32 * h + 32 ? cg.slot_lo + cg.nvalid : 32 * h + 32;
        if (vhi <= vlo) continue;
        const int64_t blkrow = cg.rowbase / 32 + h;
        for (int wd = tid; wd < nw; wd += NT * 64) {
          const uint32_t val = pk[h * BKW + wd];
          uint32_t* dst = wd < bcw ? a.codes + blkrow * bcw + wd : a.signs + blkrow * bsw + (wd - bcw);
          const uint32_t m = partial ? pk[(2 + h) * BKW + wd] : 0xFFFFFFFFu;
          if (m == 0xFFFFFFFFu) {
            *dst = val;
          } else if (m != 0u) {
            atomicAnd(dst, ~m);
            atomicOr(dst, val & m);
          }
        }
      }
    }
  }
}

// The kernel body: this workgroup quantizes tiles first_tile,
// first_tile + tile_stride, ... of `a` (t_path_ok), with NT * 64 threads and
// the dynamic LDS block `smem` (LdsT<KP, NT>::bytes).
template <int KP, int NT, bool BLK>
__device__ __forceinline__ void quantize_tiles_t_fmt(const QArgs& a, int64_t first_tile, int64_t tile_stride,
                                                     unsigned char* smem) {
  using L = LdsT<KP, NT>;
  constexpr int XH = L::XH;
  constexpr int KS = KP / 32;
  constexpr int PKW = L::PKW;
  constexpr int BKW = L::BKW;
  static_assert(KP == NT * 16 && KP % 32 == 0 && KP <= 128, "tile shape");
  uint16_t* xh = reinterpret_cast<uint16_t*>(smem + L::off_x);
  uint16_t* rlo = reinterpret_cast<uint16_t*>(smem + L::off_rl);
  float* npart = reinterpret_cast<float*>(smem + L::off_npart);
  float* gpart = reinterpret_cast<float*>(smem + L::off_gpart);
  float* nrmv = reinterpret_cast<float*>(smem + L::off_nrm);
  float* cbk = reinterpret_cast<float*>(smem + L::off_cb);
  int64_t* rows = reinterpret_cast<int64_t*>(smem + L::off_rows);
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem + L::off_pk);
  uint16_t* pk16 = reinterpret_cast<uint16_t*>(smem + L::off_pk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave = 16 output coordinates
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int d = a.d;
  constexpr bool blk = BLK;  // block records (then blk_owned), else token-major

  float cent_reg = 0.f, bnd_reg = 0.f;
  {
    const int ncent = (1 << a.gbits[0]) + (a.n_groups > 1 ? (1 << a.gbits[1]) : 0);
    cent_reg = a.centroids[tid < ncent ? tid : ncent - 1];
    const int nbt = ((1 << a.gbits[0]) - 1) + (a.n_groups > 1 ? (1 << a.gbits[1]) - 1 : 0);
    bnd_reg = a.boundaries[tid < nbt ? tid : nbt - 1];
  }
  TileGeo g;
  int64_t tile = next_live_tile(a, first_tile, tile_stride, g);
  TStage st;
  if (tile < a.n_tiles) load_t<KP, NT>(a, g, blk, tid, st);

  // this wave's matrix rows
  u32x4 rh[KS], rm[KS], rl3[KS], sh[KS], sl[KS];
  t_matrix_regs<KS>(a, w, ln, lg, rh, rm, rl3, sh, sl);

  // wave-uniform group parameters (group boundaries are multiples of 16)
  const int grp = (a.n_groups > 1 && w * 16 >= a.choff[1]) ? 1 : 0;
  const int mg = a.gbits[grp];
  const int nb = (1 << mg) - 1;
  const int coff = a.coff[grp];
  const int boff = a.boff[grp];
  const int choff = a.choff[grp];
  const int dg = a.gdim[grp];
  const int wig = w - choff / 16;          // wave index within its group
  const int gw0 = choff / 16, gw1 = (choff + dg + 15) / 16;  // the group's waves
  const int j0 = 16 * wig + 4 * lg;        // the lane's first channel within the group
  const bool lane_ok = 16 * w + 4 * lg < d;  // the lane's four coordinates exist (d % 4 == 0)
  const bool tail = 16 * w + 16 > d;       // (uniform) the wave has coordinates past d
  const int mid = (nb + 1) / 2 - 1;        // the cell of a zero vector
  constexpr bool tok = !BLK;
  const int pk_code_h = 2 * a.cwoff[grp] + mg * wig;
  const int pk_sign_h = 2 * (a.code_words + a.swoff[grp]) + wig;
  const int bcw = a.blk_code_words, bsw = a.blk_sign_words;
  const int bc_g = a.bcwoff[grp], bs_g = bcw + a.bswoff[grp];  // block staging offsets of the group
  const bool signs_on = !a.mse_only;

  // the codebook, once (the tile loop only reads it); boundaries of this
  // wave's group in registers
  if (tid < 32) {
    cbk[tid] = cent_reg;
    cbk[32 + tid] = bnd_reg;
  }
  __syncthreads();
  float tb[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) tb[k] = k < nb ? cbk[32 + boff + k] : INFINITY;
  // A zero vector (n = 0, so u = 0) takes the middle cell: its count of
  // boundaries below 0, zc, is corrected by mid - zc.
  int zc = 0;
#pragma unroll
  for (int k = 0; k < 15; ++k) zc += k < nb ? (int)(__float_as_uint(tb[k] - 0.0f) >> 31) : 0;
  const int zcorr = mid - zc;
  // 16-byte record stores: every record row and block a multiple of 16 bytes
  // on 16-byte aligned arrays
  const bool vec_out = ((reinterpret_cast<uintptr_t>(a.codes) | reinterpret_cast<uintptr_t>(a.signs)) % 16 == 0) &&
                       (blk ? (bcw % 4 == 0 && bsw % 4 == 0) : (a.code_words % 4 == 0 && a.sign_words % 4 == 0));

  // Barriers per tile: (1) the input tile is staged; (2) the per-wave sums of
  // y^2 are in; (4) the residual parts and the code fields are in; (5) the
  // sign fields are in. No barrier ends the tile:
  // what the next tile writes before its barrier (1) (the input tile) was last
  // read before (5), and what the store phase reads (destination rows, norms,
  // partial sums, staged records) is next written after the next (1).
  while (tile < a.n_tiles) {
    const TileGeo cg = g;
    {
      constexpr int CPR = KP / 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
        *reinterpret_cast<u32x4*>(xh + v * XH + k) = st.c[i];
      }
    }
    __syncthreads();  // (1)
    // the next tile's input, in flight while this one is processed
    tile = next_live_tile(a, tile + tile_stride, tile_stride, g);
    if (tile < a.n_tiles) load_t<KP, NT>(a, g, blk, tid, st);
    if (tok && a.pk_zero)
      for (int e = tid; e < QT * PKW; e += NT * 64) pk[e] = 0u;
    if (tok && tid < QT) t_tile_rows(a, cg, tid, rows);

    // ---- y = rot x ----
    // (a token-major tile of at most 16 vectors runs its first 16-vector
    // tile only; rows past the tile's vectors are zero)
    const int n_mt = (!blk && cg.nvalid <= 16) ? 1 : 4;
    f32x4 y[4];
    if (n_mt == 1)
      mfma_t_bf16x3<1, KS, XH>(xh, rh, rm, rl3, ln, lg, y);
    else
      mfma_t_bf16x3<4, KS, XH>(xh, rh, rm, rl3, ln, lg, y);
    // lane (ln, lg): y[mt][i] = coordinate 16 w + 4 lg + i of tile row 16 mt + ln
    {
      float sq[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        sq[mt] = fmaf(y[mt][3], y[mt][3], fmaf(y[mt][2], y[mt][2], fmaf(y[mt][1], y[mt][1], y[mt][0] * y[mt][0])));
      // lane l = 16 lg + ln holds the wave's sum for tile row l
      npart[w * QT + lane] = lg_sum4(sq[0], sq[1], sq[2], sq[3]);
    }
    __syncthreads();  // (2)
    // the group norm of tile row l (lane l of every wave: the group's wave
    // sums), its reciprocal and the residual scale, then gathered so that
    // lane (ln, lg) holds those of rows 16 mt + ln, mt = 0 .. 3
    float nv4[4], inv4[4], sc4[4];
    {
      float sum = 0.f;
      for (int ww = gw0; ww < gw1; ++ww) sum += npart[ww * QT + lane];
      const float n = sqrtf(sum);
      const float inv = n > 0.f ? __builtin_amdgcn_rcpf(n) : 0.f;
      const float sc = n > 0.f ? __builtin_amdgcn_ldexpf(1.0f, 10 - __builtin_amdgcn_frexp_expf(n)) : 1.0f;
      if (wig == 0) nrmv[grp * QT + lane] = n;  // for the norm stores
      lg_gather4(n, nv4);
      lg_gather4(inv, inv4);
      lg_gather4(sc, sc4);
    }

    // ---- cells, residual, residual norm partials, packed codes ----
    int idx[4][4];
    {
      float gq[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float nq[3] = {nv4[mt], inv4[mt], sc4[mt]};
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = y[mt][i] * nq[1];
        const int corr = nq[0] > 0.f ? 0 : zcorr;
        int c[4];
        if (nb == 3)
          cells4<3>(u, tb, corr, c);
        else if (nb == 7)
          cells4<7>(u, tb, corr, c);
        else if (nb == 1)
          cells4<1>(u, tb, corr, c);
        else
          cells4<15>(u, tb, corr, c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          idx[mt][i] = c[i];
          if (tail && !lane_ok) idx[mt][i] = 0;
        }
        float cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[i] = cbk[coff + idx[mt][i]];
        float rr[4];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rr[i] = fmaf(-nq[0], cv[i], y[mt][i]);
          if (tail && !lane_ok) rr[i] = 0.f;
          s = fmaf(rr[i], rr[i], s);
        }
        gq[mt] = s;
        // the residual, scaled by a power of two, as fp16 high and low parts
        // (the B operand of the sketch product; the rotation read the tile
        // before barrier (2))
        if (signs_on) {
          f16x2 hv[2], lv[2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const _Float16 h = (_Float16)(rr[i] * nq[2]);
            hv[i / 2][i % 2] = h;
            lv[i / 2][i % 2] = (_Float16)fmaf(rr[i], nq[2], -(float)h);
          }
          const int off = (16 * mt + ln) * XH + 16 * w + 4 * lg;
          *reinterpret_cast<uint2*>(xh + off) =
              uint2{__builtin_bit_cast(uint32_t, hv[0]), __builtin_bit_cast(uint32_t, hv[1])};
          *reinterpret_cast<uint2*>(rlo + off) =
              uint2{__builtin_bit_cast(uint32_t, lv[0]), __builtin_bit_cast(uint32_t, lv[1])};
        }
      }
      gpart[w * QT + lane] = lg_sum4(gq[0], gq[1], gq[2], gq[3]);
    }
    if (tok) {
      // the wave's 16 codes of a row (16 mg bits), assembled across the lane
      // groups: lane l stores the mg halfwords of tile row l
      uint32_t flo[4], fhi[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t f4 = (uint32_t)idx[mt][0] | ((uint32_t)idx[mt][1] << mg) | ((uint32_t)idx[mt][2] << (2 * mg)) |
                            ((uint32_t)idx[mt][3] << (3 * mg));
        const uint64_t f = (uint64_t)f4 << (4 * mg * lg);
        flo[mt] = (uint32_t)f;
        fhi[mt] = (uint32_t)(f >> 32);
      }
      const uint32_t lo = lg_or4(flo[0], flo[1], flo[2], flo[3]);
      const uint32_t hi = mg > 2 ? lg_or4(fhi[0], fhi[1], fhi[2], fhi[3]) : 0u;
      uint16_t* row = pk16 + lane * 2 * PKW + pk_code_h;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < mg) row[k] = (uint16_t)((k < 2 ? lo : hi) >> (16 * (k & 1)));
    } else {
      // octet fields: channel j0 + i of the 8 tokens of octet o at bits
      // 8 mg (o dg + j0 + i) + mg s; the 8 lanes of an octet OR their fields
      // (lane moves outside any branch), lane s = 0 stores the mg words
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
        uint32_t wv[4];
        if (mg == 2)
          octet_or_words<2>(idx[mt], s, wv);
        else if (mg == 3)
          octet_or_words<3>(idx[mt], s, wv);
        else if (mg == 1)
          octet_or_words<1>(idx[mt], s, wv);
        else
          octet_or_words<4>(idx[mt], s, wv);
        if (s == 0 && lane_ok) {
          uint32_t* dst = pk + h * BKW + bc_g + mg * (o * dg + j0) / 4;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < mg) dst[q] = wv[q];
        }
      }
    }
    __syncthreads();  // (4)

    // ---- s = sketch_rot r; sign bit = [s >= 0] ----
    if (signs_on) {
      f32x4 sacc[4];
      if (n_mt == 1)
        mfma_t_f16x2<1, KS, XH>(xh, rlo, sh, sl, ln, lg, sacc);
      else
        mfma_t_f16x2<4, KS, XH>(xh, rlo, sh, sl, ln, lg, sacc);
      // sign bit i of a lane: [s >= 0] = NOT the sign bit of s (s = -0 is a
      // tie that either bit may take)
      uint32_t nibs[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uint32_t nib = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) nib |= (~__float_as_uint(sacc[mt][i]) >> 31) << i;
        nibs[mt] = lane_ok ? nib : 0u;
      }
      if (tok) {
        const uint32_t bits16 =
            lg_or4(nibs[0] << (4 * lg), nibs[1] << (4 * lg), nibs[2] << (4 * lg), nibs[3] << (4 * lg));
        pk16[lane * 2 * PKW + pk_sign_h] = (uint16_t)bits16;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t nib = nibs[mt];
        if (!tok) {
          const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
          uint32_t wv = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv |= ((nib >> i) & 1u) << (8 * i + s);
          wv = oct_or(wv);
          if (s == 0 && lane_ok) pk[h * BKW + bs_g + (o * dg + j0) / 4] = wv;
        }
      }
    }
    // partial block tiles: masks of the staged words (the same fields with
    // every code bit and sign bit of a row inside the tile set)
    const bool partial = blk && (cg.slot_lo > 0 || cg.slot_lo + cg.nvalid < 64);
    if (partial) {
      const uint32_t fm = (1u << mg) - 1u;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
        const int t = 16 * mt + ln;
        const bool in = t >= cg.slot_lo && t < cg.slot_lo + cg.nvalid;
        const int fi = in ? (int)fm : 0;
        const int fl[4] = {fi, fi, fi, fi};
        uint32_t wv[4];
        if (mg == 2)
          octet_or_words<2>(fl, s, wv);
        else if (mg == 3)
          octet_or_words<3>(fl, s, wv);
        else if (mg == 1)
          octet_or_words<1>(fl, s, wv);
        else
          octet_or_words<4>(fl, s, wv);
        uint32_t sv = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) sv |= (in ? 1u : 0u) << (8 * i + s);
        sv = oct_or(sv);
        if (s == 0 && lane_ok) {
          uint32_t* dst = pk + (2 + h) * BKW + bc_g + mg * (o * dg + j0) / 4;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < mg) dst[q] = wv[q];
          if (signs_on) pk[(2 + h) * BKW + bs_g + (o * dg + j0) / 4] = sv;
        }
      }
    }
    __syncthreads();  // (5)

    // ---- store: norms, then the records ----
    t_store_tile<KP, NT, BLK>(a, cg, rows, nrmv, gpart, pk, partial, vec_out, tid);
  }
}

template <int KP, int NT>
__device__ __forceinline__ void quantize_tiles_t(const QArgs& a, int64_t first_tile, int64_t tile_stride,
                                                 unsigned char* smem) {
  if (a.fmt == TQ_BLOCK32)
    quantize_tiles_t_fmt<KP, NT, true>(a, first_tile, tile_stride, smem);
  else
    quantize_tiles_t_fmt<KP, NT, false>(a, first_tile, tile_stride, smem);
}

}  // namespace tqq
