// Software-pipelined variant of the transposed tile path for bulk calls:
// d = 128, one channel group, bf16 input.
//
// [ZB] paragraph 2 and [WD] "Como o TurboQuant funciona": rotate each vector,
// give every rotated coordinate its Lloyd-Max cell, take the residual of that
// MSE quantizer, keep the signs of a Gaussian sketch of the residual, store
// codes, sign bits and the norms. The arithmetic is that of the transposed
// tile path, operation for operation (same products, same sums in the same
// order), so both produce identical records; only the order of the work
// across tiles differs.
//
// The transposed tile path separates the steps of a tile by workgroup
// barriers, and with one workgroup per compute unit every wave of the unit
// is in the same step at once: its matrix-core products and its VALU work
// (cells, residuals, packing) never overlap. Here a workgroup has three
// tiles in flight and two phases per tile:
//   X(k): the stores of tile k - 1, the cells, residual, residual norm
//         partials and codes of tile k, and the rotation of tile k + 1 with
//         its per-wave sums of y^2;
//   Y(k): the sketch of tile k's residual and its sign bits, and the staging
//         of tile k + 2's input into LDS (its loads were issued one phase Y
//         earlier).
// Tile k's norms are the sums of the per-wave partials written in X(k - 1).
// What one phase writes and a later phase of another tile still reads (the
// per-wave partials, norms, staged records, destination rows) is
// double-buffered by tile parity; the input tile and the residual parts are
// single buffers, each rewritten only after the barrier that ends its reads.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "tq_quantize_t_dev.h"

namespace tqq {

struct LdsP {
  static constexpr int KP = 128, NT = 8;
  static constexpr int XH = KP + 8;                       // row stride (16-bit units) of the u16 tiles
  static constexpr int TILE = QT * XH * 2;                // bytes of one u16 tile
  static constexpr int off_x = 0;                         // u16 [QT][XH]: input of the next rotation
  static constexpr int off_rh = off_x + TILE;             // u16 [QT][XH]: residual, high part
  static constexpr int off_rl = off_rh + TILE;            // u16 [QT][XH]: residual, low part
  static constexpr int off_npart = off_rl + TILE;         // float [2][NT][QT]: per-wave sums of y^2
  static constexpr int off_gpart = off_npart + 2 * NT * QT * 4;  // float [2][NT][QT]: per-wave sums of r^2
  static constexpr int off_nrm = off_gpart + 2 * NT * QT * 4;    // float [2][QT]: norms n
  static constexpr int off_cb = off_nrm + 2 * QT * 4;            // float [64]: centroids [0, 32), boundaries [32, 64)
  static constexpr int off_rows = off_cb + 64 * 4;               // int64 [2][QT]: destination rows (token-major)
  static constexpr int PKN = LdsT<KP, NT>::PK_WORDS;              // words of one staged-record buffer
  static constexpr int off_pk = off_rows + 2 * QT * 8;           // u32 [2][PKN]: staged records
  static constexpr int bytes = off_pk + 2 * PKN * 4;
};

// Whether a call (validated by make_qargs) takes the pipelined path: the
// transposed tile path's conditions, d = 128, one group, every record word
// covered by the waves' fields, and at least one full tile of vectors.
inline bool p_path_ok(const QArgs& a) {
  return t_path_ok(a) && a.d == LdsP::KP && a.n_groups == 1 && !a.pk_zero && a.n_vec >= QT;
}

// The kernel body: this workgroup quantizes tiles first_tile,
// first_tile + tile_stride, ... of `a` (p_path_ok, gbits[0] == MG, block
// records iff BLK, sign bits iff SIGNS) with 512 threads and the dynamic LDS
// block `smem` (LdsP::bytes).
template <int MG, bool BLK, bool SIGNS>
__device__ __forceinline__ void quantize_tiles_p(const QArgs& a, int64_t first_tile, int64_t tile_stride,
                                                 unsigned char* smem) {
  using L = LdsP;
  constexpr int KP = L::KP, NT = L::NT, XH = L::XH, KS = KP / 32, PKN = L::PKN;
  constexpr int PKW = LdsT<KP, NT>::PKW, BKW = LdsT<KP, NT>::BKW;
  constexpr int NB = (1 << MG) - 1;
  constexpr int DG = KP;  // the one group's dimension
  constexpr bool tok = !BLK;
  uint16_t* xh = reinterpret_cast<uint16_t*>(smem + L::off_x);
  uint16_t* rhi = reinterpret_cast<uint16_t*>(smem + L::off_rh);
  uint16_t* rlo = reinterpret_cast<uint16_t*>(smem + L::off_rl);
  float* npart = reinterpret_cast<float*>(smem + L::off_npart);
  float* gpart = reinterpret_cast<float*>(smem + L::off_gpart);
  float* nrmv = reinterpret_cast<float*>(smem + L::off_nrm);
  float* cbk = reinterpret_cast<float*>(smem + L::off_cb);
  int64_t* rows = reinterpret_cast<int64_t*>(smem + L::off_rows);
  uint32_t* pk = reinterpret_cast<uint32_t*>(smem + L::off_pk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave = 16 output coordinates
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int64_t n_tiles = a.n_tiles;

  // tiles k .. k + 3 of this workgroup (n_tiles: none)
  TileGeo g0, g1, g2, g3;
  int64_t t0 = next_live_tile(a, first_tile, tile_stride, g0);
  if (t0 >= n_tiles) return;  // (uniform: no tile, no barrier)
  int64_t t1 = next_live_tile(a, t0 + tile_stride, tile_stride, g1);
  int64_t t2 = t1 < n_tiles ? next_live_tile(a, t1 + tile_stride, tile_stride, g2) : n_tiles;
  int64_t t3 = n_tiles;

  float cent_reg = 0.f, bnd_reg = 0.f;
  {
    constexpr int NC = 1 << MG;
    cent_reg = a.centroids[tid < NC ? tid : NC - 1];
    bnd_reg = a.boundaries[tid < NB ? tid : NB - 1];
  }
  TStage st;
  load_t<KP, NT>(a, g0, BLK, tid, st);
  u32x4 rh[KS], rm[KS], rl3[KS], sh[KS], sl[KS];
  t_matrix_regs<KS>(a, w, ln, lg, rh, rm, rl3, sh, sl);

  const int j0 = 16 * w + 4 * lg;  // the lane's first channel
  constexpr int mid = (NB + 1) / 2 - 1;  // the cell of a zero vector
  const int pk_code_h = 2 * a.cwoff[0] + MG * w;
  const int pk_sign_h = 2 * (a.code_words + a.swoff[0]) + w;
  const int bcw = a.blk_code_words;
  const int bc_g = a.bcwoff[0], bs_g = bcw + a.bswoff[0];
  const bool vec_out = ((reinterpret_cast<uintptr_t>(a.codes) | reinterpret_cast<uintptr_t>(a.signs)) % 16 == 0) &&
                       (BLK ? (bcw % 4 == 0 && a.blk_sign_words % 4 == 0)
                            : (a.code_words % 4 == 0 && a.sign_words % 4 == 0));

  auto stage_x = [&]() __attribute__((always_inline)) {
    constexpr int CPR = KP / 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * NT * 64, v = c / CPR, k = (c % CPR) * 8;
      *reinterpret_cast<u32x4*>(xh + v * XH + k) = st.c[i];
    }
  };
  // y = rot x of the staged tile, and the per-wave sums of y^2 into npart
  // buffer `nb` (lane l: tile row l)
  auto rotate = [&](f32x4 (&y)[4], int nb) __attribute__((always_inline)) {
    mfma_t_bf16x3<4, KS, XH>(xh, rh, rm, rl3, ln, lg, y);
    float sq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      sq[mt] = fmaf(y[mt][3], y[mt][3], fmaf(y[mt][2], y[mt][2], fmaf(y[mt][1], y[mt][1], y[mt][0] * y[mt][0])));
    npart[(nb * NT + w) * QT + lane] = lg_sum4(sq[0], sq[1], sq[2], sq[3]);
  };

  // ---- prologue: tile k's input staged and rotated, tile k + 1's staged ----
  if (tid < 32) {
    cbk[tid] = cent_reg;
    cbk[32 + tid] = bnd_reg;
  }
  stage_x();
  if (t1 < n_tiles) load_t<KP, NT>(a, g1, BLK, tid, st);
  __syncthreads();
  float tb[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) tb[k] = k < NB ? cbk[32 + k] : INFINITY;
  int zc = 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) zc += (int)(__float_as_uint(tb[k] - 0.0f) >> 31);
  const int zcorr = mid - zc;
  f32x4 yA[4], yB[4];
  rotate(yA, 0);
  __syncthreads();  // the input tile is free
  if (t1 < n_tiles) {
    stage_x();
    if (t2 < n_tiles) load_t<KP, NT>(a, g2, BLK, tid, st);
  }
  __syncthreads();

  TileGeo gp = g0;  // the previous tile (its stores are due)
  bool have_prev = false, partial_prev = false;

  // One tile: parity P selects the double buffers; yc holds tile k's
  // rotation, yn receives tile k + 1's. True after the workgroup's last tile.
  auto iter = [&](auto PAR, f32x4 (&yc)[4], f32x4 (&yn)[4]) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(PAR)::value;
    uint32_t* pkc = pk + P * PKN;
    uint16_t* pkc16 = reinterpret_cast<uint16_t*>(pkc);

    // ================= phase X(k) =================
    // Tile k's cells and codes (VALU) and tile k + 1's rotation (matrix
    // cores; past the last tile it reads a stale input and its result is
    // never used).
    auto cpart = [&]() __attribute__((always_inline)) {
      // tile k's norms (lane l: tile row l; every wave forms the same sums),
      // gathered so that lane (ln, lg) holds those of rows 16 mt + ln
      float nv4[4], inv4[4], sc4[4];
      {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) sum += npart[(P * NT + ww) * QT + lane];
        const float n = sqrtf(sum);
        const float inv = n > 0.f ? __builtin_amdgcn_rcpf(n) : 0.f;
        const float sc = n > 0.f ? __builtin_amdgcn_ldexpf(1.0f, 10 - __builtin_amdgcn_frexp_expf(n)) : 1.0f;
        nrmv[P * QT + lane] = n;
        lg_gather4(n, nv4);
        lg_gather4(inv, inv4);
        lg_gather4(sc, sc4);
      }
      // cells, residual, residual norm partials, packed codes of tile k
      int idx[4][4];
      {
        float gq[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          float u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) u[i] = yc[mt][i] * inv4[mt];
          const int corr = nv4[mt] > 0.f ? 0 : zcorr;
          cells4<NB>(u, tb, corr, idx[mt]);
          float cv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) cv[i] = cbk[idx[mt][i]];
          float rr[4];
          float s = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rr[i] = fmaf(-nv4[mt], cv[i], yc[mt][i]);
            s = fmaf(rr[i], rr[i], s);
          }
          gq[mt] = s;
          if constexpr (SIGNS) {
            f16x2 hv[2], lv[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const _Float16 h = (_Float16)(rr[i] * sc4[mt]);
              hv[i / 2][i % 2] = h;
              lv[i / 2][i % 2] = (_Float16)fmaf(rr[i], sc4[mt], -(float)h);
            }
            const int off = (16 * mt + ln) * XH + j0;
            *reinterpret_cast<uint2*>(rhi + off) =
                uint2{__builtin_bit_cast(uint32_t, hv[0]), __builtin_bit_cast(uint32_t, hv[1])};
            *reinterpret_cast<uint2*>(rlo + off) =
                uint2{__builtin_bit_cast(uint32_t, lv[0]), __builtin_bit_cast(uint32_t, lv[1])};
          }
        }
        gpart[(P * NT + w) * QT + lane] = lg_sum4(gq[0], gq[1], gq[2], gq[3]);
      }
      if constexpr (tok) {
        // the wave's 16 codes of a row (16 MG bits) across the lane groups:
        // lane l stores the MG halfwords of tile row l
        uint32_t flo[4], fhi[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint32_t f4 = (uint32_t)idx[mt][0] | ((uint32_t)idx[mt][1] << MG) | ((uint32_t)idx[mt][2] << (2 * MG)) |
                              ((uint32_t)idx[mt][3] << (3 * MG));
          const uint64_t f = (uint64_t)f4 << (4 * MG * lg);
          flo[mt] = (uint32_t)f;
          fhi[mt] = (uint32_t)(f >> 32);
        }
        const uint32_t lo = lg_or4(flo[0], flo[1], flo[2], flo[3]);
        uint32_t hi = 0u;
        if constexpr (MG > 2) hi = lg_or4(fhi[0], fhi[1], fhi[2], fhi[3]);
        uint16_t* row = pkc16 + lane * 2 * PKW + pk_code_h;
#pragma unroll
        for (int k = 0; k < MG; ++k) row[k] = (uint16_t)((k < 2 ? lo : hi) >> (16 * (k & 1)));
      } else {
        // octet fields (lane s = 0 of each 8 stores the MG words)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
          uint32_t wv[4];
          octet_or_words<MG>(idx[mt], s, wv);
          if (s == 0) {
            uint32_t* dst = pkc + h * BKW + bc_g + MG * (o * DG + j0) / 4;
#pragma unroll
            for (int q = 0; q < MG; ++q) dst[q] = wv[q];
          }
        }
      }
    };
    // tile k - 1's stores (its records were completed in Y(k - 1)), issued
    // first so that their latency overlaps this phase's work
    if (have_prev)
      t_store_tile<KP, NT, BLK>(a, gp, rows + (1 - P) * QT, nrmv + (1 - P) * QT, gpart + (1 - P) * NT * QT,
                                pk + (1 - P) * PKN, partial_prev, vec_out, tid);
    rotate(yn, 1 - P);
    cpart();
    __syncthreads();  // end of X(k)

    // ================= phase Y(k) =================
    if (t2 < n_tiles) stage_x();  // tile k + 2's input (tile k + 1's rotation is done)
    t3 = t2 < n_tiles ? next_live_tile(a, t2 + tile_stride, tile_stride, g3) : n_tiles;
    if (t3 < n_tiles) load_t<KP, NT>(a, g3, BLK, tid, st);
    // (wave 1: wave 0 stores the norms below)
    if (tok && tid >= QT && tid < 2 * QT) t_tile_rows(a, g0, tid - QT, rows + P * QT);
    const bool partial = BLK && (g0.slot_lo > 0 || g0.slot_lo + g0.nvalid < 64);
    // tile k's sketch and sign bits (matrix cores, then VALU)
    auto spart = [&]() __attribute__((always_inline)) {
      if constexpr (SIGNS) {
        f32x4 sacc[4];
        mfma_t_f16x2<4, KS, XH>(rhi, rlo, sh, sl, ln, lg, sacc);
        uint32_t nibs[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          uint32_t nib = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) nib |= (~__float_as_uint(sacc[mt][i]) >> 31) << i;
          nibs[mt] = nib;
        }
        if constexpr (tok) {
          const uint32_t bits16 =
              lg_or4(nibs[0] << (4 * lg), nibs[1] << (4 * lg), nibs[2] << (4 * lg), nibs[3] << (4 * lg));
          pkc16[lane * 2 * PKW + pk_sign_h] = (uint16_t)bits16;
        } else {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
            uint32_t wv = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv |= ((nibs[mt] >> i) & 1u) << (8 * i + s);
            wv = oct_or(wv);
            if (s == 0) pkc[h * BKW + bs_g + (o * DG + j0) / 4] = wv;
          }
        }
      }
      if (partial) {
        // masks of the staged words: every code and sign bit of a row inside
        // the tile set
        constexpr uint32_t fm = (1u << MG) - 1u;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int s = ln & 7, h = mt >> 1, o = 2 * (mt & 1) + (ln >> 3);
          const int t = 16 * mt + ln;
          const bool in = t >= g0.slot_lo && t < g0.slot_lo + g0.nvalid;
          const int fi = in ? (int)fm : 0;
          const int fl[4] = {fi, fi, fi, fi};
          uint32_t wv[4];
          octet_or_words<MG>(fl, s, wv);
          uint32_t sv = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) sv |= (in ? 1u : 0u) << (8 * i + s);
          sv = oct_or(sv);
          if (s == 0) {
            uint32_t* dst = pkc + (2 + h) * BKW + bc_g + MG * (o * DG + j0) / 4;
#pragma unroll
            for (int q = 0; q < MG; ++q) dst[q] = wv[q];
            if constexpr (SIGNS) pkc[(2 + h) * BKW + bs_g + (o * DG + j0) / 4] = sv;
          }
        }
      }
    };
    spart();
    __syncthreads();  // end of Y(k)
    if (t1 >= n_tiles) {
      // the workgroup's last tile: its stores
      t_store_tile<KP, NT, BLK>(a, g0, rows + P * QT, nrmv + P * QT, gpart + P * NT * QT, pkc, partial, vec_out,
                                tid);
      return true;
    }
    gp = g0;
    have_prev = true;
    partial_prev = partial;
    t0 = t1;
    g0 = g1;
    t1 = t2;
    g1 = g2;
    t2 = t3;
    g2 = g3;
    return false;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (;;) {
    if (iter(I0{}, yA, yB)) break;
    if (iter(I1{}, yB, yA)) break;
  }
}

}  // namespace tqq
