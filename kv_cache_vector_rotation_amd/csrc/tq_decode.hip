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
//  1. prep:    q_rot = rot q and q_sk = sketch q per query head (fp32 sums;
//              q_rot stored as an fp16 hi/lo pair, q_sk as fp16), both
//              scaled by scale * log2(e) and q_sk also by alpha_g.
//  2. split:   split-K over the context. A workgroup takes one (batch, KV
//              head, 16-query-head block) and a range of 32-token tiles; its
//              four waves take alternate tiles. Per tile a wave
//              - expands the K codes through LDS tables (two fp16 centroids
//                and, from a second table, their fp16 rounding remainders
//                per lookup) and the K sign bits through a nibble table into
//                fp16 +-1,
//              - forms both logit parts on v_mfma_f32_16x16x32_f16 (tokens x
//                channels times channels x heads); the MSE part uses the
//                hi/lo splits of centroids and queries so its products keep
//                fp32 accuracy; scales them by the tokens' norms and runs
//                the online softmax (accumulators are rescaled only when a
//                head's running maximum moves),
//              - expands the V codes four at a time and the V signs, and
//                accumulates sum_t p_t n_t c[idx_t] and sum_t p_t gamma_t z_t
//                on MFMA (channels x tokens times tokens x heads): V is
//                summed in the rotated and sketch domains, never
//                dequantized per token.
//              The MFMA output layout of the logits (lane = head, 8 tokens)
//              is exactly the operand layout the V product needs, so the
//              softmax weights never leave registers. The four waves merge
//              through LDS into one partial (max, sum, accumulators).
//  3. combine: log-sum-exp merge of the splits, then out = (rot^T acc_rot +
//              sketch^T (alpha_g acc_sk)) / sum: the back-transform runs once
//              per head, which is valid because dequantization is linear.
//
// Record formats: K rows are token-major (a lane's 8 codes of one token are
// one 8m-bit field of the row); V is stored in 32-token blocks where each
// octet of tokens keeps its 8 codes of a channel in one 8m-bit field. Both
// fields feed one lane's eight MFMA operand slots directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "tq_internal.h"
#include "tq_prep_dev.h"
#include "tq_quantize_dev.h"
#include "turboquant.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2))) __attribute__((aligned(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Low parts of the split fp16 operands are stored times 2^11 so they stay in
// the normal fp16 range; their products are scaled back by 2^-11.
constexpr float kLoInv = 1.0f / 2048.0f;
constexpr int kWaves = 4;
constexpr int kTile = 32;

struct DArgs {
  int batch, hq, hkv, group;  // group = hq / hkv (heads here are (q head, query token) pairs)
  int n_split;
  int T;  // query tokens per head: column hloc is token hloc % T, causal past n_ctx - T + t
  int64_t n_ctx, cap;
  float scale;
  const _Float16* qprep;  // [batch*hq][3d]: q_rot hi, q_rot lo * 2^11, q_sk
  const float* kscale;    // per K group: the fp16 table holds c * kscale
  const uint32_t* kc;
  const uint32_t* ks;
  const float* kn;  // norm pairs: float32, or float16 when kn_f16 (then read as words)
  const uint32_t* vc;
  const uint32_t* vs;
  const float* vn;
  int kn_f16, vn_f16;      // norms stored as float16
  int kn_shift, vn_shift;  // log2 of the norm bytes per row
  const float* kcent;  // K centroids (concatenated over groups)
  const float* vcent;
  float* logits;  // [batch, hq, n_ctx] or null
  float* part;    // [batch*hq][n_split][2 + 2d]
  // paged cache (block_table non-null): logical 32-token block j of batch b
  // is physical block block_table[b * max_blocks + j], whose rows are
  // (block * hkv + kv head) * 32 + token; seq_lens[b] (or n_ctx) tokens
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_blocks;
  int64_t n_pblocks;  // physical blocks in the caches (entries are clamped into range)
};

// two floats -> packed fp16 pair (round to nearest even; one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t h2bits(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// DPP row move in which a lane whose source lies outside its 16-lane row keeps
// its own value. Every lane uses the result, so the move is never placed
// under a lane mask (a DPP read from a masked-off lane returns nothing).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  const int x = __float_as_int(v);
  return __int_as_float(__builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false));
}
// The same move with 0 where the source lies outside the row (the compiler
// can fold it into the consuming multiply); only for results that every lane
// uses unconditionally.
template <int CTRL>
__device__ __forceinline__ float dpp_row_z(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// max over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48): swap the
// 32-lane halves, then odd and even rows, with v_permlane{32,16}_swap
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

// ---------------------------------------------------------------------------
// Lookup tables in LDS. A table of E entries of W bytes keeps each entry
// replicated across one 256-byte LDS row (entry e, replica r at byte
// e * 256 + W * r, 256 / W replicas); lane l reads replica l mod (256 / W),
// so the lanes served together in one LDS cycle hit distinct banks whatever
// entries they look up. Tables with more than 64 entries are stored plainly.
// ---------------------------------------------------------------------------
template <int E, int W>
struct Tab {
  static constexpr bool REP = E <= 64;
  static constexpr int BYTES = REP ? E * 256 : E * W;
};

template <int E, int W>
__device__ __forceinline__ uint32_t tab_addr(uint32_t e, uint32_t lane_off) {
  if constexpr (Tab<E, W>::REP)
    return (e << 8) | lane_off;
  else
    return e * W;
}

// Fills a table from value(e) (a uint32_t for W = 4, a u32x2 for W = 8). A
// replicated entry's 256-byte row is written as 16 16-byte stores, each by
// its own thread, with the value computed once per store.
template <int E, int W, typename F>
__device__ void tab_build(unsigned char* base, int tid, F value) {
  if constexpr (Tab<E, W>::REP) {
    for (int i = tid; i < E * 16; i += 256) {
      const int e = i >> 4, k = i & 15;
      u32x4 v;
      if constexpr (W == 4) {
        const uint32_t x = value(e);
        v = u32x4{x, x, x, x};
      } else {
        const u32x2 x = value(e);
        v = u32x4{x[0], x[1], x[0], x[1]};
      }
      *reinterpret_cast<u32x4*>(base + e * 256 + 16 * k) = v;
    }
  } else {
    for (int e = tid; e < E; e += 256) {
      if constexpr (W == 4)
        *reinterpret_cast<uint32_t*>(base + e * W) = value(e);
      else
        *reinterpret_cast<u32x2*>(base + e * W) = value(e);
    }
  }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Address of the table entry whose index is the ilog2(E)-bit field at bit
// pos of the word array w (pos is a constant once the callers' loops are
// unrolled; a field may run into the next word, which must exist). The
// field is brought to its position in the address by one shift, or one
// funnel shift where it crosses a word, and masked into the lane's replica
// offset by one v_and_or.
template <int E, int W>
__device__ __forceinline__ uint32_t tab_addr_at(const uint32_t* w, int pos, uint32_t lane_off) {
  constexpr int NB = ilog2(E), P = Tab<E, W>::REP ? 8 : ilog2(W);
  const int wi = pos >> 5, b = pos & 31;
  const uint32_t mask = (uint32_t)(E - 1) << P;
  uint32_t t;
  if (b + NB > 32)
    t = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], b - P);
  else if (b >= P)
    t = w[wi] >> (b - P);
  else
    t = w[wi] << (P - b);
  if constexpr (Tab<E, W>::REP)
    return (t & mask) | lane_off;
  else
    return t & mask;
}

// 8 sign bits at bit pos of w (bit s -> slot s) -> 8 fp16 values, +1 where
// set, -1 where clear.
__device__ __forceinline__ u32x4 signs8(const uint32_t* w, int pos, const unsigned char* stab, uint32_t off8) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(stab + tab_addr_at<16, 8>(w, pos, off8));
  const u32x2 hi = *reinterpret_cast<const u32x2*>(stab + tab_addr_at<16, 8>(w, pos + 4, off8));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 8 codes of M bits at bit pos of w (code s at bits [pos + M s, pos + M s + M))
// -> 8 fp16 centroids, one 4-byte lookup per pair.
template <int M>
__device__ __forceinline__ u32x4 codes8(const uint32_t* w, int pos, const unsigned char* tab, uint32_t off4) {
  constexpr int E = 1 << (2 * M);
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    r[p] = *reinterpret_cast<const uint32_t*>(tab + tab_addr_at<E, 4>(w, pos + 2 * M * p, off4));
  return r;
}

// Loads N consecutive words from a 4-byte aligned address.
template <int N>
__device__ __forceinline__ void load_w(const uint32_t* p, uint32_t* out) {
  if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const u32x2a4 v = reinterpret_cast<const u32x2a4*>(p)[i];
      out[2 * i] = v[0];
      out[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = p[i];
  }
}

// Norms (n_g, gamma_g) of 8 consecutive tokens from the wave's LDS staging.
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

constexpr int max_lane_shift(int kb) {
  int m = 0;
  for (int g = 0; g < 4; ++g) m = (kb * g) % 32 > m ? (kb * g) % 32 : m;
  return m;
}

// Compile-time geometry of one decode instantiation.
//
// Logit product: chunk c of 32 k-slots lies in quantizer group g = c / CPG
// (local chunk cl = c % CPG); lane group lg, slot s holds channel
// 8 CPG lg + 8 cl + s of that group, so a lane's channels of one token form a
// single contiguous run of 8 CPG codes (8 M CPG bits) of the row.
// V product: tile v of 16 rows lies in group g = v / MTPG; row r holds channel
// RUN r + v % MTPG of the group, so a lane's channels are one run of RUN.
template <int D, int NG, int M0, int M1>
struct Geo {
  static constexpr int DG = D / NG, CPG = DG / 32, NC = D / 32, NMT = D / 16, MTPG = NMT / NG,
                       RUN = DG / 16;
  static constexpr int MB[2] = {M0, M1};
  static constexpr int CWG[2] = {(M0 * DG + 31) / 32, NG > 1 ? (M1 * DG + 31) / 32 : 0};
  static constexpr int CW = CWG[0] + CWG[1];
  static constexpr int CWOFF[2] = {0, CWG[0]};
  static constexpr int SWG = (DG + 31) / 32;
  static constexpr int SW = SWG * NG;
  static constexpr int SWOFF[2] = {0, SWG};
  static constexpr int BCW = M0 * DG + (NG > 1 ? M1 * DG : 0);
  static constexpr int BCWOFF[2] = {0, M0 * DG};
  static constexpr int BSW = D;
  static constexpr int BSWOFF[2] = {0, DG};
  // per lane and token: K code bits, words loaded, offset in the lane's K words
  static constexpr int KB[2] = {8 * M0 * CPG, 8 * M1 * CPG};
  static constexpr int KSH[2] = {max_lane_shift(KB[0]), max_lane_shift(KB[1])};
  static constexpr int KNW[2] = {(KB[0] + KSH[0] + 31) / 32, NG > 1 ? (KB[1] + KSH[1] + 31) / 32 : 0};
  static constexpr int KOFF[2] = {0, KNW[0]};
  static constexpr int KNWT = KNW[0] + KNW[1];
  // per lane: V code words and sign words of each group
  static constexpr int VNW[2] = {RUN * M0 / 4, NG > 1 ? RUN * M1 / 4 : 0};
  static constexpr int VOFF[2] = {0, VNW[0]};
  static constexpr int VNWT = VNW[0] + VNW[1];
  static constexpr int VNS = RUN / 4;
  // table sizes
  static constexpr int KE[2] = {1 << (2 * M0), 1 << (2 * M1)};
  static constexpr int KTB[2] = {Tab<KE[0], 4>::BYTES, NG > 1 ? Tab<KE[1], 4>::BYTES : 0};
  static constexpr int VTB[2] = {Tab<KE[0], 4>::BYTES, NG > 1 ? Tab<KE[1], 4>::BYTES : 0};
  static constexpr int STB = Tab<16, 8>::BYTES;
};

// Raw record data of one 32-token tile for one lane (what it loads from HBM).
template <int D, int NG, int M0, int M1>
struct Raw {
  using G = Geo<D, NG, M0, M1>;
  uint32_t kc[2][G::KNWT];  // K code words of the lane's token in each half-tile
  uint32_t ks[2][NG];       // K sign word holding the lane's sign bits, per group
  uint32_t kn[NG];          // the words holding the lane's share of the tile's K norms
  uint32_t vn[NG];          // and of the V norms
  uint32_t vc[G::VNWT];     // V code words (octet lg, channels RUN ln ..)
  uint32_t vs[G::VNS * NG]; // V sign words
};

// Per-lane word offsets of a tile's data, relative to the tile's first row
// (K, norms) or block (V); the same for every tile.
template <int D, int NG, int M0, int M1>
struct LaneOff {
  uint32_t kc[2][NG];
  uint32_t ks[2][NG];
  uint32_t vc[NG];
  uint32_t vs[NG];
};

template <int D, int NG, int M0, int M1>
__device__ __forceinline__ LaneOff<D, NG, M0, M1> lane_offsets(int ln, int lg) {
  using G = Geo<D, NG, M0, M1>;
  LaneOff<D, NG, M0, M1> o;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    // logit-product row ln <-> token 8 (ln / 4) + 4 tau + ln % 4 of the tile
    const uint32_t row = 8 * (ln >> 2) + 4 * tau + (ln & 3);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      o.kc[tau][g] = row * G::CW + G::CWOFF[g] + ((G::KB[g] * lg) >> 5);
      o.ks[tau][g] = row * G::SW + G::SWOFF[g] + ((8 * G::CPG * lg) >> 5);
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    o.vc[g] = G::BCWOFF[g] + (G::MB[g] * (lg * G::DG + G::RUN * ln)) / 4;
    o.vs[g] = G::BSWOFF[g] + (lg * G::DG + G::RUN * ln) / 4;
  }
  return o;
}

// Loads one 32-token tile whose first cache row is row0 (wave-uniform, a
// multiple of 32): the base addresses are scalar, the lanes add their offsets.
// Byte offsets (from a tile's first row) of the words holding the lane's norm
// values i = lane NG + e of the tile's [32][2 NG] values, and the shift of a
// float16 value within its word.
template <int NG>
struct NormOff {
  uint32_t kb[NG], vb[NG], ksh[NG], vsh[NG];
};

// A stored norm value from the word that holds it.
__device__ __forceinline__ float norm_value(uint32_t w, uint32_t sh, int f16) {
  return f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> sh)) : __uint_as_float(w);
}

template <int D, int NG, int M0, int M1, int WV>
__device__ __forceinline__ void load_tile(const DArgs& a, int64_t row0, int lane,
                                          const LaneOff<D, NG, M0, M1>& o, const NormOff<NG>& no,
                                          Raw<D, NG, M0, M1>& r) {
  using G = Geo<D, NG, M0, M1>;
  const uint32_t* kc = a.kc + row0 * G::CW;
  const uint32_t* ks = a.ks + row0 * G::SW;
  auto k_rows = [&](auto gc) {
    constexpr int g = decltype(gc)::value;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      load_w<G::KNW[g]>(kc + o.kc[tau][g], &r.kc[tau][G::KOFF[g]]);
      r.ks[tau][g] = ks[o.ks[tau][g]];
    }
  };
  k_rows(std::integral_constant<int, 0>{});
  if constexpr (NG > 1) k_rows(std::integral_constant<int, 1>{});
  const unsigned char* kn = reinterpret_cast<const unsigned char*>(a.kn) + (row0 << a.kn_shift);
#pragma unroll
  for (int e = 0; e < NG; ++e) r.kn[e] = *reinterpret_cast<const uint32_t*>(kn + no.kb[e]);
  if constexpr (WV != 0) {
    const unsigned char* vn = reinterpret_cast<const unsigned char*>(a.vn) + (row0 << a.vn_shift);
#pragma unroll
    for (int e = 0; e < NG; ++e) r.vn[e] = *reinterpret_cast<const uint32_t*>(vn + no.vb[e]);
    const int64_t blk = row0 / 32;
    const uint32_t* vc = a.vc + blk * G::BCW;
    const uint32_t* vs = a.vs + blk * G::BSW;
    auto v_words = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      load_w<G::VNW[g]>(vc + o.vc[g], &r.vc[G::VOFF[g]]);
      if constexpr (WV == 1) load_w<G::VNS>(vs + o.vs[g], &r.vs[G::VNS * g]);
    };
    v_words(std::integral_constant<int, 0>{});
    if constexpr (NG > 1) v_words(std::integral_constant<int, 1>{});
  }
}

// HB = query heads per workgroup and MFMA column block: 16, or 4 ("packed",
// for KV groups of at most 4 query heads; with one quantizer group it fits
// three waves per SIMD). Packed, the 16 MFMA columns hold
// [q_rot hi | q_rot lo | q_sk | unused] x 4 heads for the logits and
// [p n | p gamma | 0 | 0] x 4 heads for the V sums, so one accumulator
// serves all three logit parts and one serves both V parts.
// WV = 0: logits only; 1: V records with sign bits; 2: MSE-only V records
// (codes and norms alone; the sign product is skipped).
template <int D, int NG, int M0, int M1, int WV, int HB>
__global__ __launch_bounds__(256, HB == 4 && NG == 1 ? 3 : 2) void decode_kernel(DArgs a) {
  using G = Geo<D, NG, M0, M1>;
  constexpr bool PK = HB == 4;
  constexpr int NC = G::NC, CPG = G::CPG, NMT = G::NMT, MTPG = G::MTPG, RUN = G::RUN, DG = G::DG;
  constexpr int KT1 = G::KTB[0], VT0 = KT1 + G::KTB[1], VT1 = VT0 + G::VTB[0];
  constexpr int ST = VT1 + G::VTB[1];
  constexpr int TAB_BYTES = ST + G::STB;
  // two merge regions of 16 heads x (2 (D + 16 D / 64) + 1) floats
  constexpr int ACC_BYTES = WV ? 2 * 16 * (2 * (D + 16 * (D / 64)) + 1) * 4 : 0;
  constexpr int SMEM = TAB_BYTES > ACC_BYTES ? TAB_BYTES : ACC_BYTES;
  __shared__ __align__(16) unsigned char s_tab[SMEM];  // tables; after the loop: merge buffer
  __shared__ __align__(16) float s_nrm[kWaves][2][64 * NG];  // per-wave norm staging (K, V)
  __shared__ float s_m[kWaves][16];
  __shared__ float s_lw[kWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;  // b * hkv + kv head
  const int hblk = blockIdx.z;
  const int b = bh / a.hkv;
  const int kvh = bh % a.hkv;
  const uint32_t off8 = 8u * (lane & 31), off4 = 4u * lane;

  // ---- this wave's tiles; the first one is loaded before the tables are
  // built, so its memory latency overlaps the table setup ----
  // tokens of this sequence (a paged call may give each its own length)
  int64_t N = a.n_ctx;
  if (a.seq_lens) {
    const int64_t n = a.seq_lens[b];
    N = n < 1 ? 1 : (n > a.n_ctx ? a.n_ctx : n);
  }
  const int64_t n_tiles = (N + kTile - 1) / kTile;
  const int64_t tps = (n_tiles + a.n_split - 1) / a.n_split;
  const int64_t t_begin = split * tps;
  const int64_t t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;
  const int64_t rowbase = (int64_t)bh * a.cap;
  // first cache row of tile t of this (batch, KV head)
  auto tile_row = [&](int64_t t) __attribute__((always_inline)) -> int64_t {
    if (!a.block_table) return rowbase + t * kTile;
    int64_t pb = a.block_table[(int64_t)b * a.max_blocks + t];
    pb = pb < 0 ? 0 : (pb >= a.n_pblocks ? a.n_pblocks - 1 : pb);
    return (pb * a.hkv + kvh) * kTile;
  };
  const LaneOff<D, NG, M0, M1> lo = lane_offsets<D, NG, M0, M1>(ln, lg);
  NormOff<NG> no;
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    const uint32_t i = lane * NG + e;
    no.kb[e] = a.kn_f16 ? 4 * (i >> 1) : 4 * i;
    no.ksh[e] = a.kn_f16 ? 16 * (i & 1) : 0;
    no.vb[e] = a.vn_f16 ? 4 * (i >> 1) : 4 * i;
    no.vsh[e] = a.vn_f16 ? 16 * (i & 1) : 0;
  }
  // lane l stages floats l NG + e of a tile's K norms [32][n_0, gamma_0, ..]:
  // an n_g is divided by the group's codebook scale s_g
  float kn_mul[NG];
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    const int f = (lane * NG + e) % (2 * NG);
    kn_mul[e] = (f & 1) ? 1.0f : 1.0f / a.kscale[f >> 1];
  }

  // ---- tables (built from an LDS copy of the centroids) ----
  __shared__ float s_cent[2][32];
  float cent_k = 0.f, cent_v = 0.f;
  if (tid < 32) {
    // K centroids are tabulated as fp16(s_g c): scaled here by the group's s_g
    const int nc = (1 << M0) + (NG > 1 ? (1 << M1) : 0);
    const int tc = tid < nc ? tid : nc - 1;
    cent_k = a.kcent[tc] * a.kscale[NG > 1 && tc >= (1 << M0) ? 1 : 0];
    if constexpr (WV != 0) cent_v = a.vcent[tc];
  }
  // ---- this lane's head and its query operands (B operand: channels x heads) ----
  // (loaded before the first tile: loads complete in issue order, so using
  // them then does not wait for the tile)
  // packed: column ln = (role, head) with role = ln / 4: 0 q_rot hi / rot
  // weights, 1 q_rot lo / sketch weights, 2 q_sk, 3 unused
  const int role = PK ? ln >> 2 : 0;
  const int hcol = PK ? ln & 3 : ln;  // head of this lane's column within the block
  const int hloc = hblk * HB + hcol;  // head index within the KV group
  const bool hvalid = hloc < a.group;
  const int hq = kvh * a.group + hloc;
  u32x4 qr[NC], qrl[PK ? 1 : NC], qs[NC];  // packed: qr = B of the code product, qs = B of the sign product
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int g = c / CPG, cl = c % CPG;
    const _Float16* qp = a.qprep + ((int64_t)b * a.hq + (hvalid ? hq : 0)) * (3 * D) + g * DG + 8 * CPG * lg + 8 * cl;
    if constexpr (PK) {
      const u32x4 z{0, 0, 0, 0};
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + (role == 0 ? 0 : role == 1 ? D : 2 * D));
      qr[c] = hvalid && role < 2 ? v : z;
      qs[c] = hvalid && role == 2 ? v : z;
    } else {
      const u32x4 z{0, 0, 0, 0};
      const u32x4 vr = *reinterpret_cast<const u32x4*>(qp);
      const u32x4 vl = *reinterpret_cast<const u32x4*>(qp + D);
      const u32x4 vs = *reinterpret_cast<const u32x4*>(qp + 2 * D);
      qr[c] = hvalid ? vr : z;
      qrl[c] = hvalid ? vl : z;
      qs[c] = hvalid ? vs : z;
    }
  }
  // register buffers: NBUF - 1 tiles in flight while one is computed. One
  // tile ahead measures faster than two or three: every workgroup starts at
  // once, and a smaller initial burst of loads brings each wave's first tile
  // sooner.
  constexpr int NBUF = 2;
  Raw<D, NG, M0, M1> rb0, rb1, rb2, rb3;  // (the first NBUF are used)
  auto rbuf = [&](auto kc) __attribute__((always_inline)) -> Raw<D, NG, M0, M1>& {
    constexpr int k = decltype(kc)::value % NBUF;
    if constexpr (k == 0) return rb0;
    else if constexpr (k == 1) return rb1;
    else if constexpr (k == 2) return rb2;
    else return rb3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int64_t tile = t_begin + wv;
  // (unconditional, so the wait for the centroids below need not drain it;
  // a wave without tiles loads tile 0, which always exists, and drops it)
  load_tile<D, NG, M0, M1, WV>(a, tile_row(tile < t_end ? tile : 0), lane, lo, no, rb0);
  if (tid < 32) {
    s_cent[0][tid] = cent_k;
    s_cent[1][tid] = cent_v;
  }
  __syncthreads();
  {
    // pair entry e = (code e mod L, code e div L): two fp16 centroids
    auto hi_val = [](const float* cent, int m) {
      return [=](int e) { return h2bits(cent[e & ((1 << m) - 1)], cent[e >> m]); };
    };
    tab_build<G::KE[0], 4>(s_tab, tid, hi_val(s_cent[0], M0));
    if constexpr (NG > 1) tab_build<G::KE[1], 4>(s_tab + KT1, tid, hi_val(s_cent[0] + (1 << M0), M1));
    if constexpr (WV != 0) {
      tab_build<G::KE[0], 4>(s_tab + VT0, tid, hi_val(s_cent[1], M0));
      if constexpr (NG > 1) tab_build<G::KE[1], 4>(s_tab + VT1, tid, hi_val(s_cent[1] + (1 << M0), M1));
    }
    // nibble -> four fp16 values, +1 where the bit is set, -1 where clear
    tab_build<16, 8>(s_tab + ST, tid, [](int e) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        w[h] = (((e >> (2 * h)) & 1) ? 0x3C00u : 0xBC00u) | (((e >> (2 * h + 1)) & 1) ? 0x3C000000u : 0xBC000000u);
      return u32x2{w[0], w[1]};
    });
  }

  __syncthreads();

  const unsigned char* stab = s_tab + ST;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_r[WV ? NMT : 1], acc_s[WV && !PK ? NMT : 1];  // packed: acc_r holds both
#pragma unroll
  for (int v = 0; v < (WV ? NMT : 1); ++v) acc_r[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < (WV && !PK ? NMT : 1); ++v) acc_s[v] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Raw<D, NG, M0, M1>& r, int64_t T0) __attribute__((always_inline)) {
    // tokens past n_ctx (only in the last tile): norms staged as 0 (rows past
    // the context may hold anything) and logits masked to -inf below
    const bool full = T0 + kTile <= N;
    // stage this tile's norms for the head-major lanes
    {
      // lane l holds float l NG + e of the tile's [32][2 NG] norms
      const bool nok = full || T0 + (lane * NG) / (2 * NG) < N;
#pragma unroll
      for (int e = 0; e < NG; ++e) {
        s_nrm[wv][0][lane * NG + e] = nok ? norm_value(r.kn[e], no.ksh[e], a.kn_f16) * kn_mul[e] : 0.f;
        if constexpr (WV != 0)
          s_nrm[wv][1][lane * NG + e] = nok ? norm_value(r.vn[e], no.vsh[e], a.vn_f16) : 0.f;
      }
    }
    // LDS operations of one wave execute in order; the wave barrier only keeps
    // the compiler from moving the reads above the writes (a memory fence here
    // would also wait for the next tile's loads in flight)
    __builtin_amdgcn_wave_barrier();
    // ---------------- K: logits ----------------
    f32x4 lr[2][NG], lrl[PK ? 1 : 2][NG], ls[PK ? 1 : 2][NG];  // packed: lr holds all three parts
    auto k_group = [&](auto gc, int tau) {
      constexpr int g = decltype(gc)::value;
      constexpr int M = G::MB[g];
      lr[tau][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!PK) lrl[tau][g] = ls[tau][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      // the lane's K code bits of this group start at bit (KB lg) mod 32 of its words
      uint32_t w[G::KNW[g] + 1];
      const int sh = (G::KB[g] * lg) & 31;
#pragma unroll
      for (int i = 0; i < G::KNW[g]; ++i) {
        const uint32_t lo = r.kc[tau][G::KOFF[g] + i];
        const uint32_t hi = i + 1 < G::KNW[g] ? r.kc[tau][G::KOFF[g] + i + 1] : 0u;
        w[i] = G::KSH[g] ? __builtin_amdgcn_alignbit(hi, lo, sh) : lo;
      }
      w[G::KNW[g]] = 0u;
      const uint32_t sword[1] = {r.ks[tau][g] >> ((8 * CPG * lg) & 31)};
      const unsigned char* kt = g == 0 ? s_tab : s_tab + KT1;
#pragma unroll
      for (int cl = 0; cl < CPG; ++cl) {
        const int c = g * CPG + cl;
        const u32x4 ak = codes8<M>(w, 8 * M * cl, kt, off4);
        const u32x4 az = signs8(sword, 8 * cl, stab, off8);
        // (s c) q = (s c)16 (q_hi + 2^-11 q_lo'): products exact, fp32 sums;
        // 1 / s is applied with the token's norm
        if constexpr (PK) {
          lr[tau][g] = mfma16(ak, qr[c], lr[tau][g]);
          lr[tau][g] = mfma16(az, qs[c], lr[tau][g]);
        } else {
          lr[tau][g] = mfma16(ak, qr[c], lr[tau][g]);
          lrl[tau][g] = mfma16(ak, qrl[c], lrl[tau][g]);
          ls[tau][g] = mfma16(az, qs[c], ls[tau][g]);
        }
      }
    };
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      k_group(std::integral_constant<int, 0>{}, tau);
      if constexpr (NG > 1) k_group(std::integral_constant<int, 1>{}, tau);
    }
    // lane (head ln, lg) now holds tokens 8 lg + j, j = 4 tau + i
    const int64_t tok0 = T0 + 8 * lg;
    float kn[8][2 * NG];
    load_norms<NG>(&s_nrm[wv][0][8 * lg * 2 * NG], kn);
    float l2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tau = j >> 2, i = j & 3;
      // (the prepared queries carry scale * log2(e), and alpha_g on the
      // sketch part, so this is the logit in the log2 domain)
      float s;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float t;
        if constexpr (PK) {
          // this lane's column is q_rot hi; q_rot lo and q_sk are 4 and 8 lanes up
          const float v = lr[tau][g][i];
          const float vl = dpp_row_z<0x104>(v), vs = dpp_row_z<0x108>(v);  // row_shl:4, row_shl:8
          t = kn[j][2 * g] * fmaf(kLoInv, vl, v) + kn[j][2 * g + 1] * vs;
        } else {
          t = kn[j][2 * g] * fmaf(kLoInv, lrl[tau][g][i], lr[tau][g][i]) + kn[j][2 * g + 1] * ls[tau][g][i];
        }
        s = g == 0 ? t : s + t;
      }
      l2[j] = s;
    }
    // tokens of the tile before n_ctx (32 except in the last tile)
    const int nvt = full ? kTile : (int)(N - T0);
    // a chunk of T query tokens: this column's token t sees [0, N - T + t]
    if (a.T > 1) {
      const int64_t lim = N - a.T + hloc % a.T + 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) l2[j] = tok0 + j < lim ? l2[j] : -INFINITY;
    }
    // (packed: only the role-0 columns are logits; the other columns carry
    // finite values that no result uses)
    if (a.logits) {
      if (hvalid && role == 0) {
        float* lp = a.logits + ((int64_t)b * a.hq + hq) * a.n_ctx + tok0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * lg + j < nvt) lp[j] = l2[j] * kLn2;
      }
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) l2[j] = 8 * lg + j < nvt ? l2[j] : -INFINITY;
    }
    if constexpr (WV != 0) {
      // ---------------- online softmax ----------------
      float mx = l2[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, l2[j]);
      mx = rows4_max(mx);
      // The reference is kept at an integer (log2 domain): every weight and
      // every rescale is then an exact power of two times the same mantissa,
      // so the fp16 weights, and hence the result, do not depend on how the
      // context is split.
      const float m_new = fmaxf(m_run, ceilf(mx));
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        // some head's maximum moved: rescale (factor 1 for the others; a
        // head that has seen only masked tokens keeps -inf and factor 1)
        const float corr = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
        if constexpr (PK) {
          // the sketch column of a head (role 1) takes its head's factor
          // from 4 lanes down; the role 2 and 3 columns are zero
          const float cc = dpp_row<0x114>(corr);  // row_shr:4
#pragma unroll
          for (int v = 0; v < NMT; ++v) acc_r[v] *= cc;
        } else {
#pragma unroll
          for (int v = 0; v < NMT; ++v) {
            acc_r[v] *= corr;
            acc_s[v] *= corr;
          }
        }
        m_run = m_new;
      }
      float p[8], psum;
      // (m_run is -inf only while every token seen is masked: then p = 0)
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(l2[j] - m_ref);
        psum = j == 0 ? p[j] : psum + p[j];
      }
      l_run += psum;
      // B operands of the V product: slot j <-> token 8 lg + j
      float vn[8][2 * NG];
      load_norms<NG>(&s_nrm[wv][1][8 * lg * 2 * NG], vn);
      u32x4 pr[NG], pz[NG];
      if constexpr (PK) {
        // column role 0 carries p n (code product), role 1 carries p gamma of
        // the head 4 lanes down (sign product); the other columns are 0
        float pp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[j] = dpp_row<0x114>(p[j]);  // row_shr:4; role 0 keeps its own
        const u32x4 z{0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          u32x4 w;
          // (a select of two constant indices: an index that depends on the
          // lane would be lowered to a search over the whole array)
          const bool r1 = role == 1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float n0 = r1 ? vn[2 * q][2 * g + 1] : vn[2 * q][2 * g];
            const float n1 = r1 ? vn[2 * q + 1][2 * g + 1] : vn[2 * q + 1][2 * g];
            w[q] = h2bits(pp[2 * q] * n0, pp[2 * q + 1] * n1);
          }
          pr[g] = role == 0 ? w : z;
          pz[g] = role == 1 ? w : z;
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j0 = 2 * q, j1 = 2 * q + 1;
            // (alpha_g is applied once per head in the combine; past n_ctx p = 0
            // and the staged norms are 0)
            pr[g][q] = h2bits(p[j0] * vn[j0][2 * g], p[j1] * vn[j1][2 * g]);
            pz[g][q] = h2bits(p[j0] * vn[j0][2 * g + 1], p[j1] * vn[j1][2 * g + 1]);
          }
        }
      }
      // ---------------- V: accumulate in the rotated / sketch domains ----------------
      auto v_group = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int M = G::MB[g];
        uint32_t cw[G::VNW[g] + 1];
#pragma unroll
        for (int i = 0; i < G::VNW[g]; ++i) cw[i] = r.vc[G::VOFF[g] + i];
        cw[G::VNW[g]] = 0u;
        const unsigned char* vt = g == 0 ? s_tab + VT0 : s_tab + VT1;
#pragma unroll
        for (int u = 0; u < RUN; ++u) {
          const u32x4 av = codes8<M>(cw, 8 * M * u, vt, off4);
          acc_r[g * MTPG + u] = mfma16(av, pr[g], acc_r[g * MTPG + u]);
          if constexpr (WV == 1) {  // (MSE-only V: no sign product; the sketch sums stay 0)
            const u32x4 az = signs8(&r.vs[G::VNS * g], 8 * u, stab, off8);
            if constexpr (PK)
              acc_r[g * MTPG + u] = mfma16(az, pz[g], acc_r[g * MTPG + u]);
            else
              acc_s[g * MTPG + u] = mfma16(az, pz[g], acc_s[g * MTPG + u]);
          }
        }
      };
      v_group(std::integral_constant<int, 0>{});
      if constexpr (NG > 1) v_group(std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- software-pipelined loop ----
  // NBUF - 1 tiles stay in flight while one is computed: NBUF register
  // buffers in rotation (the loop is unrolled NBUF times so no data is
  // copied). The prefetch is unconditional: past the wave's last tile it
  // reloads that tile (in bounds, a cache hit, dropped), so the compiler sees
  // one straight-line load stream.
  if (tile < t_end) {
    const int64_t last = t_end - 1 - ((t_end - 1 - tile) % kWaves);  // this wave's last tile
    auto next = [&](int64_t t, int k) { return t + k * kWaves <= last ? t + k * kWaves : last; };
    if constexpr (NBUF > 2) load_tile<D, NG, M0, M1, WV>(a, tile_row(next(tile, 1)), lane, lo, no, rb1);
    if constexpr (NBUF > 3) load_tile<D, NG, M0, M1, WV>(a, tile_row(next(tile, 2)), lane, lo, no, rb2);
    // one pass of the rotation: true after the wave's last tile
    auto stage = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      load_tile<D, NG, M0, M1, WV>(a, tile_row(next(tile, NBUF - 1)), lane, lo, no,
                                   rbuf(std::integral_constant<int, k + NBUF - 1>{}));
      compute(rbuf(kc), tile * kTile);
      if (tile == last) return true;
      tile += kWaves;
      return false;
    };
    for (;;) {
      if (stage(I0{})) break;
      if (stage(I1{})) break;
      if constexpr (NBUF > 2)
        if (stage(I2{})) break;
      if constexpr (NBUF > 3)
        if (stage(I3{})) break;
    }
  }

  if constexpr (WV != 0) {
    // ---- merge the four waves into one partial (the table space is reused) ----
    // Region r (r = 0, 1) holds, head-major, the sum of the accumulators of
    // waves r and r + 2 scaled to the workgroup maximum: waves 0 and 1 store,
    // then waves 2 and 3 add. Head h, part pt, channel ch sits at
    // h HS + pt DP + ch + 16 (ch / 64): the odd head stride and the skew of
    // every 64 channels keep both the register-order stores and the
    // channel-order reads free of bank conflicts.
    constexpr int DP = D + 16 * (D / 64), HS = 2 * DP + 1, REG = 16 * HS;
    float* s_red = reinterpret_cast<float*>(s_tab);
    __syncthreads();  // tables are no longer read
    l_run = rows4_sum(l_run);
    // (packed: the role-0 lanes own a head's maximum and sum; the role-1
    // lanes, which hold its sketch sums, read the maximum back from LDS)
    if (lg == 0 && role == 0) s_m[wv][hcol] = m_run;
    __syncthreads();
    float M = s_m[0][hcol];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][hcol]);
    const float m_own = PK ? s_m[wv][hcol] : m_run;
    const float e = (m_own == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_own - M);
    if (lg == 0 && role == 0) s_lw[wv][hcol] = l_run * e;
    float* reg = s_red + (wv & 1) * REG + hcol * HS;
    auto slot = [&](int pt, int v, int i) {
      const int g = v / MTPG, u = v % MTPG;
      const int ch = g * DG + RUN * (4 * lg + i) + u;
      return pt * DP + ch + 16 * (ch >> 6);
    };
    if (wv < 2) {
#pragma unroll
      for (int v = 0; v < NMT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PK) {
            if (role < 2) reg[slot(role, v, i)] = acc_r[v][i] * e;
          } else {
            reg[slot(0, v, i)] = acc_r[v][i] * e;
            reg[slot(1, v, i)] = acc_s[v][i] * e;
          }
        }
    }
    __syncthreads();
    if (wv >= 2) {
#pragma unroll
      for (int v = 0; v < NMT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PK) {
            if (role < 2) reg[slot(role, v, i)] += acc_r[v][i] * e;
          } else {
            reg[slot(0, v, i)] += acc_r[v][i] * e;
            reg[slot(1, v, i)] += acc_s[v][i] * e;
          }
        }
    }
    __syncthreads();
    // write the partial of every valid head: [max (log2 domain), sum, acc_rot[D], acc_sk[D]]
    const int nh = a.group - hblk * HB < HB ? a.group - hblk * HB : HB;
    for (int e2 = tid; e2 < nh * (2 + 2 * D); e2 += 256) {
      const int h = e2 / (2 + 2 * D), k = e2 % (2 + 2 * D);
      float val;
      if (k < 2) {
        float Mh = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_m[w][h]);
        val = k == 0 ? Mh : s_lw[0][h] + s_lw[1][h] + s_lw[2][h] + s_lw[3][h];
      } else {
        const int pt = (k - 2) / D, ch = (k - 2) % D;
        const int idx = h * HS + pt * DP + ch + 16 * (ch >> 6);
        val = s_red[idx] + s_red[REG + idx];
      }
      const int hq2 = kvh * a.group + hblk * HB + h;
      a.part[(((int64_t)b * a.hq + hq2) * a.n_split + split) * (2 + 2 * D) + k] = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Query preparation (see tq_prep_dev.h), 256 threads per block.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(tqp::PrepArgs p) {
  __shared__ __align__(16) unsigned char smem[tqp::prep_lds_bytes<D>()];
  tqp::prep_block<D, 256>(p, blockIdx.x, blockIdx.y, threadIdx.x, smem);
}

// ---------------------------------------------------------------------------
// Split merge and back-transform, kCombCols blocks per query head:
//   M = max_s m_s, w_s = 2^(m_s - M), L = sum_s w_s l_s, acc = sum_s w_s acc_s,
//   out = (rot^T acc_rot + sketch^T (alpha_g acc_sk)) / L.
// Every block of a head forms the whole merged accumulator (the partials are
// read by each of them) and back-transforms one slice of D / kCombCols
// outputs, so a block pulls only that slice's columns of rot and sketch
// through its compute unit (the matrices are the larger part of the bytes).
// ---------------------------------------------------------------------------
constexpr int kMaxSplit = 1024;

// NTHR threads per block: 1024 for a few heads (the split sums cut four ways
// across thread groups and the back-transform 32 ways, rows of [rot;
// sketch], both finished through LDS), 256 for many heads (chunks of query
// tokens, large batches), where more blocks resident per compute unit
// overlap more heads' chains of dependent reductions.
constexpr int kCombThreads = 1024;
constexpr int kCombThreadsMany = 256;
constexpr int kCombManyHeads = 128;  // more heads than this: the 256-thread blocks
constexpr int kCombCols = 4;

// Heads are ordered (batch, q head, query token); out rows are (batch, query
// token, q head) (the same order when T = 1).
template <int D, int NTHR>
__global__ __launch_bounds__(NTHR) void combine_kernel(const float* part, int n_split,
                                                               const float* rot, const float* sketch,
                                                               int group_dim0, int T, int hq, float* out) {
  constexpr int NW = NTHR / 64, NG = NTHR / (2 * D);  // waves, groups
  constexpr int PS = 2 + 2 * D;                                      // floats per partial
  constexpr int OC = D / kCombCols;                                  // outputs per block
  constexpr int RP = NTHR / OC;                              // row parts of [rot; sketch]
  constexpr int JR = 2 * D / RP;                                     // rows per part
  static_assert(JR * RP == 2 * D && D % JR == 0 && NG >= 1, "combine shape");
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_part[NG][2 * D];
  __shared__ float s_acc[2 * D];
  __shared__ float s_red[NW];
  __shared__ float s_out[RP][OC + 1];
  const int head = blockIdx.x;
  const int cs = blockIdx.y;  // output slice
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const float* P = part + (int64_t)head * n_split * PS;
  // this thread's back-transform operands (no dependence on the merge, so
  // their loads overlap it): output i = cs OC + t % OC, rows
  // [JR r, JR r + JR) of [rot; sketch] with r = t / OC
  const int io = t % OC, rp = t / OC;
  const int i = cs * OC + io;
  const int j0 = JR * rp;
  const float* mat = (j0 < D ? rot + (int64_t)j0 * D : sketch + (int64_t)(j0 - D) * D) + i;
  float mv[JR];
#pragma unroll
  for (int j = 0; j < JR; ++j) mv[j] = mat[(int64_t)j * D];
  // max over splits (log2 domain)
  float mx = -INFINITY;
  for (int s = t; s < n_split; s += NTHR) mx = fmaxf(mx, P[(int64_t)s * PS]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();
  // split weights and the total sum
  float lsum = 0.f;
  for (int s = t; s < n_split; s += NTHR) {
    const float ms = P[(int64_t)s * PS];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    s_w[s] = w;
    lsum += w * P[(int64_t)s * PS + 1];
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  if (lane == 0) s_red[wv] = lsum;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += s_red[w];
  // merged accumulators: group g sums the splits s = g (mod NG)
  {
    const int c = t % (2 * D), g = t / (2 * D);
    float acc = 0.f;
#pragma unroll 8
    for (int s = g; s < n_split; s += NG) acc = fmaf(s_w[s], P[(int64_t)s * PS + 2 + c], acc);
    s_part[g][c] = acc;
  }
  __syncthreads();
  if (t < 2 * D) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc += s_part[g][t];
    if (t >= D) {  // alpha_g on the sketch half
      const int j = t - D;
      const int dg = j < group_dim0 ? group_dim0 : D - group_dim0;
      acc *= 1.2533141373155003f / (float)dg;
    }
    s_acc[t] = acc;
  }
  __syncthreads();
  // back-transform of this block's outputs: out[i] = sum over the rows j of
  // [rot; sketch] of M[j][i] acc[j], cut into RP parts of JR rows
  {
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < JR; ++j) o = fmaf(mv[j], s_acc[j0 + j], o);
    s_out[rp][io] = o;
  }
  __syncthreads();
  if (t < OC) {
    float o = 0.f;
#pragma unroll 8
    for (int r = 0; r < RP; ++r) o += s_out[r][t];
    const int64_t orow = T <= 1 ? head : ((int64_t)(head / T / hq) * T + head % T) * hq + (head / T) % hq;
    out[orow * D + cs * OC + t] = o / L;
  }
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

// query tokens per head of a shape
inline int q_tokens(const tq_decode_shape* s) { return s->n_q_tokens < 1 ? 1 : s->n_q_tokens; }

bool shape_valid(const tq_decode_shape* s) {
  if (!s) return false;
  if (s->n_q_tokens < 0 || q_tokens(s) > s->n_ctx) return false;
  // (prepared heads per launch column of the prep grid: at most 65535 x 64)
  if ((int64_t)s->batch * s->n_q_heads * q_tokens(s) > (int64_t)65535 * 64) return false;
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

// workspace: [prepared queries][K codebook scales, 2 floats][split partials]
size_t workspace_for(const tq_decode_shape* s, int d, bool with_v, int n_split) {
  const size_t heads = (size_t)s->batch * s->n_q_heads * q_tokens(s);
  size_t bytes = align256(heads * 3 * d * sizeof(_Float16)) + 256;
  if (with_v) bytes += align256(heads * (size_t)n_split * (2 + 2 * d) * sizeof(float));
  return bytes;
}

// heads per workgroup: 4 (packed columns) for KV groups of at most 4 query
// heads with V, else 16
inline int heads_per_block(int group, bool with_v) { return with_v && group <= 4 ? 4 : 16; }

template <int D, int NG, int M0, int M1, int WV>
hipError_t launch_decode(const DArgs& a, int n_hblk, hipStream_t st) {
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv), (unsigned)n_hblk);
  if constexpr (WV != 0) {
    if (heads_per_block(a.group, WV != 0) == 4)
      hipLaunchKernelGGL((decode_kernel<D, NG, M0, M1, WV, 4>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<D, NG, M0, M1, WV, 16>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, NG, M0, M1, WV, 16>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int NG, int M0, int WV>
hipError_t dispatch_m1(const DArgs& a, int m1, int n_hblk, hipStream_t st) {
  switch (m1) {
    case 1: return launch_decode<D, NG, M0, 1, WV>(a, n_hblk, st);
    case 2: return launch_decode<D, NG, M0, 2, WV>(a, n_hblk, st);
    case 3: return launch_decode<D, NG, M0, 3, WV>(a, n_hblk, st);
    default: return launch_decode<D, NG, M0, 4, WV>(a, n_hblk, st);
  }
}

template <int D, int NG, int WV>
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
  const int grp = shape->n_q_heads / shape->n_kv_heads * q_tokens(shape);
  const int hb = heads_per_block(grp, vq != nullptr);
  const int n_hblk = (grp + hb - 1) / hb;
  *bytes = workspace_for(shape, kq->layout.d, vq != nullptr, choose_split(shape, n_hblk));
  return TQ_OK;
}

namespace {

// Everything a decode call launches, validated and laid out in the workspace.
struct Plan {
  DArgs a;
  tqp::PrepArgs prep;
  int n_hblk, prep_grid_y, n_heads, n_groups, m0, m1, group_dim0, T, hq_orig;
  bool with_v, v_mse;  // V records present; V records without sign bits
  const float* vrot;
  const float* vsketch;
  float* out;
};

constexpr int kD = 128;  // the decode kernels' dimension

tq_status plan_decode(const tq_quantizer* kq, const tq_quantizer* vq, const tq_decode_shape* shape,
                      const void* q, tq_dtype q_dtype, const tq_cache* k_cache, const tq_cache* v_cache,
                      float* logits, float* out, void* workspace, size_t workspace_bytes, Plan* pl,
                      const tq_paging* paging = nullptr) {
  if (!tq::quantizer_pointers_valid(kq) || !shape_valid(shape)) return TQ_ERR_INVALID;
  if (paging && (!paging->block_table || paging->max_blocks < 1 ||
                 reinterpret_cast<uintptr_t>(paging->block_table) % 4 != 0 ||
                 reinterpret_cast<uintptr_t>(paging->seq_lens) % 4 != 0 ||
                 shape->cache_capacity != (int64_t)kTile * paging->max_blocks))
    return TQ_ERR_INVALID;
  if (vq && !tq::quantizer_pointers_valid(vq)) return TQ_ERR_INVALID;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID;
  if (!q || reinterpret_cast<uintptr_t>(q) % 16 != 0) return TQ_ERR_INVALID;
  if (!k_cache || !k_cache->codes || !k_cache->signs || !k_cache->norms) return TQ_ERR_INVALID;
  // (keys need the sign bits: the logits are the unbiased two-stage estimate)
  if (kq->layout.mse_only) return TQ_ERR_UNSUPPORTED;
  // (paged: at least one physical block of every KV head)
  const int64_t rows_needed =
      paging ? (int64_t)shape->n_kv_heads * kTile : (int64_t)shape->batch * shape->n_kv_heads * shape->cache_capacity;
  if (k_cache->n_rows < rows_needed) return TQ_ERR_INVALID;
  const bool with_v = vq != nullptr;
  if (with_v) {
    if (!v_cache || !v_cache->codes || (!v_cache->signs && !vq->layout.mse_only) || !v_cache->norms)
      return TQ_ERR_INVALID;
    if (v_cache->n_rows < rows_needed || !out) return TQ_ERR_INVALID;
    if (!same_layout(kq->layout, vq->layout)) return TQ_ERR_UNSUPPORTED;
  } else {
    if (!logits || out) return TQ_ERR_INVALID;
  }
  const void* ptrs[] = {k_cache->codes, k_cache->signs, k_cache->norms, logits, out, workspace,
                        with_v ? (const void*)v_cache->codes : nullptr,
                        with_v ? (const void*)v_cache->signs : nullptr,
                        with_v ? (const void*)v_cache->norms : nullptr};
  for (const void* ptr : ptrs)
    if (ptr && reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return TQ_ERR_INVALID;
  if (!decode_supported(kq->layout)) return TQ_ERR_UNSUPPORTED;
  const tq_layout& l = kq->layout;
  const int T = q_tokens(shape);
  const int group = shape->n_q_heads / shape->n_kv_heads * T;  // (q head, query token) columns per KV head
  const int hb = heads_per_block(group, with_v);
  const int n_hblk = (group + hb - 1) / hb;
  const int n_split = choose_split(shape, n_hblk);
  const size_t need = workspace_for(shape, l.d, with_v, n_split);
  if (!workspace || workspace_bytes < need) return TQ_ERR_WORKSPACE;

  constexpr int D = kD;
  const int n_heads = shape->batch * shape->n_q_heads * T;
  _Float16* qprep = reinterpret_cast<_Float16*>(workspace);
  float* kscale = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                           align256((size_t)n_heads * 3 * D * sizeof(_Float16)));
  float* part = kscale + 64;

  *pl = Plan{};
  pl->n_hblk = n_hblk;
  pl->n_heads = n_heads;
  pl->n_groups = l.n_groups;
  pl->m0 = l.mse_bits[0];
  pl->m1 = l.n_groups == 2 ? l.mse_bits[1] : 0;
  pl->group_dim0 = l.n_groups == 2 ? l.group_dim[0] : D;
  pl->with_v = with_v;
  pl->v_mse = with_v && vq->layout.mse_only;
  pl->out = out;
  pl->prep_grid_y = (n_heads + tqp::kPrepHeads - 1) / tqp::kPrepHeads;
  tqp::PrepArgs& pp = pl->prep;
  pp.q = q;
  pp.q_bf16 = q_dtype == TQ_BF16;
  pp.n_heads = n_heads;
  pp.rot = kq->rot;
  pp.sketch = kq->sketch;
  pp.scale_l2 = shape->scale * kLog2e;
  pp.group_dim0 = pl->group_dim0;
  pp.qprep = qprep;
  pp.kcent = kq->centroids;
  pp.n_groups = l.n_groups;
  pp.m0 = pl->m0;
  pp.m1 = pl->m1;
  pp.kscale = kscale;
  pp.T = T;
  pp.hq = shape->n_q_heads;
  pl->T = T;
  pl->hq_orig = shape->n_q_heads;

  DArgs& a = pl->a;
  a.batch = shape->batch;
  a.hq = shape->n_q_heads * T;
  a.T = T;
  a.hkv = shape->n_kv_heads;
  a.group = group;
  a.n_split = n_split;
  a.n_ctx = shape->n_ctx;
  a.cap = shape->cache_capacity;
  a.scale = shape->scale;
  a.qprep = qprep;
  a.kscale = kscale;
  a.kc = k_cache->codes;
  a.ks = k_cache->signs;
  a.kn = k_cache->norms;
  a.kn_f16 = l.norm_f16;
  a.kn_shift = (l.n_groups == 2 ? 3 : 2) + (l.norm_f16 ? 0 : 1);  // 2 n_groups values of 2 or 4 bytes
  a.kcent = kq->centroids;
  if (with_v) {
    a.vc = v_cache->codes;
    a.vs = v_cache->signs;
    a.vn = v_cache->norms;
    a.vn_f16 = vq->layout.norm_f16;
    a.vn_shift = (l.n_groups == 2 ? 3 : 2) + (vq->layout.norm_f16 ? 0 : 1);
    a.vcent = vq->centroids;
    pl->vrot = vq->rot;
    pl->vsketch = vq->sketch;
  }
  a.logits = logits;
  a.part = part;
  if (paging) {
    a.block_table = paging->block_table;
    a.seq_lens = paging->seq_lens;
    a.max_blocks = paging->max_blocks;
    int64_t nb = k_cache->n_rows / ((int64_t)kTile * shape->n_kv_heads);
    if (with_v) {
      const int64_t nv = v_cache->n_rows / ((int64_t)kTile * shape->n_kv_heads);
      nb = nv < nb ? nv : nb;
    }
    a.n_pblocks = nb;
  }
  return TQ_OK;
}

tq_status run_phases(const Plan& pl, unsigned phases, hipStream_t st) {
  constexpr int D = kD;
  if (phases & TQ_PHASE_PREP) {
    (void)hipGetLastError();  // a launch error is reported below, not an older one
    hipLaunchKernelGGL((prep_kernel<D>), dim3(tqp::prep_blocks_x<D>(), pl.prep_grid_y), dim3(256), 0, st,
                       pl.prep);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  }
  if (phases & TQ_PHASE_SPLIT) {
    hipError_t e;
    if (pl.n_groups == 1)
      e = !pl.with_v  ? dispatch_m0<D, 1, 0>(pl.a, pl.m0, 0, pl.n_hblk, st)
          : pl.v_mse ? dispatch_m0<D, 1, 2>(pl.a, pl.m0, 0, pl.n_hblk, st)
                     : dispatch_m0<D, 1, 1>(pl.a, pl.m0, 0, pl.n_hblk, st);
    else
      e = !pl.with_v  ? dispatch_m0<D, 2, 0>(pl.a, pl.m0, pl.m1, pl.n_hblk, st)
          : pl.v_mse ? dispatch_m0<D, 2, 2>(pl.a, pl.m0, pl.m1, pl.n_hblk, st)
                     : dispatch_m0<D, 2, 1>(pl.a, pl.m0, pl.m1, pl.n_hblk, st);
    if (e != hipSuccess) return TQ_ERR_DEVICE;
  }
  if (pl.with_v && (phases & TQ_PHASE_COMBINE)) {
    (void)hipGetLastError();  // a launch error is reported below, not an older one
    if (pl.n_heads > kCombManyHeads)
      hipLaunchKernelGGL((combine_kernel<D, kCombThreadsMany>), dim3(pl.n_heads, kCombCols), dim3(kCombThreadsMany),
                         0, st, pl.a.part, pl.a.n_split, pl.vrot, pl.vsketch, pl.group_dim0, pl.T, pl.hq_orig, pl.out);
    else
      hipLaunchKernelGGL((combine_kernel<D, kCombThreads>), dim3(pl.n_heads, kCombCols), dim3(kCombThreads), 0, st,
                         pl.a.part, pl.a.n_split, pl.vrot, pl.vsketch, pl.group_dim0, pl.T, pl.hq_orig, pl.out);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Fused appends + query preparation: the blocks of one launch quantize the
// new K vectors, then the new V vectors, then run the query preparation (the
// three are independent, so their latencies overlap).
// ---------------------------------------------------------------------------
constexpr int kStepKP = 128, kStepNT = 8;  // quantize shape for d = 128

struct StepArgs {
  tqq::QArgs k, v;
  int nk, nv;  // blocks given to the K and V appends (0 = none)
  int k_small, v_small;  // append takes the one-block-per-vector path
  tqp::PrepArgs prep;
  int prep_x;  // prep blocks along x; the prep blocks are laid out x-major
};

// SMALL: every append takes the few-vector path (a smaller kernel without the
// tile path, which is the usual decode step of one token per head).
template <bool SMALL>
__global__ __launch_bounds__(kStepNT * 64) void step_kernel(StepArgs s) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  if (b < s.nk + s.nv) {
    const bool is_k = b < s.nk;
    if (SMALL || (is_k ? s.k_small : s.v_small))
      tqq::quantize_small<kStepNT * 64>(is_k ? s.k : s.v, is_k ? b : b - s.nk, smem);
    else if constexpr (!SMALL)
      tqq::quantize_tiles<kStepKP, kStepNT>(is_k ? s.k : s.v, is_k ? b : b - s.nk, is_k ? s.nk : s.nv, smem);
  } else {
    const int pb = b - s.nk - s.nv;
    tqp::prep_block<kD, kStepNT * 64>(s.prep, pb % s.prep_x, pb / s.prep_x, threadIdx.x, smem);
  }
}

}  // namespace

extern "C" tq_status tq_attn_decode_phases(unsigned phases, const tq_quantizer* kq,
                                           const tq_quantizer* vq, const tq_decode_shape* shape,
                                           const void* q, tq_dtype q_dtype, const tq_cache* k_cache,
                                           const tq_cache* v_cache, float* logits, float* out,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  if (phases == 0 || (phases & ~(unsigned)TQ_PHASE_ALL) != 0) return TQ_ERR_INVALID;
  Plan pl;
  const tq_status st = plan_decode(kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out, workspace,
                                   workspace_bytes, &pl);
  if (st != TQ_OK) return st;
  return run_phases(pl, phases, reinterpret_cast<hipStream_t>(stream));
}

extern "C" tq_status tq_attn_decode_append(const tq_quantizer* kq, const tq_quantizer* vq,
                                           const tq_decode_shape* shape, const tq_append* k_new,
                                           const tq_append* v_new, const void* q, tq_dtype q_dtype,
                                           const tq_cache* k_cache, const tq_cache* v_cache,
                                           float* logits, float* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  Plan pl;
  tq_status st = plan_decode(kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out, workspace,
                             workspace_bytes, &pl);
  if (st != TQ_OK) return st;
  if (v_new && !vq) return TQ_ERR_INVALID;
  StepArgs sa{};
  bool k_empty = true, v_empty = true;
  if (k_new) {
    st = tqq::make_qargs(kq, TQ_TOKEN_MAJOR, k_new->x, k_new->dtype, k_new->n_vec, k_new->x_row_stride,
                         &k_new->rows, k_cache, &sa.k, &k_empty);
    if (st != TQ_OK) return st;
  }
  if (v_new) {
    st = tqq::make_qargs(vq, TQ_BLOCK32, v_new->x, v_new->dtype, v_new->n_vec, v_new->x_row_stride,
                         &v_new->rows, v_cache, &sa.v, &v_empty);
    if (st != TQ_OK) return st;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (tqq::quantize_kp(kq->layout.d) != kStepKP) return TQ_ERR_UNSUPPORTED;
  // blocks per append: every tile of an append gets its own block, up to one
  // round of the machine
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) n_cu = v;
  }
  // (a few vectors: one block per vector, as tq_quantize does for them)
  sa.k_small = !k_empty && tqq::small_path_ok(sa.k);
  sa.v_small = !v_empty && tqq::small_path_ok(sa.v);
  sa.nk = k_empty ? 0 : sa.k_small ? (int)sa.k.n_vec : (int)(sa.k.n_tiles < n_cu ? sa.k.n_tiles : n_cu);
  sa.nv = v_empty ? 0 : sa.v_small ? (int)sa.v.n_vec : (int)(sa.v.n_tiles < n_cu ? sa.v.n_tiles : n_cu);
  sa.prep = pl.prep;
  sa.prep_x = tqp::prep_blocks_x<kD>();
  const int grid = sa.nk + sa.nv + sa.prep_x * pl.prep_grid_y;
  using L = tqq::Lds<kStepKP, kStepNT>;
  constexpr int lds_small = tqp::prep_lds_bytes<kD>() > tqq::SmallLds<kStepNT * 64>::bytes
                                ? tqp::prep_lds_bytes<kD>()
                                : tqq::SmallLds<kStepNT * 64>::bytes;
  constexpr int lds = L::bytes > lds_small ? L::bytes : lds_small;
  const bool all_small = (k_empty || sa.k_small) && (v_empty || sa.v_small);
  const void* fn = all_small ? reinterpret_cast<const void*>(&step_kernel<true>)
                             : reinterpret_cast<const void*>(&step_kernel<false>);
  const int lds_use = all_small ? lds_small : lds;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_use) != hipSuccess)
    return TQ_ERR_DEVICE;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  if (all_small)
    hipLaunchKernelGGL(step_kernel<true>, dim3(grid), dim3(kStepNT * 64), lds_use, hs, sa);
  else
    hipLaunchKernelGGL(step_kernel<false>, dim3(grid), dim3(kStepNT * 64), lds_use, hs, sa);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
  return run_phases(pl, TQ_PHASE_SPLIT | TQ_PHASE_COMBINE, hs);
}

extern "C" tq_status tq_attn_decode_paged(const tq_quantizer* kq, const tq_quantizer* vq,
                                          const tq_decode_shape* shape, const tq_paging* paging,
                                          const void* q, tq_dtype q_dtype, const tq_cache* k_cache,
                                          const tq_cache* v_cache, float* logits, float* out,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!paging) return TQ_ERR_INVALID;
  Plan pl;
  const tq_status st = plan_decode(kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out, workspace,
                                   workspace_bytes, &pl, paging);
  if (st != TQ_OK) return st;
  return run_phases(pl, TQ_PHASE_ALL, reinterpret_cast<hipStream_t>(stream));
}

extern "C" tq_status tq_attn_decode(const tq_quantizer* kq, const tq_quantizer* vq,
                                    const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                                    const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return tq_attn_decode_phases(TQ_PHASE_ALL, kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out,
                               workspace, workspace_bytes, stream);
}
