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
//              each stored as an fp16 hi/lo pair), both scaled by
//              scale * log2(e) and q_sk also by alpha_g.
//  2. split:   split-K over the context. A workgroup takes one (batch, KV
//              head, block of query heads) and a range of 32-token tiles;
//              its waves take alternate tiles. Three kernels share this
//              structure: the byte-table kernel (one group of code width
//              1, 2 or 4, d = 128; 12 waves, 8 for width 4), the general
//              kernel below (4 waves; described here) and the chunk kernel for many query
//              columns per KV head. Per tile a wave of the general kernel
//              - expands the K codes through an LDS table of pairs of fp16
//                scaled centroids fp16(s c) (one scale s per codebook, its
//                1/s applied with the token's norm) and the K sign bits
//                through a nibble table into fp16 +-1,
//              - forms both logit parts on v_mfma_f32_16x16x32_f16 (tokens x
//                channels times channels x heads), with the rotated query
//                as an fp16 hi/lo pair so the MSE part keeps fp32-grade
//                accuracy; scales them by the tokens' norms and runs the
//                online softmax (accumulators are rescaled only when a
//                head's running maximum moves),
//              - expands the V codes and signs the same way and accumulates
//                sum_t p_t n_t c[idx_t] and sum_t p_t gamma_t z_t on MFMA
//                (channels x tokens times tokens x heads): V is summed in
//                the rotated and sketch domains, never dequantized per
//                token.
//              The MFMA output layout of the logits (lane = head, 8 tokens)
//              is exactly the operand layout the V product needs, so the
//              softmax weights never leave registers. The four waves merge
//              through LDS into one partial (max, sum, accumulators).
//              In the packed mode (at most 4 query heads per KV head) the
//              softmax weights, like the queries, are an fp16 part and its
//              remainder; the 16-head mode takes plain fp16 weights.
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
#include <mutex>
#include <type_traits>

#include "tq_internal.h"
#include "tq_prep_dev.h"
#include "tq_quantize_dev.h"
#include "tq_quantize_t_dev.h"
#include "tq_quantize_p_dev.h"
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
// offset of the split-K kernels' log2-domain softmax argument: their weights
// are exp2(logit - reference + kTOff), and their V norms carry 2^-kTOff
constexpr float kTOff = 96.0f;
constexpr int kWaves = 4;
constexpr int kTile = 32;

struct DArgs {
  int batch, hq, hkv, group;  // group = hq / hkv (heads here are (q head, query token) pairs)
  int n_split;
  int T;  // query tokens per head: column hloc is token hloc % T, causal past n_ctx - T + t
  int64_t n_ctx, cap;
  float scale;
  const _Float16* qprep;  // [batch*hq][4d]: q_rot hi, q_rot lo * 2^11, q_sk hi, q_sk lo * 2^11
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

// Weight operand of a column: w split into an fp16 part (its leading 11
// bits, exact in fp16 for normal magnitudes) and the remainder times 2^11;
// (bsel, csel) = (0, 1) gives the leading part, (2^11, -2^11) the remainder.
__device__ __forceinline__ float wsplit(float w, float bsel, float csel) {
  const float hi = __uint_as_float(__float_as_uint(w) & 0xFFFFE000u);
  return fmaf(bsel, w, csel * hi);
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

// DPP move whose pattern sends every lane a value from inside its row
// (rotations, quad permutations, row broadcasts): no lane keeps its old value.
template <int CTRL>
__device__ __forceinline__ float dpp_full(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// max over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48): swap the
// 32-lane halves, then odd and even rows, with v_permlane{32,16}_swap. IEEE
// maximum (v_maximum3_f32 on gfx950: no canonicalizing moves), for values
// that are never NaN.
__device__ __forceinline__ float rows4_maximum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// sum over the four 16-lane rows (the same exchange)
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
// (at least two workgroups of 256 threads per compute unit: a register
// budget of 256 per lane, which the packed mode's hi / lo columns need
// without spills)
#ifndef TQ_PK_MINB
#define TQ_PK_MINB 2
#endif
template <int D, int NG, int M0, int M1, int WV, int HB>
__global__ __launch_bounds__(256, TQ_PK_MINB) void decode_kernel(DArgs a) {
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
    // V centroids likewise as fp16(s_g c) with the V group's scale (divided
    // out when the partial is written)
    if constexpr (WV != 0) cent_v = a.vcent[tc] * a.kscale[2 + (NG > 1 && tc >= (1 << M0) ? 1 : 0)];
  }
  // ---- this lane's head and its query operands (B operand: channels x heads) ----
  // (loaded before the first tile: loads complete in issue order, so using
  // them then does not wait for the tile)
  // packed: column ln = 4 head + role, the four columns of a head in one
  // lane quad; K roles 0 q_rot hi, 1 q_rot lo, 2 q_sk hi, 3 q_sk lo; V roles
  // 0 p n hi, 1 p gamma hi (sign product), 2 p n lo, 3 p gamma lo
  const int role = PK ? ln & 3 : 0;
  const int hcol = PK ? ln >> 2 : ln;  // head of this lane's column within the block
  const int hloc = hblk * HB + hcol;  // head index within the KV group
  const bool hvalid = hloc < a.group;
  const int hq = kvh * a.group + hloc;
  u32x4 qr[NC], qrl[PK ? 1 : NC], qs[NC];  // packed: qr = B of the code product, qs = B of the sign product
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int g = c / CPG, cl = c % CPG;
    const _Float16* qp = a.qprep + ((int64_t)b * a.hq + (hvalid ? hq : 0)) * (4 * D) + g * DG + 8 * CPG * lg + 8 * cl;
    if constexpr (PK) {
      const u32x4 z{0, 0, 0, 0};
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + role * D);
      // the lo roles take the remainder at its own scale (lo * 2^11 times
      // 2^-11; small remainders become fp16 subnormals, exact to 2^-25), so
      // a head's four columns add without factors
      if (role & 1) v = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, v) * (_Float16)0x1p-11f);
      qr[c] = hvalid && role < 2 ? v : z;
      qs[c] = hvalid && role >= 2 ? v : z;
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
  // values that follow from the running reference, recomputed only when it
  // moves: the softmax offset this lane folds into its logit sum (packed:
  // the role-0 lane only, the quad adding its four parts) and the
  // running-max threshold above which the reference moves
  float t_offc = 0.f, thr = -INFINITY;
  auto ref_vals = [&]() __attribute__((always_inline)) {
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    const float t_off = (WV != 0 ? kTOff : 0.f) - m_ref;
    t_offc = (PK && role != 0) ? 0.f : t_off;
    thr = m_run == -INFINITY ? -INFINITY : kTOff;
  };
  ref_vals();
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
        // (packed: K norms as [2 NG][32], part-major, so a lane reads the
        // 8 values of its column's part as two 16-byte words)
        const int fk = lane * NG + e;
        const int ik = PK ? (fk % (2 * NG)) * kTile + fk / (2 * NG) : fk;
        s_nrm[wv][0][ik] = nok ? norm_value(r.kn[e], no.ksh[e], a.kn_f16) * kn_mul[e] : 0.f;
        // (V norms times 2^-kTOff: the weights exp2(t) carry 2^kTOff)
        if constexpr (WV != 0) s_nrm[wv][1][ik] = nok ? norm_value(r.vn[e], no.vsh[e], a.vn_f16) * 0x1p-96f : 0.f;
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
    float l2[8];
    if constexpr (PK) {
      // each lane scales its column by its part's norm (n for the code
      // columns, gamma for the sign columns), sums the groups, and the quad
      // adds its four columns by two DPP-folded adds: every lane of the quad
      // forms the same logit (the sums only commute between lanes)
      float kf[NG][8];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const f32x4* kp = reinterpret_cast<const f32x4*>(&s_nrm[wv][0][(2 * g + (role >> 1)) * kTile + 8 * lg]);
        const f32x4 x0 = kp[0], x1 = kp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[g][e] = x0[e];
          kf[g][4 + e] = x1[e];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tau = j >> 2, i = j & 3;
        float c = fmaf(lr[tau][0][i], kf[0][j], t_offc);
#pragma unroll
        for (int g = 1; g < NG; ++g) c = fmaf(lr[tau][g][i], kf[g][j], c);
        c = c + dpp_full<0xB1>(c);  // quad_perm [1, 0, 3, 2]
        l2[j] = c + dpp_full<0x4E>(c);  // quad_perm [2, 3, 0, 1]
      }
    } else {
      float kn[8][2 * NG];
      load_norms<NG>(&s_nrm[wv][0][8 * lg * 2 * NG], kn);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tau = j >> 2, i = j & 3;
        // (the prepared queries carry scale * log2(e), and alpha_g on the
        // sketch part, so this is the logit in the log2 domain)
        float s = t_offc;
#pragma unroll
        for (int g = 0; g < NG; ++g)
          s = fmaf(kn[j][2 * g + 1], ls[tau][g][i], fmaf(kn[j][2 * g], fmaf(kLoInv, lrl[tau][g][i], lr[tau][g][i]), s));
        l2[j] = s;
      }
    }
    // tokens of the tile before n_ctx (32 except in the last tile)
    const int nvt = full ? kTile : (int)(N - T0);
    // a chunk of T query tokens: this column's token t sees [0, N - T + t]
    if (a.T > 1) {
      const int64_t lim = N - a.T + hloc % a.T + 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) l2[j] = tok0 + j < lim ? l2[j] : -INFINITY;
    }
    // (packed: the four lanes of a head's quad hold the same logits; the
    // role-0 lane stores them)
    if (a.logits) {
      if (hvalid && role == 0) {
        const float t_off = (WV != 0 ? kTOff : 0.f) - (m_run == -INFINITY ? 0.f : m_run);
        float* lp = a.logits + ((int64_t)b * a.hq + hq) * a.n_ctx + tok0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * lg + j < nvt) lp[j] = (l2[j] - t_off) * kLn2;
      }
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) l2[j] = 8 * lg + j < nvt ? l2[j] : -INFINITY;
    }
    if constexpr (WV != 0) {
      // ---------------- online softmax ----------------
      // (IEEE maximum: no NaN arises here, and it takes no canonicalizing moves)
      float mx = l2[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = __builtin_elementwise_maximum(mx, l2[j]);
      mx = rows4_maximum(mx);
      // The reference is kept at an integer (log2 domain), and the logit sums
      // carry the offset kTOff - m_ref (l2 = logit - m_ref + kTOff, in
      // [64, 128) for |logit - m_ref| < 32, where fp32 values sit on the
      // fixed grid 2^-17): every weight and every rescale is then an exact
      // power of two times the same mantissa, so the fp16 weights, and hence
      // the result, do not depend on how the context is split. A head's
      // candidate m_ref + ceil(mx) - kTOff exceeds m_run exactly when mx
      // exceeds the threshold.
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        // some head's maximum moved: rescale (factor 1 for the others; a
        // head that has seen only masked tokens keeps -inf and factor 1)
        const float m_ref0 = m_run == -INFINITY ? 0.f : m_run;
        const float m_new = fmaxf(m_run, m_ref0 + (ceilf(mx) - kTOff));
        const float corr = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
        if constexpr (PK) {
#pragma unroll
          for (int v = 0; v < NMT; ++v) acc_r[v] *= corr;
        } else {
#pragma unroll
          for (int v = 0; v < NMT; ++v) {
            acc_r[v] *= corr;
            acc_s[v] *= corr;
          }
        }
        m_run = m_new;
        // the sums relative to the new reference (m_run is -inf only while
        // every token seen is masked: then they stay -inf and p = 0)
        const float delta = m_run == -INFINITY ? 0.f : m_run - m_ref0;
#pragma unroll
        for (int j = 0; j < 8; ++j) l2[j] -= delta;
        ref_vals();
      }
      float p[8], psum;
      // (exp2(l2) <= 2^kTOff)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(l2[j]);
        psum = j == 0 ? p[j] : psum + p[j];
      }
      l_run += psum;  // (in units of 2^kTOff)
      // B operands of the V product: slot j <-> token 8 lg + j
      u32x4 pr[NG], pz[NG];
      if constexpr (PK) {
        // column roles of the V products: the leading fp16 part of p n (0)
        // and its remainder times 2^11 (2) for the code product, the same
        // of p gamma (1, 3) for the sign product
        const float* pp = p;
        const bool rem = role >= 2;
        const float bsel = rem ? 2048.0f : 0.0f, csel = rem ? -2048.0f : 1.0f;
        const u32x4 z{0, 0, 0, 0};
        const bool r1 = (role & 1) != 0;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          // this column's part (n or gamma) of the lane's 8 tokens, read
          // directly from the part-major staging (a select between two
          // register arrays would be folded into a lane-dependent index,
          // which the compiler places in scratch memory)
          const f32x4* vp = reinterpret_cast<const f32x4*>(&s_nrm[wv][1][(2 * g + (r1 ? 1 : 0)) * kTile + 8 * lg]);
          const f32x4 x0 = vp[0], x1 = vp[1];
          const float vs8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = h2bits(wsplit(pp[2 * q] * vs8[2 * q], bsel, csel), wsplit(pp[2 * q + 1] * vs8[2 * q + 1], bsel, csel));
          pr[g] = r1 ? z : w;
          pz[g] = r1 ? w : z;
        }
      } else {
        float vn[8][2 * NG];
        load_norms<NG>(&s_nrm[wv][1][8 * lg * 2 * NG], vn);
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
    l_run = rows4_sum(l_run) * 0x1p-96f;  // back from units of 2^kTOff
    // (packed: every lane of a head's quad has run its softmax; the role-0
    // lane stores its maximum and sum)
    if (lg == 0 && role == 0) s_m[wv][hcol] = m_run;
    __syncthreads();
    float M = s_m[0][hcol];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][hcol]);
    const float e = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    if (lg == 0 && role == 0) s_lw[wv][hcol] = l_run * e;
    float* reg = s_red + (wv & 1) * REG + hcol * HS;
    auto slot = [&](int pt, int v, int i) {
      const int g = v / MTPG, u = v % MTPG;
      const int ch = g * DG + RUN * (4 * lg + i) + u;
      return pt * DP + ch + 16 * (ch >> 6);
    };
    if constexpr (PK) {
      // a head's remainder columns (roles 2, 3) join their leading columns
      // (roles 0, 1), two lanes down in the quad
#pragma unroll
      for (int v = 0; v < NMT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float rem = dpp_full<0xEE>(acc_r[v][i]);  // quad_perm [2, 3, 2, 3]
          acc_r[v][i] = role < 2 ? fmaf(kLoInv, rem, acc_r[v][i]) : acc_r[v][i];
        }
    }
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
    // write the partial of every valid head: [max (log2 domain), sum,
    // acc_rot[D] / s_V,g, acc_sk[D]]
    const int nh = a.group - hblk * HB < HB ? a.group - hblk * HB : HB;
    const float vinv[2] = {1.0f / a.kscale[2], NG > 1 ? 1.0f / a.kscale[3] : 1.0f};
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
        if (pt == 0) val *= vinv[NG > 1 && ch >= DG ? 1 : 0];
      }
      const int hq2 = kvh * a.group + hblk * HB + h;
      a.part[(((int64_t)b * a.hq + hq2) * a.n_split + split) * (2 + 2 * D) + k] = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Byte-table split-K kernel: one quantizer group whose code width m divides
// 8 (m = 1, 2, 4), d = 128. One workgroup per compute unit (12 waves for
// m <= 2, 8 for m = 4, whose wider code words would spill at 12) holds
// two 64 KB LDS tables of 256 rows x 256 bytes, indexed by one byte of a
// record:
//   code table  row e: the 8 / m fp16 scaled centroids fp16(s c[code]) of
//               the codes packed in byte e (K centroids in bytes [0, 128),
//               V centroids in [128, 256)), each entry replicated across
//               its half row;
//   sign table  row e: eight fp16 +-1 for the bits of e (bit 1 -> +1),
//               replicated 16 times.
// A lane reads the replica at its own offset within the row, so any mix of
// rows is read without bank conflicts between the lanes served together,
// and the LDS address of a lookup is one v_perm_b32: the record byte
// becomes address bits 8..15, the lane's replica offset bits 0..7 and the
// table base bit 16. A lane's 8 MFMA operand values of one token (K) or one
// channel (V) are m lookups of codes and one of signs.
//
// Column packing of the 16 MFMA columns:
//   HB = 8 (KV groups of more than 4 query heads, in blocks of 8 heads):
//     K codes x [q_rot hi | q_rot lo] (8 heads each; the lo parts at their
//     own scale), K signs x [q_sk hi | q_sk lo]; V codes x [w_n | 0] and
//     V signs x [0 | w_g] into one
//     accumulator set, with w_n = p n and w_g = p gamma the softmax weights
//     times the token's norms, both plain fp16 (relative rounding 2^-11 per
//     weight; a hi / lo split of w_n took 32 more accumulator registers,
//     which kept the kernel at 8 waves);
//   HB = 4 (at most 4 query heads per KV head): column 4 h + r, role r =
//     0 q_rot hi / w_n hi, 1 q_rot lo / w_n lo, 2 q_sk hi / w_g hi, 3 q_sk lo
//     / w_g lo;
//     codes and signs accumulate into the same accumulator (their B columns
//     are disjoint).
// Each column's lanes form their head's logit (exchanging the hi / lo / sketch
// parts by DPP), so every lane runs its head's online softmax.
// ---------------------------------------------------------------------------
#ifndef TQ_BYTE_NBK
#define TQ_BYTE_NBK 2
#endif
#ifndef TQ_BYTE_NBV
#define TQ_BYTE_NBV 2
#endif
// waves per workgroup for code width m (a multiple of 4)
constexpr int byte_waves(int m) { return m == 4 ? 8 : 12; }
constexpr uint32_t kBSignBase = 1u << 16;    // LDS byte offset of the sign table
constexpr int kBTabBytes = 2 << 16;          // both tables
constexpr int kBMerge = 4 * (128 * 16 + 64) * 4;  // merge regions (reuse the table space)
static_assert(kBMerge <= kBTabBytes, "merge regions fit in the table space");
// LDS layout past the tables for BW waves: per-wave norm staging [BW][2][64]
// floats, then s_m, s_lw [BW][8] floats and the centroids [2][16]
template <int BW>
struct BLds {
  static constexpr int nrm = kBTabBytes;
  static constexpr int misc = nrm + BW * 2 * 64 * 4;
  static constexpr int bytes = misc + (2 * BW * 8 + 32) * 4;
};

template <int M>
struct BTab {
  static constexpr int CPB = 8 / M;     // codes per record byte
  static constexpr int EB = 2 * CPB;    // entry bytes: CPB fp16 centroids
  static constexpr int REP = 128 / EB;  // replicas per half row
};

// LDS byte address of the table row selected by byte k of w, at the lane's
// replica offset `off` (bits 0..7) and table base (bit 16 of off).
__device__ __forceinline__ uint32_t baddr(uint32_t w, uint32_t off, int k) {
  return __builtin_amdgcn_perm(w, off, 0x0C020000u | ((4u + (uint32_t)k) << 8));
}

// Loads at an absolute LDS byte address (the kernel's dynamic LDS starts at
// address 0; the launch checks that it has no static LDS).
template <typename T>
__device__ __forceinline__ T lds_at(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>((size_t)addr);
}

// 8 codes of M bits starting at byte b of the word array w -> 8 fp16 (the A
// operand slots 0..7 in code order)
template <int M>
__device__ __forceinline__ u32x4 bcodes8(const uint32_t* w, int b, uint32_t off) {
  if constexpr (M == 1) {
    return lds_at<u32x4>(baddr(w[b >> 2], off, b & 3));
  } else if constexpr (M == 2) {
    const u32x2 x = lds_at<u32x2>(baddr(w[b >> 2], off, b & 3));
    const u32x2 y = lds_at<u32x2>(baddr(w[(b + 1) >> 2], off, (b + 1) & 3));
    return u32x4{x[0], x[1], y[0], y[1]};
  } else {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = lds_at<uint32_t>(baddr(w[(b + i) >> 2], off, (b + i) & 3));
    return r;
  }
}

// 8 sign bits in byte b of w -> 8 fp16 +-1
__device__ __forceinline__ u32x4 bsigns8(const uint32_t* w, int b, uint32_t off) {
  return lds_at<u32x4>(baddr(w[b >> 2], off, b & 3));
}




// Record words of one 32-token tile held by one lane of the byte-table
// kernel (the K rows of token rows r and r + 4, the lane's share of the
// tile's norms, and the lane's V block fields).
template <int M>
struct BRaw {
  uint32_t kc[2][M];    // K codes of the lane's 32 channels, token rows r, r + 4
  uint32_t ks[2];       // K sign words, same rows
  uint32_t kn, vn;      // word holding norm value `lane` of the tile's [32][n, gamma] (K, V)
  uint32_t vc[2 * M];   // V codes: octet lg, channels 8 ln .. 8 ln + 7
  uint32_t vs[2];       // V signs, same channels
};

template <int M, int WV, int HB>
__global__ __launch_bounds__(64 * byte_waves(M), 1) void decode_byte_kernel(DArgs a) {
  using BT = BTab<M>;
  constexpr int D = 128, NC = 4, NMT = 8;
  constexpr bool P8 = HB == 8;
  constexpr int kBW = byte_waves(M), kBThreads = 64 * kBW;
  using BL = BLds<kBW>;
  // (the kernel has no static LDS: the dynamic area starts at LDS address 0,
  // so the table addresses formed in registers are used as they are)
  extern __shared__ __align__(16) unsigned char lds[];
  float* s_nrm = reinterpret_cast<float*>(lds + BL::nrm);
  float* s_m = reinterpret_cast<float*>(lds + BL::misc);
  float* s_lw = s_m + kBW * 8;
  float* s_cent = s_lw + kBW * 8;  // [0, 16) K, [16, 32) V

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
  const uint32_t soff = kBSignBase | (16u * (lane & 15));

  int64_t N = a.n_ctx;
  if (a.seq_lens) {
    const int64_t n = a.seq_lens[b];
    N = n < 1 ? 1 : (n > a.n_ctx ? a.n_ctx : n);
  }
  // tile indices are 32-bit (wave-uniform, so their compares stay scalar)
  const int n_tiles = (int)((N + kTile - 1) / kTile);
  const int n_full = (int)(N / kTile);  // tiles whose 32 tokens all exist
  const int tps = (n_tiles + a.n_split - 1) / a.n_split;
  const int t_begin = split * tps;
  const int t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;
  const int64_t rowbase = (int64_t)bh * a.cap;
  const int npb = a.n_pblocks < INT32_MAX ? (int)a.n_pblocks : INT32_MAX;  // entries clamp into [0, npb)
  auto tile_row = [&](int t) __attribute__((always_inline)) -> int64_t {
    if (!a.block_table) return rowbase + (int64_t)t * kTile;
    // the block table is read-only during the launch: read it through the
    // constant address space, so the wave-uniform entry comes from a scalar
    // load (a vector load would make the wave wait for its prefetched tiles)
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(uintptr_t)a.block_table;
    int pb = bt[(int64_t)b * a.max_blocks + t];
    pb = pb < 0 ? 0 : (pb >= npb ? npb - 1 : pb);
    return ((int64_t)pb * a.hkv + kvh) * kTile;
  };
  // Code table rows: when the K and V scaled codebooks are equal (equal
  // layouts have equal Lloyd-Max codebooks), a row holds one entry
  // replicated across all 256 bytes and K and V read the same replica;
  // otherwise K entries fill bytes [0, 128) and V entries [128, 256).
  // (The b64 reads of m = 2 serve 32 lanes together: a full-row replica per
  // lane keeps them free of bank conflicts.)
  bool shared_tab = true;
  if constexpr (WV != 0) {
    const int L = 1 << M;
    for (int i = 0; i < L; ++i)
      shared_tab = shared_tab && a.kcent[i] * a.kscale[0] == a.vcent[i] * a.kscale[2];
  }
  const uint32_t koff = shared_tab ? BT::EB * (lane % (2 * BT::REP)) : BT::EB * (lane % BT::REP);
  const uint32_t voff = shared_tab ? koff : 128u + BT::EB * (lane % BT::REP);
  // Per-lane byte offsets inside a tile (32-bit; the tile's base addresses
  // are wave-uniform). MFMA row ln of the logit products is token row
  // 8 (ln / 4) + ln % 4 (tau = 0) or that + 4 (tau = 1), lane group lg takes
  // channels 32 lg .. 32 lg + 31, so a lane's K words of a row are M code
  // words and one sign word; its V fields are octet lg, channels 8 ln ...
  const uint32_t r0 = 8u * (ln >> 2) + (ln & 3);
  const uint32_t okc = r0 * (16u * M) + 4u * M * lg, oks = r0 * 16u + 4u * lg;
  const uint32_t okn = a.kn_f16 ? 4u * (lane >> 1) : 4u * lane;
  const uint32_t ovn = a.vn_f16 ? 4u * (lane >> 1) : 4u * lane;
  // odd lanes stage gamma (K: n / s_K on even lanes); with fp16 norms they
  // take the upper half of the shared word (a wave-constant lane mask, kept
  // in scalar registers rather than per-lane values)
  const bool odd = (lane & 1) != 0;
  auto bnorm = [&](uint32_t w, int f16) __attribute__((always_inline)) -> float {
    if (!f16) return __uint_as_float(w);
    // both halves converted, then a select on the lane mask (written so
    // that the compiler does not fold it into a per-lane shift amount,
    // which would hold one more vector register through the tile loop)
    const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)w);
    float hi;
    asm("v_cvt_f32_f16_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1" : "=v"(hi) : "v"(w));
    return odd ? hi : lo;
  };
  const uint32_t ovc = M * (128u * lg + 8u * ln), ovs = 4u * (32u * lg + 2u * ln);
  // Record loads carry the non-temporal hint (aux bit 1): the words are read
  // once. Measured on the 70B-shaped pass: 1.7% faster than plain loads,
  // although HBM reads rise from 100.4% to 102.7% of the algorithmic bytes
  // (the two row sets of a tile, tau 0 and 1, each take half of every K
  // line, and the second request sometimes finds the line gone).
  constexpr int kNT = 2;
  // Record loads go through buffer resources based at the tile's first row
  // (wave-uniform, built in scalar registers), so a load's address is the
  // lane's constant 32-bit offset above plus an immediate: no per-tile
  // vector address arithmetic.
  auto rsrc = [](const void* base) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
  };
  // K words of a tile (codes, signs, norms)
  auto load_k = [&](int64_t row0, BRaw<M>& r) __attribute__((always_inline)) {
    const auto kc = rsrc(reinterpret_cast<const char*>(a.kc) + row0 * (16 * M));
    const auto ks = rsrc(reinterpret_cast<const char*>(a.ks) + row0 * 16);
    const auto kn = rsrc(reinterpret_cast<const char*>(a.kn) + (row0 << a.kn_shift));
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      // (the second row set's constant offset goes in the scalar offset, so
      // that no per-lane register holds the sum)
      const int so = tau * 64 * M;
      if constexpr (M == 1) {
        r.kc[tau][0] = __builtin_amdgcn_raw_buffer_load_b32(kc, okc, so, kNT);
      } else if constexpr (M == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(kc, okc, so, kNT);
        r.kc[tau][0] = v[0];
        r.kc[tau][1] = v[1];
      } else {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(kc, okc, so, kNT);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.kc[tau][i] = v[i];
      }
      r.ks[tau] = __builtin_amdgcn_raw_buffer_load_b32(ks, oks, tau * 64, kNT);
    }
    r.kn = __builtin_amdgcn_raw_buffer_load_b32(kn, okn, 0, kNT);
  };
  // V words of a tile (block fields and norms)
  auto load_v = [&](int64_t row0, BRaw<M>& r) __attribute__((always_inline)) {
    if constexpr (WV != 0) {
      const int64_t blk = row0 >> 5;
      const auto vc = rsrc(reinterpret_cast<const char*>(a.vc) + blk * (512 * M));
      const auto vn = rsrc(reinterpret_cast<const char*>(a.vn) + (row0 << a.vn_shift));
      if constexpr (M == 1) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(vc, ovc, 0, kNT);
        r.vc[0] = v[0];
        r.vc[1] = v[1];
      } else {
#pragma unroll
        for (int h = 0; h < M / 2; ++h) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(vc, ovc, 16 * h, kNT);
#pragma unroll
          for (int i = 0; i < 4; ++i) r.vc[4 * h + i] = v[i];
        }
      }
      if constexpr (WV == 1) {
        const auto vs = rsrc(reinterpret_cast<const char*>(a.vs) + blk * 512);
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(vs, ovs, 0, kNT);
        r.vs[0] = v[0];
        r.vs[1] = v[1];
      }
      r.vn = __builtin_amdgcn_raw_buffer_load_b32(vn, ovn, 0, kNT);
    }
  };
  // lane l stages float l of a tile's K norms [32][n, gamma]: n / s_K
  const float kinv = 1.0f / a.kscale[0];

  // ---- this lane's column: head and role ----
  const int hcol = P8 ? (ln & 7) : (ln >> 2);  // head within the block
  const int role = P8 ? (ln >> 3) : (ln & 3);  // P8: 0 hi, 1 lo; else 0 n hi, 1 n lo, 2 gamma hi, 3 gamma lo
  const int hloc = hblk * HB + hcol;
  const bool hvalid = hloc < a.group;
  const int hq = kvh * a.group + hloc;
  u32x4 bq[NC], bs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const _Float16* qp = a.qprep + ((int64_t)b * a.hq + (hvalid ? hq : 0)) * (4 * D) + 32 * lg + 8 * c;
    const u32x4 z{0, 0, 0, 0};
    const u32x4 vh = *reinterpret_cast<const u32x4*>(qp);
    const u32x4 vl = *reinterpret_cast<const u32x4*>(qp + D);
    const u32x4 vs = *reinterpret_cast<const u32x4*>(qp + 2 * D);
    const u32x4 vsl = *reinterpret_cast<const u32x4*>(qp + 3 * D);
    // lo parts at their own scale (lo * 2^11 times 2^-11; small remainders
    // become fp16 subnormals, exact to 2^-25), so a hi and a lo column's
    // sums add without a factor
    const u32x4 slo = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, vsl) * (_Float16)0x1p-11f);
    if constexpr (P8) {
      // K codes x [q_rot hi | q_rot lo], K signs x [q_sk hi | q_sk lo]
      const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, vl) * (_Float16)0x1p-11f);
      bq[c] = hvalid ? (role ? lo : vh) : z;
      bs[c] = hvalid ? (role ? slo : vs) : z;
    } else {
      bq[c] = hvalid && role < 2 ? (role ? vl : vh) : z;
      bs[c] = hvalid && role >= 2 ? (role == 3 ? slo : vs) : z;
    }
  }
  // weight split factors of this lane's column (HB = 4: remainder columns)
  const bool wlo = (role & 1) != 0;
  const float bsel = wlo ? 2048.0f : 0.0f, csel = wlo ? -2048.0f : 1.0f;

  // ---- the first tiles in flight while the tables are built ----
  // K words are loaded NBK - 1 tiles ahead (ring of NBK buffers), V words
  // NBV - 1 tiles ahead (ring of NBV): the K part of a tile is consumed
  // first, so its words get the longer lead. Tile i of this wave uses K
  // buffer i mod NBK and V buffer i mod NBV.
  constexpr int NBK = TQ_BYTE_NBK, NBV = TQ_BYTE_NBV;
  static_assert(NBK >= 2 && NBK <= 3 && NBV >= 2 && NBV <= 3, "buffer rings of 2 or 3");
  BRaw<M> kb0, kb1, kb2, vb0, vb1, vb2;
  auto kbuf = [&](auto kc) __attribute__((always_inline)) -> BRaw<M>& {
    constexpr int k = decltype(kc)::value % NBK;
    if constexpr (k == 0) return kb0;
    else if constexpr (k == 1) return kb1;
    else return kb2;
  };
  auto vbuf = [&](auto kc) __attribute__((always_inline)) -> BRaw<M>& {
    constexpr int k = decltype(kc)::value % NBV;
    if constexpr (k == 0) return vb0;
    else if constexpr (k == 1) return vb1;
    else return vb2;
  };
  int tile = t_begin + wv;
  const int last = tile < t_end ? t_end - 1 - ((t_end - 1 - tile) % kBW) : 0;  // this wave's last tile
  // (a wave without tiles loads tile 0, which always exists, and drops it;
  // past the last tile the prefetch reloads it)
  auto ahead = [&](int k) __attribute__((always_inline)) -> int {
    if (tile >= t_end) return 0;
    return tile + k * kBW <= last ? tile + k * kBW : last;
  };
  {
    const int64_t r0 = tile_row(ahead(0));
    load_k(r0, kb0);
    load_v(r0, vb0);
    if constexpr (NBK > 2) load_k(tile_row(ahead(1)), kb1);
    if constexpr (NBV > 2) load_v(tile_row(ahead(1)), vb1);
  }
  if (tid < 16) {
    const int L = 1 << M;
    const int tc = tid < L ? tid : L - 1;
    s_cent[tid] = a.kcent[tc] * a.kscale[0];
    if constexpr (WV != 0) s_cent[16 + tid] = a.vcent[tc] * a.kscale[2];
  }
  __syncthreads();
  {
    // code table: 256 rows x 16 stores of 16 bytes (8 K, then 8 V)
    constexpr uint32_t MASK = (1u << M) - 1;
    for (int i = tid; i < 256 * 16; i += kBThreads) {
      const int e = i >> 4, k = i & 15;
      const float* cen = s_cent + (k < 8 || shared_tab ? 0 : 16);
      uint32_t wd[4];
      if constexpr (M == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) wd[j] = h2bits(cen[(e >> (2 * j)) & 1], cen[(e >> (2 * j + 1)) & 1]);
      } else if constexpr (M == 2) {
        wd[0] = wd[2] = h2bits(cen[e & MASK], cen[(e >> 2) & MASK]);
        wd[1] = wd[3] = h2bits(cen[(e >> 4) & MASK], cen[(e >> 6) & MASK]);
      } else {
        wd[0] = wd[1] = wd[2] = wd[3] = h2bits(cen[e & MASK], cen[(e >> 4) & MASK]);
      }
      *reinterpret_cast<u32x4*>(lds + e * 256 + 16 * k) = u32x4{wd[0], wd[1], wd[2], wd[3]};
    }
    // sign table: 256 rows x 16 replicas of eight fp16 +-1
    for (int i = tid; i < 256 * 16; i += kBThreads) {
      const int e = i >> 4, k = i & 15;
      uint32_t wd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wd[j] = (((e >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u) | (((e >> (2 * j + 1)) & 1) ? 0x3C000000u : 0xBC000000u);
      *reinterpret_cast<u32x4*>(lds + kBSignBase + e * 256 + 16 * k) = u32x4{wd[0], wd[1], wd[2], wd[3]};
    }
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  // values that follow from the running reference, recomputed only when it
  // moves: the softmax offset this lane folds into its logit part (8-head
  // blocks: the hi lane only) and the running-max threshold above which the
  // reference moves (ceil(max t) > kTOff, or any token while all were masked)
  float t_offc = 0.f, thr = -INFINITY;
  auto ref_vals = [&]() __attribute__((always_inline)) {
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    const float t_off = (WV != 0 ? kTOff : 0.f) - m_ref;
    t_offc = (P8 && role) ? 0.f : t_off;
    thr = m_run == -INFINITY ? -INFINITY : kTOff;
  };
  ref_vals();
  float* nrm_k = s_nrm + wv * 128;
  float* nrm_v = nrm_k + 64;
  constexpr int NVA = WV ? NMT : 1;
  f32x4 avr[NVA];
#pragma unroll
  for (int v = 0; v < NVA; ++v) avr[v] = f32x4{0.f, 0.f, 0.f, 0.f};

  // V norms of a wave's tile are staged as [2][32] (all n, then all gamma),
  // so a lane reads the 8 values its column takes (n for code columns,
  // gamma for sign columns) as two 16-byte words.
  const int vpart_sel = P8 ? role : (role >= 2 ? 1 : 0);
  const uint32_t vst = 32u * (lane & 1) + (lane >> 1);

  // K part of a tile: logits, online softmax, and the V weight operands
  // (bvc: code product, bvs: sign product) of its tokens.
  auto kpart = [&](const BRaw<M>& r, const BRaw<M>& rv, int t, u32x4& bvc, u32x4& bvs) __attribute__((always_inline)) {
    const bool full = t < n_full;
    const int nvt = full ? kTile : (int)(N - (int64_t)t * kTile);  // valid tokens of the tile
    const int nvl = nvt - 8 * lg;  // valid tokens among the lane's 8 (j < nvl)
    {
      const bool nok = full || (int)(lane >> 1) < nvt;
      const float x = bnorm(r.kn, a.kn_f16);
      nrm_k[lane] = nok ? (odd ? x : x * kinv) : 0.f;
      // (V norms times 2^-kTOff: the weights exp2(t) carry 2^kTOff)
      if constexpr (WV != 0) nrm_v[vst] = nok ? bnorm(rv.vn, a.vn_f16) * 0x1p-96f : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    f32x4 ak[2], as[P8 ? 2 : 1];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      ak[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (P8) as[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 kc = bcodes8<M>(r.kc[tau], M * c, koff);
        const u32x4 ks = bsigns8(&r.ks[tau], c, soff);
        ak[tau] = mfma16(kc, bq[c], ak[tau]);
        if constexpr (P8)
          as[tau] = mfma16(ks, bs[c], as[tau]);
        else
          ak[tau] = mfma16(ks, bs[c], ak[tau]);
      }
    }
    float kn[8][2];
    load_norms<1>(nrm_k + 16 * lg, kn);
    // logits relative to the running integer reference (log2 domain):
    // t = logit - m_ref + kTOff, the offset folded into the inner fma. For
    // |logit - m_ref| < 32 the offset sums (both fma results; in 8-head
    // blocks the hi lane's and the final sum, the lo lane's part not
    // depending on the reference) lie in [64, 128), where fp32 values sit on
    // the fixed grid 2^-17: their roundings commute with the integer
    // reference, so a weight is the same power-of-two multiple for any split
    // (or wave) whose reference differs
    // (logits only: no offset; 8-head blocks: the hi lane carries it, the
    // lo lane none)
    float t2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tau = j >> 2, i = j & 3;
      const float v = ak[tau][i];
      if constexpr (P8) {
        // the hi and lo columns hold the two parts of the same products at
        // the same scale: each lane forms its part of the logit (codes times
        // n, signs times gamma; the hi lane with the offset, in [64, 128)),
        // and the partner column ln ^ 8 (one DPP row rotation) adds the
        // other part; the sum commutes, so both lanes hold the same value
        const float u = fmaf(kn[j][1], as[tau][i], fmaf(kn[j][0], v, t_offc));
        t2[j] = u + dpp_full<0x128>(u);
      } else {
        // quad_perm broadcasts of the quad's columns: q_rot hi, q_rot lo
        // (times 2^11), q_sk hi, q_sk lo (own scale)
        const float v0 = dpp_full<0x00>(v), v1 = dpp_full<0x55>(v), v2 = dpp_full<0xAA>(v),
                    v3 = dpp_full<0xFF>(v);
        t2[j] = fmaf(kn[j][1], v2 + v3, fmaf(kn[j][0], fmaf(kLoInv, v1, v0), t_offc));
      }
    }
    if (a.T > 1) {
      const int64_t lim = N - a.T + hloc % a.T + 1;
      const int64_t tok0 = (int64_t)t * kTile + 8 * lg;
#pragma unroll
      for (int j = 0; j < 8; ++j) t2[j] = tok0 + j < lim ? t2[j] : -INFINITY;
    }
    if (a.logits) {
      if (hvalid && role == 0) {
        const float t_off = (WV != 0 ? kTOff : 0.f) - (m_run == -INFINITY ? 0.f : m_run);
        // the block's logits from the tile's first token on; the lane's head
        // and tokens as a 32-bit offset (contexts of up to 2^26 tokens)
        const auto lr = rsrc(a.logits + ((int64_t)b * a.hq + kvh * a.group + hblk * HB) * a.n_ctx + (int64_t)t * kTile);
        const uint32_t lo = 4u * ((uint32_t)hcol * (uint32_t)a.n_ctx + 8u * lg);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < nvl)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((t2[j] - t_off) * kLn2), lr, lo, 4 * j, 0);
      }
    }
    if (!full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) t2[j] = j < nvl ? t2[j] : -INFINITY;
    }
    if constexpr (WV != 0) {
      // ---------------- online softmax (every lane: its column's head) ----------------
      // (IEEE maximum: no NaN arises here, and it takes no canonicalizing moves)
      float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(t2[0], t2[1]),
                                               __builtin_elementwise_maximum(t2[2], t2[3]));
      mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(t2[4], t2[5]));
      mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(t2[6], t2[7]));
      mx = rows4_maximum(mx);
      // integer log2-domain reference: weights and rescales are exact powers
      // of two times the same mantissa, independent of the split count; a
      // head's candidate m_ref + ceil(mx) - kTOff exceeds m_run exactly when
      // mx exceeds the threshold
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        // some head's maximum moved: rescale (factor 1 for the others; a
        // head that has seen only masked tokens keeps -inf and factor 1)
        const float m_ref = m_run == -INFINITY ? 0.f : m_run;
        const float m_cand = m_ref + (ceilf(mx) - kTOff);
        const float m_new = fmaxf(m_run, m_cand);
        const float corr = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int v = 0; v < NMT; ++v) avr[v] *= corr;
        m_run = m_new;
        // t relative to the new reference (m_run is -inf only while every
        // token seen is masked: then t stays -inf and p = 0)
        const float delta = m_run == -INFINITY ? 0.f : m_run - m_ref;
#pragma unroll
        for (int j = 0; j < 8; ++j) t2[j] -= delta;
        ref_vals();
      }
      // (when no reference moved, m_ref is this lane's m_run, or 0 while
      // every token seen is masked, so t is already relative to it;
      // exp2(t) <= 2^kTOff)
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(t2[j]);
      float psum = p[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) psum += p[j];
      l_run += psum;  // (in units of 2^kTOff)
      // this column's V norms (n or gamma) of the lane's 8 tokens
      float vn[8];
      {
        const f32x4* vp = reinterpret_cast<const f32x4*>(nrm_v + 32 * vpart_sel + 8 * lg);
        const f32x4 x0 = vp[0], x1 = vp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vn[e] = x0[e];
          vn[4 + e] = x1[e];
        }
      }
      if constexpr (P8) {
        // columns h: w_n = p n (code product), columns h + 8: w_g = p gamma
        // (sign product), plain fp16, one accumulator set
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = h2bits(p[2 * q] * vn[2 * q], p[2 * q + 1] * vn[2 * q + 1]);
        const u32x4 z{0, 0, 0, 0};
        bvc = role ? z : w;
        bvs = role ? w : z;
      } else {
        const bool gsel = role >= 2;
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = h2bits(wsplit(p[2 * q] * vn[2 * q], bsel, csel), wsplit(p[2 * q + 1] * vn[2 * q + 1], bsel, csel));
        const u32x4 z{0, 0, 0, 0};
        bvc = gsel ? z : w;
        bvs = gsel ? w : z;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // V part of a tile: accumulate its weighted codes and signs in the rotated
  // and sketch domains
  auto vpart = [&](const BRaw<M>& r, const u32x4& bvc, const u32x4& bvs) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NMT; ++u) {
      const u32x4 vc = bcodes8<M>(r.vc, M * u, voff);
      avr[u] = mfma16(vc, bvc, avr[u]);
      if constexpr (WV == 1) {
        const u32x4 vs = bsigns8(r.vs, u, soff);
        avr[u] = mfma16(vs, bvs, avr[u]);
      }
    }
  };

  if (tile < t_end) {
    // stage of tile i: the loads of tile i + NBV - 1 (V words, into the V
    // buffer of tile i - 1) and tile i + NBK - 1 (K words), then this tile's
    // K part and V part; true after the wave's last tile
    auto stage = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      // (V first: loads complete in issue order, so waiting for this tile's
      // V words then leaves the later tiles' K words in flight)
      if constexpr (WV != 0) load_v(tile_row(ahead(NBV - 1)), vbuf(std::integral_constant<int, k + NBV - 1>{}));
      load_k(tile_row(ahead(NBK - 1)), kbuf(std::integral_constant<int, k + NBK - 1>{}));
      u32x4 bvc, bvs;
      kpart(kbuf(kc), vbuf(kc), tile, bvc, bvs);
      if constexpr (WV != 0) vpart(vbuf(kc), bvc, bvs);
      if (tile == last) return true;
      tile += kBW;
      return false;
    };
    // the loop body runs lcm(NBK, NBV) stages, so every stage's buffers are
    // fixed registers
    constexpr int NS = NBK == NBV ? NBK : NBK * NBV;
    auto run = [&](auto self, auto kc) __attribute__((always_inline)) -> bool {
      constexpr int k = decltype(kc)::value;
      if constexpr (k == NS) {
        return false;
      } else {
        if (stage(kc)) return true;
        return self(self, std::integral_constant<int, k + 1>{});
      }
    };
    while (!run(run, std::integral_constant<int, 0>{})) {
    }
  }

  if constexpr (WV != 0) {
    // ---- merge the workgroup's waves into one partial per head ----
    // Region r (0..3) holds, per channel, the sum of the 16 accumulator
    // columns of waves r, r + 4, ... scaled to the workgroup maximum:
    // float (ch, col) at 16 ch + col + 16 (ch / 32), so the 64 lanes of one
    // store fall in 64 different banks.
    constexpr int RS = 128 * 16 + 64;
    float* s_red = reinterpret_cast<float*>(lds);
    __syncthreads();  // tables are no longer read
    l_run = rows4_sum(l_run) * 0x1p-96f;  // back from units of 2^kTOff
    if (lg == 0 && role == 0) s_m[wv * 8 + hcol] = m_run;
    __syncthreads();
    float Mh = s_m[hcol];
#pragma unroll
    for (int w = 1; w < kBW; ++w) Mh = fmaxf(Mh, s_m[w * 8 + hcol]);
    const float e = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - Mh);
    if (lg == 0 && role == 0) s_lw[wv * 8 + hcol] = l_run * e;
    float* reg = s_red + (wv & 3) * RS;
    auto put = [&](bool add) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NMT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 8 * (4 * lg + i) + u;
          const int idx = 16 * ch + ln + 16 * (ch >> 5);
          if (add) {
            reg[idx] += avr[u][i] * e;
          } else {
            reg[idx] = avr[u][i] * e;
          }
        }
    };
    for (int pass = 0; pass < kBW / 4; ++pass) {
      if (wv / 4 == pass) put(pass > 0);
      __syncthreads();
    }
    // partial of every valid head: [max (log2 domain), sum, acc_rot[D] / s_V, acc_sk[D]]
    const int nh = a.group - hblk * HB < HB ? a.group - hblk * HB : HB;
    const float vinv = 1.0f / a.kscale[2];
    for (int e2 = tid; e2 < nh * (2 + 2 * D); e2 += kBThreads) {
      const int h = e2 / (2 + 2 * D), k = e2 % (2 + 2 * D);
      float val;
      if (k < 2) {
        float Mx = s_m[h];
#pragma unroll
        for (int w = 1; w < kBW; ++w) Mx = fmaxf(Mx, s_m[w * 8 + h]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kBW; ++w) L += s_lw[w * 8 + h];
        val = k == 0 ? Mx : L;
      } else {
        const int pt = (k - 2) / D, ch = (k - 2) % D;
        // columns (P8: the code product in column h, the sign product in
        // column h + 8, both plain; HB = 4: the leading and remainder
        // columns of each part)
        const int chi = P8 ? h + 8 * pt : 4 * h + 2 * pt, clo = P8 ? chi : 4 * h + 2 * pt + 1;
        const int base = 16 * ch + 16 * (ch >> 5);
        float hi = 0.f, lo = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hi += s_red[r * RS + base + chi];
          lo += s_red[r * RS + base + clo];
        }
        val = P8 ? hi : fmaf(kLoInv, lo, hi);
        if (pt == 0) val *= vinv;
      }
      const int hq2 = kvh * a.group + hblk * HB + h;
      a.part[(((int64_t)b * a.hq + hq2) * a.n_split + split) * (2 + 2 * D) + k] = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk kernel: the split-K pass when a KV head has many query columns (a
// causal chunk of T query tokens gives G T columns), for one quantizer group
// of d = 128. The 16-column kernel would decode every tile once per 16
// columns; here a workgroup of 8 waves decodes each 32-token tile of its
// split once into LDS as fp16 MFMA operands, and each wave then runs the
// logits, softmax and V products of one 16-column block from them:
//   K tile  [32 rows][128 channels]: fp16(s c[code]) and fp16 +-1 signs, row
//           16 tau + r holding the token that MFMA row r of half tau takes
//           (8 (r / 4) + r % 4 + 4 tau), so the 16 rows one operand read
//           spans fall in disjoint banks;
//   V tile  [128 channels][32 tokens]: the same for V;
//   norms   [32][n, gamma] for K (n / s_K) and V.
// Decoding: thread t takes 8 K codes and 8 K sign bits of token t / 16
// (channels 8 (t mod 16) ...), and 8 V codes and sign bits of channel t / 4
// (octet t mod 4), turns code pairs into fp16 pairs through a 2^(2m)-entry
// LDS table, and stores 16 bytes per operand. Two tile buffers: tile t + 1 is
// decoded (and tile t + 2 loaded) while tile t is computed, one barrier per
// tile. Columns, weights and partials
// are those of the 16-column kernel (q_rot hi / lo and q_sk; plain fp16
// weights), so the combine reads the same partial layout.
// ---------------------------------------------------------------------------
constexpr int kCW = 8;                // waves (16-column blocks) per workgroup
constexpr int kCThreads = 64 * kCW;
constexpr int kCKS = 128 + 8;         // row stride (fp16) of the K operand tiles
constexpr int kCVS = 32 + 8;          // row stride (fp16) of the V operand tiles

struct ChunkTile {
  _Float16 ka[32 * kCKS], ks[32 * kCKS];
  _Float16 va[128 * kCVS], vs[128 * kCVS];
  float kn[64], vn[64];
};
// pair tables: entry e = (fp16(s c[e & mask]), fp16(s c[e >> m])) for a pair
// of codes, 16 replicas side by side (a lane reads replica lane mod 16, so
// lanes that look up different entries mostly hit different banks)
constexpr int kCRep = 16;
struct ChunkLds {
  ChunkTile tile[2];  // tile t in tile[t % 2]: one decoded while the other is computed
  uint32_t kpair[256 * kCRep], vpair[256 * kCRep];
};

// Raw record words of one tile held by one thread between load and decode.
struct ChunkRaw {
  uint32_t kc0, kc1, ks, vc0, vc1, vs, nrm;
};

// eight fp16 +-1 of the bits of byte b (bit 1 -> +1), as four words
__device__ __forceinline__ u32x4 sign_operand(uint32_t b) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (b >> (2 * i)) & 1u, hi = (b >> (2 * i + 1)) & 1u;
    r[i] = 0xBC00BC00u ^ (lo << 15) ^ (hi << 31);
  }
  return r;
}

template <int M, int WV>
__global__ __launch_bounds__(kCThreads, 1) void chunk_kernel(DArgs a) {
  constexpr int D = 128, NC = 4, NMT = 8;
  constexpr uint32_t PMASK = (1u << (2 * M)) - 1u;
  constexpr int CW = 4 * M;    // K code words per row
  constexpr int BCW = 128 * M; // V code words per 32-row block
  __shared__ __align__(16) ChunkLds L;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.hkv;
  const int kvh = bh % a.hkv;

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
  auto tile_row = [&](int64_t t) __attribute__((always_inline)) -> int64_t {
    if (!a.block_table) return rowbase + t * kTile;
    int64_t pb = a.block_table[(int64_t)b * a.max_blocks + t];
    pb = pb < 0 ? 0 : (pb >= a.n_pblocks ? a.n_pblocks - 1 : pb);
    return (pb * a.hkv + kvh) * kTile;
  };

  // ---- what this thread decodes ----
  const int kr = tid >> 4, kch = (tid & 15) * 8;  // K: token kr, channels kch ..
  const int krow = 16 * ((kr >> 2) & 1) + 4 * (kr >> 3) + (kr & 3);  // its LDS row
  const int kbit = M * kch;                       // first code bit in the row
  const int vj = tid >> 2, vo = tid & 3;          // V: channel vj, octet vo
  const int vbit = 8 * M * (vo * D + vj);         // first code bit in the block
  auto load = [&](int64_t t, ChunkRaw& r) __attribute__((always_inline)) {
    const int64_t row0 = tile_row(t);
    const uint32_t* kcp = a.kc + (row0 + kr) * CW;
    const int kw = kbit >> 5;
    r.kc0 = kcp[kw];
    r.kc1 = kcp[kw + 1 < CW ? kw + 1 : CW - 1];
    r.ks = a.ks[(row0 + kr) * 4 + (kch >> 5)];
    r.nrm = 0u;
    if (tid < 64) {
      const char* kn = reinterpret_cast<const char*>(a.kn) + (row0 << a.kn_shift);
      r.nrm = *reinterpret_cast<const uint32_t*>(kn + (a.kn_f16 ? 4 * (tid >> 1) : 4 * tid));
    }
    if constexpr (WV != 0) {
      const uint32_t* vcp = a.vc + (row0 >> 5) * BCW;
      const int vw = vbit >> 5;
      r.vc0 = vcp[vw];
      r.vc1 = vcp[vw + 1 < BCW ? vw + 1 : BCW - 1];
      if constexpr (WV == 1) r.vs = a.vs[(row0 >> 5) * D + ((vo * D + vj) >> 2)];
      if (tid >= 64 && tid < 128) {
        const char* vn = reinterpret_cast<const char*>(a.vn) + (row0 << a.vn_shift);
        const int e = tid - 64;
        r.nrm = *reinterpret_cast<const uint32_t*>(vn + (a.vn_f16 ? 4 * (e >> 1) : 4 * e));
      }
    }
  };
  const float kinv = 1.0f / a.kscale[0];
  auto decode = [&](const ChunkRaw& r, int64_t T0, ChunkTile& B) __attribute__((always_inline)) {
    {
      const uint32_t f = __builtin_amdgcn_alignbit(r.kc1, r.kc0, kbit & 31);  // 8 M code bits
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = L.kpair[((f >> (2 * M * i)) & PMASK) * kCRep + (lane & (kCRep - 1))];
      *reinterpret_cast<u32x4*>(&B.ka[krow * kCKS + kch]) = w;
      *reinterpret_cast<u32x4*>(&B.ks[krow * kCKS + kch]) = sign_operand((r.ks >> (kch & 31)) & 0xFFu);
    }
    if constexpr (WV != 0) {
      const uint32_t f = __builtin_amdgcn_alignbit(r.vc1, r.vc0, vbit & 31);
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = L.vpair[((f >> (2 * M * i)) & PMASK) * kCRep + (lane & (kCRep - 1))];
      *reinterpret_cast<u32x4*>(&B.va[vj * kCVS + 8 * vo]) = w;
      if constexpr (WV == 1)
        *reinterpret_cast<u32x4*>(&B.vs[vj * kCVS + 8 * vo]) =
            sign_operand((r.vs >> (8 * ((vo * D + vj) & 3))) & 0xFFu);
    }
    // norms past the sequence read as 0 (their tokens are masked)
    if (tid < 128) {
      const int e = tid & 63;
      const bool nok = T0 + (e >> 1) < N;
      const bool is_k = tid < 64;
      const int f16 = is_k ? a.kn_f16 : a.vn_f16;
      const float v = nok ? norm_value(r.nrm, f16 ? 16u * (e & 1) : 0u, f16) : 0.f;
      if (is_k)
        B.kn[e] = (e & 1) ? v : v * kinv;
      else if constexpr (WV != 0)
        B.vn[e] = v;
    }
  };

  // ---- pair tables of the scaled codebooks ----
  {
    const float ks0 = a.kscale[0];
    for (int x = tid; x < (int)(PMASK + 1) * kCRep; x += kCThreads) {
      const int e = x / kCRep, c0 = e & ((1 << M) - 1), c1 = e >> M;
      L.kpair[x] = h2bits(a.kcent[c0] * ks0, a.kcent[c1] * ks0);
      if constexpr (WV != 0) L.vpair[x] = h2bits(a.vcent[c0] * a.kscale[2], a.vcent[c1] * a.kscale[2]);
    }
  }

  // ---- this wave's 16 columns and their query operands ----
  const int hloc = (blockIdx.z * kCW + wv) * 16 + ln;
  const bool hvalid = hloc < a.group;
  const bool wave_on = __builtin_amdgcn_readfirstlane((blockIdx.z * kCW + wv) * 16 < a.group ? 1 : 0) != 0;
  const int hq = kvh * a.group + hloc;
  u32x4 qr[NC], qrl[NC], qs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const _Float16* qp = a.qprep + ((int64_t)b * a.hq + (hvalid ? hq : 0)) * (4 * D) + 32 * c + 8 * lg;
    const u32x4 z{0, 0, 0, 0};
    qr[c] = hvalid ? *reinterpret_cast<const u32x4*>(qp) : z;
    qrl[c] = hvalid ? *reinterpret_cast<const u32x4*>(qp + D) : z;
    qs[c] = hvalid ? *reinterpret_cast<const u32x4*>(qp + 2 * D) : z;
  }
  const int64_t lim = a.T > 1 ? N - a.T + hloc % a.T + 1 : N;  // tokens this column sees

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_r[WV ? NMT : 1], acc_s[WV == 1 ? NMT : 1];
#pragma unroll
  for (int u = 0; u < (WV ? NMT : 1); ++u) acc_r[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < (WV == 1 ? NMT : 1); ++u) acc_s[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int64_t T0, const ChunkTile& B) __attribute__((always_inline)) {
    // ---- logits: MFMA row ln of half tau is token 8 (ln / 4) + ln % 4 + 4 tau,
    // so lane (ln, lg) ends with tokens 8 lg + j, j = 4 tau + i, of column ln
    f32x4 lr[2], lrl[2], ls[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      lr[tau] = lrl[tau] = ls[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * tau + ln;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 ak = *reinterpret_cast<const u32x4*>(&B.ka[row * kCKS + 32 * c + 8 * lg]);
        const u32x4 az = *reinterpret_cast<const u32x4*>(&B.ks[row * kCKS + 32 * c + 8 * lg]);
        lr[tau] = mfma16(ak, qr[c], lr[tau]);
        lrl[tau] = mfma16(ak, qrl[c], lrl[tau]);
        ls[tau] = mfma16(az, qs[c], ls[tau]);
      }
    }
    float kn[8][2];
    load_norms<1>(&B.kn[16 * lg], kn);
    const int64_t tok0 = T0 + 8 * lg;
    float l2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tau = j >> 2, i = j & 3;
      l2[j] = kn[j][0] * fmaf(kLoInv, lrl[tau][i], lr[tau][i]) + kn[j][1] * ls[tau][i];
      if (tok0 + j >= lim) l2[j] = -INFINITY;  // causal limit and the sequence end
    }
    if (a.logits && hvalid) {
      float* lp = a.logits + ((int64_t)b * a.hq + hq) * a.n_ctx + tok0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tok0 + j < N) lp[j] = l2[j] * kLn2;
    }
    if constexpr (WV != 0) {
      // (IEEE maximum: no NaN arises here, and it takes no canonicalizing moves)
      float mx = l2[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = __builtin_elementwise_maximum(mx, l2[j]);
      mx = rows4_maximum(mx);
      // integer log2-domain reference (as the other split-K kernels)
      const float m_new = fmaxf(m_run, ceilf(mx));
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float corr = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int u = 0; u < NMT; ++u) acc_r[u] *= corr;
        if constexpr (WV == 1) {
#pragma unroll
          for (int u = 0; u < NMT; ++u) acc_s[u] *= corr;
        }
        m_run = m_new;
      }
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(l2[j] - m_ref);
        l_run += p[j];
      }
      float vn[8][2];
      load_norms<1>(&B.vn[16 * lg], vn);
      u32x4 pr, pz;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pr[q] = h2bits(p[2 * q] * vn[2 * q][0], p[2 * q + 1] * vn[2 * q + 1][0]);
        pz[q] = h2bits(p[2 * q] * vn[2 * q][1], p[2 * q + 1] * vn[2 * q + 1][1]);
      }
#pragma unroll
      for (int u = 0; u < NMT; ++u) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(&B.va[(16 * u + ln) * kCVS + 8 * lg]);
        acc_r[u] = mfma16(av, pr, acc_r[u]);
        if constexpr (WV == 1) {
          const u32x4 az = *reinterpret_cast<const u32x4*>(&B.vs[(16 * u + ln) * kCVS + 8 * lg]);
          acc_s[u] = mfma16(az, pz, acc_s[u]);
        }
      }
    }
  };

  // ---- tile loop: compute tile j from one buffer while tile j + 1 is
  // decoded into the other; the records of tile i sit in register slot i mod 3
  // from their load, three tiles ahead, to their decode ----
  if (t_begin < t_end) {
    ChunkRaw r0, r1, r2;
    auto slot = [&](auto kc) __attribute__((always_inline)) -> ChunkRaw& {
      constexpr int k = decltype(kc)::value;
      if constexpr (k == 0) return r0;
      else if constexpr (k == 1) return r1;
      else return r2;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    load(t_begin, r0);
    if (t_begin + 1 < t_end) load(t_begin + 1, r1);
    if (t_begin + 2 < t_end) load(t_begin + 2, r2);
    __syncthreads();  // pair tables
    decode(r0, t_begin * kTile, L.tile[0]);
    if (t_begin + 3 < t_end) load(t_begin + 3, r0);
    __syncthreads();
    int64_t t = t_begin;
    // stage of tile t = t_begin + j: slot k holds tile j + 1
    auto stage = [&](auto kc) __attribute__((always_inline)) {
      const int j = (int)(t - t_begin);
      if (t + 1 < t_end) {
        decode(slot(kc), (t + 1) * kTile, L.tile[(j + 1) & 1]);
        if (t + 4 < t_end) load(t + 4, slot(kc));
      }
      if (wave_on) compute(t * kTile, L.tile[j & 1]);
      __syncthreads();
      ++t;
      return t >= t_end;
    };
    for (;;) {
      if (stage(I1{})) break;
      if (stage(I2{})) break;
      if (stage(I0{})) break;
    }
  }

  // ---- partial of each of this wave's columns: [max, sum, acc_rot / s_V, acc_sk] ----
  if constexpr (WV != 0) {
    l_run = rows4_sum(l_run);
    if (hvalid) {
      float* pp = a.part + (((int64_t)b * a.hq + hq) * a.n_split + split) * (2 + 2 * D);
      if (lg == 0) {
        pp[0] = m_run;
        pp[1] = l_run;
      }
      const float vinv = 1.0f / a.kscale[2];
#pragma unroll
      for (int u = 0; u < NMT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * u + 4 * lg + i;
          pp[2 + ch] = acc_r[u][i] * vinv;
          pp[2 + D + ch] = WV == 1 ? acc_s[u][i] : 0.f;
        }
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
    // (a query token that sees no key at all -- a paged sequence shorter
    // than the chunk -- has L = 0 and gets a zero output)
    out[orow * D + cs * OC + t] = L > 0.f ? o / L : 0.f;
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
  size_t bytes = align256(heads * 4 * d * sizeof(_Float16)) + 256;
  if (with_v) bytes += align256(heads * (size_t)n_split * (2 + 2 * d) * sizeof(float));
  return bytes;
}

// heads per workgroup: 4 (packed columns) for KV groups of at most 4 query
// heads with V, else 16
inline int heads_per_block(int group, bool with_v) { return with_v && group <= 4 ? 4 : 16; }

// The byte-table kernel takes one quantizer group of d = 128 whose code
// width divides 8.
inline bool byte_kernel_ok(const tq_layout& l) {
  const int m = l.mse_bits[0];
  return l.d == 128 && l.n_groups == 1 && (m == 1 || m == 2 || m == 4);
}

// Kernel, head block and split count of a decode call (the workspace size
// and the launch both follow from it).
struct DecodeCfg {
  bool byte, chunk;
  int hb, n_hblk, n_split;
};

// The chunk kernel serves a KV head's many columns from tiles decoded once:
// one quantizer group of d = 128 and more than one 16-column block.
inline bool chunk_kernel_ok(const tq_layout& l, int group) { return l.d == 128 && l.n_groups == 1 && group > 16; }

DecodeCfg decode_cfg(const tq_layout& l, bool with_v, const tq_decode_shape* s) {
  DecodeCfg c{};
  const int T = s->n_q_tokens < 1 ? 1 : s->n_q_tokens;
  const int group = s->n_q_heads / s->n_kv_heads * T;
  c.chunk = chunk_kernel_ok(l, group);
  if (c.chunk) {
    // 16-column blocks, kCW of them per workgroup (grid z); about one
    // workgroup per compute unit, at least one tile per split
    c.hb = 16;
    c.n_hblk = (group + 15) / 16;
    const int n_z = (c.n_hblk + kCW - 1) / kCW;
    const int64_t n_tiles = (s->n_ctx + kTile - 1) / kTile;
    int64_t max_split = n_tiles < kMaxSplit ? n_tiles : kMaxSplit;
    if (max_split < 1) max_split = 1;
    if (s->n_split > 0) {
      c.n_split = (int)(s->n_split < max_split ? s->n_split : max_split);
      return c;
    }
    const int64_t per = (int64_t)s->batch * s->n_kv_heads * n_z;
    int64_t want = (256 + per - 1) / per;
    if (want > max_split) want = max_split;
    c.n_split = (int)(want < 1 ? 1 : want);
    return c;
  }
  // (the byte kernel keeps tile indices and per-lane logit offsets in 32
  // bits: contexts of up to 2^26 tokens)
  c.byte = byte_kernel_ok(l) && s->n_ctx <= (int64_t(1) << 26);
  c.hb = c.byte ? (group <= 4 ? 4 : 8) : heads_per_block(group, with_v);
  c.n_hblk = (group + c.hb - 1) / c.hb;
  if (!c.byte) {
    c.n_split = choose_split(s, c.n_hblk);
    return c;
  }
  // one workgroup per compute unit; at least one tile per wave
  const int64_t n_tiles = (s->n_ctx + kTile - 1) / kTile;
  const int bw = byte_waves(l.mse_bits[0]);
  int64_t max_split = (n_tiles + bw - 1) / bw;
  if (max_split > kMaxSplit) max_split = kMaxSplit;
  if (max_split < 1) max_split = 1;
  if (s->n_split > 0) {
    c.n_split = (int)(s->n_split < max_split ? s->n_split : max_split);
    return c;
  }
  const int64_t per = (int64_t)s->batch * s->n_kv_heads * c.n_hblk;
  int64_t want = (256 + per - 1) / per;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  c.n_split = (int)want;
  return c;
}

template <int M, int WV, int HB>
hipError_t launch_byte(const DArgs& a, int n_hblk, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&decode_byte_kernel<M, WV, HB>);
  // the table addresses are absolute LDS addresses: the kernel must have no
  // static LDS, so that its dynamic LDS starts at address 0
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, fn) != hipSuccess || fa.sharedSizeBytes != 0) return hipErrorInvalidValue;
  constexpr int lds = BLds<byte_waves(M)>::bytes;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return hipErrorInvalidValue;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv), (unsigned)n_hblk);
  hipLaunchKernelGGL((decode_byte_kernel<M, WV, HB>), grid, dim3(64 * byte_waves(M)), lds, st, a);
  return hipGetLastError();
}

template <int M, int WV>
hipError_t dispatch_byte_hb(const DArgs& a, int hb, int n_hblk, hipStream_t st) {
  return hb == 4 ? launch_byte<M, WV, 4>(a, n_hblk, st) : launch_byte<M, WV, 8>(a, n_hblk, st);
}

template <int WV>
hipError_t dispatch_byte(const DArgs& a, int m, int hb, int n_hblk, hipStream_t st) {
  switch (m) {
    case 1: return dispatch_byte_hb<1, WV>(a, hb, n_hblk, st);
    case 2: return dispatch_byte_hb<2, WV>(a, hb, n_hblk, st);
    default: return dispatch_byte_hb<4, WV>(a, hb, n_hblk, st);
  }
}

template <int M, int WV>
hipError_t launch_chunk(const DArgs& a, int n_hblk, hipStream_t st) {
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv), (unsigned)((n_hblk + kCW - 1) / kCW));
  hipLaunchKernelGGL((chunk_kernel<M, WV>), grid, dim3(kCThreads), 0, st, a);
  return hipGetLastError();
}

template <int WV>
hipError_t dispatch_chunk(const DArgs& a, int m, int n_hblk, hipStream_t st) {
  switch (m) {
    case 1: return launch_chunk<1, WV>(a, n_hblk, st);
    case 2: return launch_chunk<2, WV>(a, n_hblk, st);
    case 3: return launch_chunk<3, WV>(a, n_hblk, st);
    default: return launch_chunk<4, WV>(a, n_hblk, st);
  }
}

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
  const DecodeCfg cfg = decode_cfg(kq->layout, vq != nullptr, shape);
  *bytes = workspace_for(shape, kq->layout.d, vq != nullptr, cfg.n_split);
  return TQ_OK;
}

namespace {

// Everything a decode call launches, validated and laid out in the workspace.
struct Plan {
  DArgs a;
  tqp::PrepArgs prep;
  int n_hblk, hb, prep_grid_y, n_heads, n_groups, m0, m1, group_dim0, T, hq_orig;
  bool with_v, v_mse;  // V records present; V records without sign bits
  bool byte;           // the byte-table split-K kernel
  bool chunk;          // the decode-once chunk kernel
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
  (void)group;
  const DecodeCfg cfg = decode_cfg(l, with_v, shape);
  const int n_hblk = cfg.n_hblk;
  const int n_split = cfg.n_split;
  const size_t need = workspace_for(shape, l.d, with_v, n_split);
  if (!workspace || workspace_bytes < need) return TQ_ERR_WORKSPACE;

  constexpr int D = kD;
  const int n_heads = shape->batch * shape->n_q_heads * T;
  _Float16* qprep = reinterpret_cast<_Float16*>(workspace);
  float* kscale = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                           align256((size_t)n_heads * 4 * D * sizeof(_Float16)));
  float* part = kscale + 64;

  *pl = Plan{};
  pl->n_hblk = n_hblk;
  pl->hb = cfg.hb;
  pl->byte = cfg.byte;
  pl->chunk = cfg.chunk;
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
  pp.vcent = with_v ? vq->centroids : nullptr;
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
    if (pl.chunk)
      e = !pl.with_v  ? dispatch_chunk<0>(pl.a, pl.m0, pl.n_hblk, st)
          : pl.v_mse ? dispatch_chunk<2>(pl.a, pl.m0, pl.n_hblk, st)
                     : dispatch_chunk<1>(pl.a, pl.m0, pl.n_hblk, st);
    else if (pl.byte)
      e = !pl.with_v  ? dispatch_byte<0>(pl.a, pl.m0, pl.hb, pl.n_hblk, st)
          : pl.v_mse ? dispatch_byte<2>(pl.a, pl.m0, pl.hb, pl.n_hblk, st)
                     : dispatch_byte<1>(pl.a, pl.m0, pl.hb, pl.n_hblk, st);
    else if (pl.n_groups == 1)
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
// Fused appends + query preparation: the blocks of one launch run the query
// preparation, then quantize the new K vectors, then the new V vectors (the
// three are independent, so their latencies overlap).
// ---------------------------------------------------------------------------
constexpr int kStepKP = 128, kStepNT = 8;  // quantize shape for d = 128

struct StepArgs {
  tqq::QArgs k, v;
  int nk, nv;  // blocks given to the K and V appends (0 = none)
  int k_small, v_small;  // append takes the one-block-per-vector path
  tqp::PrepArgs prep;
  int prep_x;  // prep blocks along x; the prep blocks are laid out x-major
  int n_prep;  // prep blocks (the first blocks of the grid: they are short and
               // then leave every compute unit to the appends)
};

// SMALL: every append takes the few-vector path (a smaller kernel without the
// tile path, which is the usual decode step of one token per head). H: the
// tile path takes its transposed half-precision variant (both appends qualify).
template <bool SMALL, bool H>
__global__ __launch_bounds__(kStepNT * 64) void step_kernel(StepArgs s) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < s.n_prep) {
    const int pb = blockIdx.x;
    tqp::prep_block<kD, kStepNT * 64>(s.prep, pb % s.prep_x, pb / s.prep_x, threadIdx.x, smem);
    return;
  }
  const int b = blockIdx.x - s.n_prep;
  {
    const bool is_k = b < s.nk;
    if (SMALL || (is_k ? s.k_small : s.v_small))
      tqq::quantize_small<kStepNT * 64>(is_k ? s.k : s.v, is_k ? b : b - s.nk, smem);
    else if constexpr (!SMALL)
    {
      if constexpr (H)
        tqq::quantize_tiles_t<kStepKP, kStepNT>(is_k ? s.k : s.v, is_k ? b : b - s.nk, is_k ? s.nk : s.nv, smem);
      else
        tqq::quantize_tiles<kStepKP, kStepNT>(is_k ? s.k : s.v, is_k ? b : b - s.nk, is_k ? s.nk : s.nv, smem);
    }
  }
}

// The same with the pipelined tile path for the bulk appends (both take it
// with code width MG; V carries sign bits iff VSIGNS).
template <int MG, bool VSIGNS>
__global__ __launch_bounds__(kStepNT * 64) void step_kernel_p(StepArgs s) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < s.n_prep) {
    const int pb = blockIdx.x;
    tqp::prep_block<kD, kStepNT * 64>(s.prep, pb % s.prep_x, pb / s.prep_x, threadIdx.x, smem);
    return;
  }
  const int b = blockIdx.x - s.n_prep;
  const bool is_k = b < s.nk;
  if (is_k ? s.k_small : s.v_small)
    tqq::quantize_small<kStepNT * 64>(is_k ? s.k : s.v, is_k ? b : b - s.nk, smem);
  else if (is_k)
    tqq::quantize_tiles_p<MG, false, true>(s.k, b, s.nk, smem);
  else
    tqq::quantize_tiles_p<MG, true, VSIGNS>(s.v, b - s.nk, s.nv, smem);
}

template <int MG>
const void* step_kernel_p_fn(bool vsigns) {
  return vsigns ? reinterpret_cast<const void*>(&step_kernel_p<MG, true>)
                : reinterpret_cast<const void*>(&step_kernel_p<MG, false>);
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
  sa.n_prep = sa.prep_x * pl.prep_grid_y;
  const int grid = sa.n_prep + sa.nk + sa.nv;
  constexpr int lds_small = tqp::prep_lds_bytes<kD>() > tqq::SmallLds<kStepNT * 64>::bytes
                                ? tqp::prep_lds_bytes<kD>()
                                : tqq::SmallLds<kStepNT * 64>::bytes;
  constexpr int lds_f = tqq::Lds<kStepKP, kStepNT, false>::bytes;
  constexpr int lds_h = tqq::LdsT<kStepKP, kStepNT>::bytes;
  const bool all_small = (k_empty || sa.k_small) && (v_empty || sa.v_small);
  const bool h = (k_empty || sa.k_small || tqq::t_path_ok(sa.k)) && (v_empty || sa.v_small || tqq::t_path_ok(sa.v));
  const void* fn = all_small ? reinterpret_cast<const void*>(&step_kernel<true, false>)
                   : h       ? reinterpret_cast<const void*>(&step_kernel<false, true>)
                             : reinterpret_cast<const void*>(&step_kernel<false, false>);
  // the pipelined tile path: every bulk append takes it with one code width
  // (K with sign bits)
  const bool kp = k_empty || sa.k_small || (tqq::p_path_ok(sa.k) && !sa.k.mse_only);
  const bool vp = v_empty || sa.v_small || tqq::p_path_ok(sa.v);
  const int kbits = (k_empty || sa.k_small) ? 0 : sa.k.gbits[0];
  const int vbits = (v_empty || sa.v_small) ? 0 : sa.v.gbits[0];
  const int pbits = kbits ? kbits : vbits;
  const bool pipe = !all_small && kp && vp && (kbits == 0 || vbits == 0 || kbits == vbits);
  const bool vsigns = v_empty || !sa.v.mse_only;
  const int lds_tiles = pipe ? tqq::LdsP::bytes : h ? lds_h : lds_f;
  const int lds_use = all_small ? lds_small : lds_tiles > lds_small ? lds_tiles : lds_small;
  if (pipe) {
    fn = pbits == 1 ? step_kernel_p_fn<1>(vsigns)
         : pbits == 2 ? step_kernel_p_fn<2>(vsigns)
         : pbits == 3 ? step_kernel_p_fn<3>(vsigns)
                      : step_kernel_p_fn<4>(vsigns);
  }
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_use) != hipSuccess)
    return TQ_ERR_DEVICE;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  if (pipe) {
    void* args[] = {&sa};
    if (hipLaunchKernel(fn, dim3(grid), dim3(kStepNT * 64), args, lds_use, hs) != hipSuccess) return TQ_ERR_DEVICE;
  } else if (all_small)
    hipLaunchKernelGGL((step_kernel<true, false>), dim3(grid), dim3(kStepNT * 64), lds_use, hs, sa);
  else if (h)
    hipLaunchKernelGGL((step_kernel<false, true>), dim3(grid), dim3(kStepNT * 64), lds_use, hs, sa);
  else
    hipLaunchKernelGGL((step_kernel<false, false>), dim3(grid), dim3(kStepNT * 64), lds_use, hs, sa);
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

// ---------------------------------------------------------------------------
// Decode without a caller-supplied workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation). The workspace lives in a file-scope
// device array; each device holds its own copy at its own address, looked up
// once per device (with that device current) and kept for the process.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kScratchMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};

// Device address of `scratch` on the current device (null on failure).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" tq_status tq_attn_decode_scratch(const tq_quantizer* kq, const tq_quantizer* vq,
                                            const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                                            const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                            float* out, void* stream) {
  size_t need = 0;
  tq_status st = tq_attn_decode_workspace_bytes(kq, vq, shape, &need);
  if (st != TQ_OK) return st;
  if (need > kScratchBytes) return TQ_ERR_WORKSPACE;
  // full validation on the host before any HIP call (an aligned stand-in for
  // the workspace address; the real address is looked up afterwards)
  Plan pl;
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
  st = plan_decode(kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out, stand_in, kScratchBytes, &pl);
  if (st != TQ_OK) return st;
  void* ws = scratch_address();
  if (!ws) return TQ_ERR_DEVICE;
  st = plan_decode(kq, vq, shape, q, q_dtype, k_cache, v_cache, logits, out, ws, kScratchBytes, &pl);
  if (st != TQ_OK) return st;
  return run_phases(pl, TQ_PHASE_ALL, reinterpret_cast<hipStream_t>(stream));
}
