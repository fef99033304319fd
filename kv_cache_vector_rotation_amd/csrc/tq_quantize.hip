// Quantize-on-append for gfx950: one fused kernel per call.
//
// [ZB] paragraph 2 and [WD] "Como o TurboQuant funciona": rotate each vector
// by a random orthogonal matrix, give every rotated coordinate its Lloyd-Max
// cell, take the residual of that MSE quantizer, keep the signs of a Gaussian
// sketch of the residual, and store codes, sign bits and the norms.
//
// Work decomposition (calls with more than a few vectors; a few vectors take
// the one-workgroup-per-vector latency path described with quantize_small).
// A workgroup owns a tile of 64 vectors at a time and
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
#include "tq_quantize_dev.h"
#include "tq_quantize_t_dev.h"
#include "tq_quantize_p_dev.h"
#include "turboquant.h"

namespace {

using tqq::Lds;
using tqq::QArgs;

template <int KP, int NT, bool H>
__global__ __launch_bounds__(NT * 64) void quantize_kernel(QArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  tqq::quantize_tiles<KP, NT, H>(a, blockIdx.x, gridDim.x, smem);
}

template <int KP, int NT>
__global__ __launch_bounds__(NT * 64) void quantize_t_kernel(QArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  tqq::quantize_tiles_t<KP, NT>(a, blockIdx.x, gridDim.x, smem);
}

template <int MG, bool BLK, bool SIGNS>
__global__ __launch_bounds__(tqq::LdsP::NT * 64) void quantize_p_kernel(QArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  tqq::quantize_tiles_p<MG, BLK, SIGNS>(a, blockIdx.x, gridDim.x, smem);
}

__global__ __launch_bounds__(tqq::kSmallThreads) void quantize_small_kernel(QArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  tqq::quantize_small<tqq::kSmallThreads>(a, blockIdx.x, smem);
}

tq_status launch_quantize_small(const QArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  hipLaunchKernelGGL(quantize_small_kernel, dim3((unsigned)a.n_vec), dim3(tqq::kSmallThreads),
                     tqq::SmallLds<tqq::kSmallThreads>::bytes, stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

// The tile kernel loops over tiles (grid-stride), so the grid is one round
// of resident workgroups: compute units times the workgroups that fit on one
// at once (registers and LDS, from the occupancy query).
template <int KP, int NT, bool H, bool T = false>
tq_status launch_quantize(const QArgs& a, hipStream_t stream) {
  constexpr int lds = T ? tqq::LdsT<KP, NT>::bytes : Lds<KP, NT, H>::bytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const void* fn;
  if constexpr (T)
    fn = reinterpret_cast<const void*>(&quantize_t_kernel<KP, NT>);
  else
    fn = reinterpret_cast<const void*>(&quantize_kernel<KP, NT, H>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return TQ_ERR_DEVICE;
  const int64_t n_tiles = a.n_tiles;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n_cu = v;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT * 64, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t grid = n_tiles < (int64_t)per_cu * n_cu ? n_tiles : (int64_t)per_cu * n_cu;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  if constexpr (T)
    hipLaunchKernelGGL((quantize_t_kernel<KP, NT>), dim3((unsigned)grid), dim3(NT * 64), lds, stream, a);
  else
    hipLaunchKernelGGL((quantize_kernel<KP, NT, H>), dim3((unsigned)grid), dim3(NT * 64), lds, stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

// The pipelined path: one resident workgroup round, as above.
template <int MG, bool BLK, bool SIGNS>
tq_status launch_quantize_p(const QArgs& a, hipStream_t stream) {
  constexpr int lds = tqq::LdsP::bytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const void* fn = reinterpret_cast<const void*>(&quantize_p_kernel<MG, BLK, SIGNS>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return TQ_ERR_DEVICE;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n_cu = v;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, tqq::LdsP::NT * 64, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t grid = a.n_tiles < (int64_t)per_cu * n_cu ? a.n_tiles : (int64_t)per_cu * n_cu;
  (void)hipGetLastError();  // a launch error is reported below, not an older one
  hipLaunchKernelGGL((quantize_p_kernel<MG, BLK, SIGNS>), dim3((unsigned)grid), dim3(tqq::LdsP::NT * 64), lds,
                     stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

template <int MG>
tq_status launch_quantize_p_fmt(const QArgs& a, hipStream_t stream) {
  if (a.fmt == TQ_TOKEN_MAJOR) return launch_quantize_p<MG, false, true>(a, stream);
  return a.mse_only ? launch_quantize_p<MG, true, false>(a, stream) : launch_quantize_p<MG, true, true>(a, stream);
}

// (p_path_ok) token-major records with sign bits, or block records
inline bool p_launchable(const QArgs& a) {
  return tqq::p_path_ok(a) && (a.fmt == TQ_BLOCK32 || !a.mse_only);
}

}  // namespace

extern "C" tq_status tq_quantize(const tq_quantizer* qz, tq_format fmt, const void* x,
                                 tq_dtype x_dtype, int64_t n_vec, int64_t x_row_stride,
                                 const tq_rows* rows, const tq_cache* cache, void* stream) {
  QArgs a;
  bool empty = false;
  const tq_status st = tqq::make_qargs(qz, fmt, x, x_dtype, n_vec, x_row_stride, rows, cache, &a, &empty);
  if (st != TQ_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // a few vectors (an append): one workgroup per vector, for latency
  if (tqq::small_path_ok(a)) return launch_quantize_small(a, s);
  if (p_launchable(a)) {
    switch (a.gbits[0]) {
      case 1: return launch_quantize_p_fmt<1>(a, s);
      case 2: return launch_quantize_p_fmt<2>(a, s);
      case 3: return launch_quantize_p_fmt<3>(a, s);
      default: return launch_quantize_p_fmt<4>(a, s);
    }
  }
  const bool h = tqq::h_path_ok(a), t = tqq::t_path_ok(a);
  switch (tqq::quantize_kp(a.d)) {
    case 64:
      return t ? launch_quantize<64, 4, true, true>(a, s)
               : h ? launch_quantize<64, 4, true>(a, s) : launch_quantize<64, 4, false>(a, s);
    case 128:
      return t ? launch_quantize<128, 8, true, true>(a, s)
               : h ? launch_quantize<128, 8, true>(a, s) : launch_quantize<128, 8, false>(a, s);
    case 208: return launch_quantize<208, 13, false>(a, s);
    default: return launch_quantize<256, 16, false>(a, s);
  }
}
