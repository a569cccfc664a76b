// Host-side launch of the dense GEMM kernel (gemm_kernel.hpp): tile shape per
// problem size and per accumulation mode, and the operand-format switch.
// Shared by gemm.hip (fp32 / bf16 outputs) and gemm_requant.hip (FP8 outputs).
#pragma once

#include "gemm_kernel.hpp"

namespace fp8mi {

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, int MODE, bool BT>
inline hipError_t gemm_run(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sa,
                           const float* sb, void* C, const RequantArgs& rq, hipStream_t st,
                           const MxScales& mxs = MxScales{nullptr, nullptr}) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  // Bands of 4 tile-rows: with one 256x256 workgroup per CU, each XCD's 32
  // resident tiles then form a 4 x 8 block, whose K steps fill the XCD's L2
  // with 12 operand slabs instead of the 18 of a 16 x 2 block.  Measured on
  // MI355X in steady state (after the clock has settled): 0.7-1.8 % faster
  // for the exact kernel and 3.5 % for the FP8 one than bands of 16; bands of
  // 8 and 2 in between.
  const int group_m = 4;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, FA, FB, OUT, MODE, BT>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * WM * WN), 0, st, A, B, (int)M, (int)N, (int)K, sa, sb, C, tiles_m, tiles_n, group_m,
                     rq, mxs);
  return hipGetLastError();
}

// 256x256 tiles.  bf16 (exact) paths: 8 wavefronts (two per SIMD, 128x64
// each, accumulators and operands in the VGPRs), faster on the FC1 GEMM than 4
// wavefronts of 128x128 (one per SIMD, accumulators in the AGPR half of the
// register file) once the waves' priority window breaks their lockstep
// (gemm_kernel.hpp): per-tensor 2-3 %, MXFP8 8 % (812 against 881 us).
// FP8 path: 8 wavefronts (two per SIMD, 64x128 each).  Small problems:
// 128x128 tiles of four 64x64 wavefronts.  BT: B stored [K x N] (read through
// the LDS transpose path), same tiles.
template <int FA, int FB, int OUT, int MODE, bool BT = false>
inline hipError_t gemm_dispatch_shape(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K,
                                      const float* sa, const float* sb, void* C, const RequantArgs& rq,
                                      hipStream_t st, const MxScales& mxs = MxScales{nullptr, nullptr}) {
  if (M >= 1024 && N >= 1024) {
    if constexpr (MODE == kAccumExact || MODE == kAccumMxExact)
      return gemm_run<256, 256, 2, 4, FA, FB, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
    else return gemm_run<256, 256, 4, 2, FA, FB, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
  }
  return gemm_run<128, 128, 2, 2, FA, FB, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
}

template <int OUT, int MODE, bool BT = false>
inline hipError_t gemm_dispatch_fmt(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                                    int64_t K, const float* sa, const float* sb, void* C, const RequantArgs& rq,
                                    hipStream_t st, const MxScales& mxs = MxScales{nullptr, nullptr}) {
  if (fa == kE4M3 && fb == kE4M3) return gemm_dispatch_shape<kE4M3, kE4M3, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
  if (fa == kE5M2 && fb == kE4M3) return gemm_dispatch_shape<kE5M2, kE4M3, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
  if (fa == kE4M3 && fb == kE5M2) return gemm_dispatch_shape<kE4M3, kE5M2, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
  return gemm_dispatch_shape<kE5M2, kE5M2, OUT, MODE, BT>(A, B, M, N, K, sa, sb, C, rq, st, mxs);
}

}  // namespace fp8mi
