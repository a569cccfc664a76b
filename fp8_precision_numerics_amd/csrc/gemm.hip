// Per-tensor-scaled FP8 GEMM: C = (A · Bᵀ) × sinv_a × sinv_b, FP32 accumulation.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the GEMM runs on FP8
// inputs, the result is accumulated in FP32 and restored with ×(1/scale);
// accumulation is always high precision.  §4.2.6: HYBRID pairs E4M3 forward
// operands with E5M2 gradients, so each operand carries its own format.
//
// Design (gfx950): a workgroup computes a BM x BN output tile with WM x WN
// wavefronts.  Each 128-deep K step moves a BM x 128 slab of A and a BN x 128
// slab of B from HBM/L2 straight into one of two LDS buffers (buffer loads
// with the LDS as destination, issued one step ahead, no register staging),
// while the wavefronts contract the other buffer on the matrix cores (see
// gemm_tile.hpp for the two accumulation modes).  One barrier per K step.
// The epilogue multiplies by sinv_a·sinv_b and writes the tile through LDS as
// whole bf16 or fp32 rows.
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, int MODE>
hipError_t run(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K,
               const float* sa, const float* sb, void* C, hipStream_t st) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int group_m = 16;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, FA, FB, OUT, MODE>),
                     dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WM * WN), 0, st, A, B, (int)M,
                     (int)N, (int)K, sa, sb, C, tiles_m, tiles_n, group_m);
  return hipGetLastError();
}

template <int FA, int FB, int OUT, int MODE>
hipError_t dispatch_shape(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K,
                          const float* sa, const float* sb, void* C, hipStream_t st) {
  // 256x256 tiles.  fp16 path: 4 wavefronts (one per SIMD, 128x128 each, the
  // accumulators in the AGPR half of the register file).  FP8 path: 8
  // wavefronts (two per SIMD, 64x128 each) to hide more latency.
  if (M >= 1024 && N >= 1024) {
    if constexpr (MODE == kAccumExact) return run<256, 256, 2, 2, FA, FB, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
    else return run<256, 256, 4, 2, FA, FB, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
  }
  return run<128, 128, 2, 2, FA, FB, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
}

template <int OUT, int MODE>
hipError_t dispatch_fmt(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                        int64_t K, const float* sa, const float* sb, void* C, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) return dispatch_shape<kE4M3, kE4M3, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
  if (fa == kE5M2 && fb == kE4M3) return dispatch_shape<kE5M2, kE4M3, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
  if (fa == kE4M3 && fb == kE5M2) return dispatch_shape<kE4M3, kE5M2, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
  return dispatch_shape<kE5M2, kE5M2, OUT, MODE>(A, B, M, N, K, sa, sb, C, st);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                       int64_t K, const float* sinv_a, const float* sinv_b, void* C, int ctype,
                       int accum, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (accum == kAccumMfma8) {
    if (ctype == kBF16) return dispatch_fmt<kBF16, kAccumMfma8>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
    return dispatch_fmt<kF32, kAccumMfma8>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
  }
  if (ctype == kBF16) return dispatch_fmt<kBF16, kAccumExact>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
  return dispatch_fmt<kF32, kAccumExact>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
}

}  // namespace fp8mi
