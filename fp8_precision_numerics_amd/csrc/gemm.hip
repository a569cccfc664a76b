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
// whole bf16 or fp32 rows (gemm_requant.hip: FP8 rows re-quantised with the
// next consumer's scale).  With b_trans, B is stored [K x N]: its slabs are
// loaded in that orientation and the B fragments are read with the LDS
// transpose read, in the same K order as the [N x K] path (so the two give
// identical results).
#include "gemm_dispatch.hpp"
#include "launch.hpp"

namespace fp8mi {

template <bool BT>
hipError_t launch_gemm_t(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N, int64_t K,
                         const float* sinv_a, const float* sinv_b, void* C, int ctype, int accum, hipStream_t stream) {
  const RequantArgs none{nullptr, nullptr, nullptr};
  if (accum == kAccumMfma8) {
    if (ctype == kBF16) return gemm_dispatch_fmt<kBF16, kAccumMfma8, BT>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, none, stream);
    return gemm_dispatch_fmt<kF32, kAccumMfma8, BT>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, none, stream);
  }
  if (ctype == kBF16) return gemm_dispatch_fmt<kBF16, kAccumExact, BT>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, none, stream);
  return gemm_dispatch_fmt<kF32, kAccumExact, BT>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, none, stream);
}

hipError_t launch_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int b_trans, int64_t M, int64_t N,
                       int64_t K, const float* sinv_a, const float* sinv_b, void* C, int ctype,
                       int accum, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (b_trans) return launch_gemm_t<true>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, ctype, accum, stream);
  return launch_gemm_t<false>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, ctype, accum, stream);
}

}  // namespace fp8mi
