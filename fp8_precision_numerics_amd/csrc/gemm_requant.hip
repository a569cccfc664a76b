// FP8 GEMM whose epilogue re-quantises the result to FP8 with the next
// consumer's scale, recording the result's amax and saturation count.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the GEMM output is restored
// by x(1/scale) of its operands, or that factor is combined with the next
// stage's scale so the result goes on in FP8; each FP8 tensor's amax feeds its
// own delayed-scaling history.
//
// The kernel is the dense one (gemm_kernel.hpp) with an FP8 output kind: the
// accumulation is unchanged, c = acc x sinv_a x sinv_b is the fp32 value the
// fp32-output GEMM stores, and the epilogue writes round_to_fp8(fp32(c x s))
// through the same LDS-staged row writer (one byte per output), so the result
// equals casting the fp32 output with fp8_quantize, without the fp32 round trip
// through HBM.
#include "gemm_dispatch.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

__global__ void clear_requant_stats(uint32_t* amax_bits, unsigned long long* sat) {
  if (threadIdx.x == 0) {
    if (amax_bits) *amax_bits = 0u;
    if (sat) *sat = 0ull;
  }
}

template <int OUT>
hipError_t by_mode(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N, int64_t K,
                   const float* sa, const float* sb, uint8_t* Cq, const RequantArgs& rq, int accum,
                   hipStream_t st) {
  if (accum == kAccumMfma8) return gemm_dispatch_fmt<OUT, kAccumMfma8>(A, fa, B, fb, M, N, K, sa, sb, Cq, rq, st);
  return gemm_dispatch_fmt<OUT, kAccumExact>(A, fa, B, fb, M, N, K, sa, sb, Cq, rq, st);
}

}  // namespace

hipError_t launch_gemm_requant(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                               int64_t K, const float* sinv_a, const float* sinv_b, int out_fmt,
                               const float* out_scale, uint8_t* Cq, float* amax, unsigned long long* sat,
                               int accum, hipStream_t stream) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(amax);
  if (amax_bits || sat) {
    hipLaunchKernelGGL(clear_requant_stats, dim3(1), dim3(64), 0, stream, amax_bits, sat);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipSuccess;
  const RequantArgs rq{out_scale, amax_bits, sat};
  if (out_fmt == kE4M3) return by_mode<kOutE4M3>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, Cq, rq, accum, stream);
  return by_mode<kOutE5M2>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, Cq, rq, accum, stream);
}

}  // namespace fp8mi
