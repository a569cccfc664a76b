// Delayed-scaling history step: push this step's amax into the ring, take
// the max over the ring, derive the scale the next cast will use.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4 (delayed scaling: predict
// this step's scale from the amax history of past steps, e.g. the max of the
// last N) and §4.2.6 (recipe: amax_history_len = 16, amax_compute_algo =
// "max"; TE refreshes amax internally to set the next step's scale).
//
// One wavefront does the whole update on the device, so the delayed-scaling
// loop never needs the host: the scale stays in HBM between the update and the
// next fp8_quantize.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

template <int FMT>
__global__ __launch_bounds__(64) void amax_update_kernel(float* __restrict__ history, int len,
                                                         int32_t* __restrict__ head,
                                                         const float* __restrict__ amax,
                                                         float* __restrict__ scale,
                                                         float* __restrict__ scale_inv,
                                                         int32_t* __restrict__ status) {
  const int lane = threadIdx.x;
  int h = *head;
  int flags = 0;
  if (h < 0 || h >= len) {
    h = 0;
    flags |= 2;
  }
  const uint32_t a_bits = f2u(*amax);
  uint32_t m = 0u;
  for (int i = lane; i < len; i += 64) {
    // Every slot is loaded, the one at the head replaced afterwards: a load
    // made conditional on the head waited for the head's own load first.
    const uint32_t stored = f2u(history[i]);
    const uint32_t b = (i == h) ? a_bits : stored;
    const uint32_t mag = b & 0x7FFFFFFFu;  // the amax is a magnitude; keep the rule sign-free
    m = m > mag ? m : mag;
  }
  m = wave_max_u32(m);
  if (lane == 0) {
    history[h] = u2f(a_bits);
    *head = (h + 1 == len) ? 0 : h + 1;
    float s, si;
    if (scale_from_amax_bits<FMT>(m, &s, &si)) {
      *scale = s;
      *scale_inv = si;
    } else {
      flags |= 1;
    }
    if (status && flags) *status |= flags;
  }
}

}  // namespace

hipError_t launch_amax_update(float* history, int history_len, int32_t* head, const float* amax,
                              int fmt, float* scale, float* scale_inv, int32_t* status,
                              hipStream_t stream) {
  if (fmt == kE4M3)
    hipLaunchKernelGGL(amax_update_kernel<kE4M3>, dim3(1), dim3(64), 0, stream, history,
                       history_len, head, amax, scale, scale_inv, status);
  else
    hipLaunchKernelGGL(amax_update_kernel<kE5M2>, dim3(1), dim3(64), 0, stream, history,
                       history_len, head, amax, scale, scale_inv, status);
  return hipGetLastError();
}

}  // namespace fp8mi
