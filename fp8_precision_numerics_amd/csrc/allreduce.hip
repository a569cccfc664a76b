// One GPU's parts of an FP8 gradient all-reduce with automatic scaling.
//
// "FP8 and low-precision formats" (use cases): gradients travel as E5M2 to
// cut the inter-node bandwidth of distributed training.  "#fp8" tag page, the
// discussion of FP8 LLM training: "automatic scaling" adjusts the scaling
// factors so gradient values stay inside FP8's range during the all-reduce.
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: scale = MAX / amax,
// x(1/scale) restore, high-precision accumulation.
//
// With R ranks, each rank: amax of its gradient (the cast kernels' amax-only
// mode), a MAX all-reduce of that one float, the shared scale from the
// largest amax (shared_scale_kernel), the cast of its gradient with that
// scale, an all-to-all of the FP8 chunks, and the sum of the R chunks it
// receives in fp32, restored by x(1/scale) (dequant_sum_kernel).  Only the
// collectives need more than one GPU; these kernels are the rest.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

// One wave: m = the largest amax bit pattern over the R ranks (NaN above Inf
// above every finite value); scale = fp32(MAX / m) and its inverse when
// 0 < m < Inf and the quotient is finite, else both 1.
template <int FMT>
__global__ void shared_scale_kernel(const float* __restrict__ amaxes, int R, float* __restrict__ scale,
                                    float* __restrict__ scale_inv) {
  uint32_t m = 0;
  for (int r = threadIdx.x; r < R; r += 64) {
    const uint32_t b = f2u(amaxes[r]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  m = wave_max_u32(m);
  if (threadIdx.x == 0) {
    float s = 1.0f, si = 1.0f;
    if (!scale_from_amax_bits<FMT>(m, &s, &si)) {
      s = 1.0f;
      si = 1.0f;
    }
    *scale = s;
    *scale_inv = si;
  }
}

// Four FP8 codes (bytes of w) to fp32, exactly.
template <int FMT>
__device__ __forceinline__ v4f decode4(uint32_t w) {
  v2f lo, hi;
  if constexpr (FMT == kE4M3) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  return (v4f){lo[0], lo[1], hi[0], hi[1]};
}

typedef unsigned int ds_u2 __attribute__((ext_vector_type(2)));

// Four consecutive outputs, one 16-byte (fp32) or 8-byte (bf16) nontemporal store.
template <int OUT>
__device__ __forceinline__ void store_out4(void* out, int64_t i, const v4f& v) {
  if constexpr (OUT == kF32) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + i));
  } else {
    const v2bf lo = __builtin_convertvector((v2f){v[0], v[1]}, v2bf);
    const v2bf hi = __builtin_convertvector((v2f){v[2], v[3]}, v2bf);
    ds_u2 w;
    w[0] = __builtin_bit_cast(uint32_t, lo);
    w[1] = __builtin_bit_cast(uint32_t, hi);
    __builtin_nontemporal_store(w, reinterpret_cast<ds_u2*>(reinterpret_cast<uint16_t*>(out) + i));
  }
}

template <int OUT>
__device__ __forceinline__ void store_out1(void* out, int64_t i, float v) {
  if constexpr (OUT == kF32) {
    reinterpret_cast<float*>(out)[i] = v;
  } else {
    const v2bf b = __builtin_convertvector((v2f){v, 0.0f}, v2bf);
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)(__builtin_bit_cast(uint32_t, b) & 0xFFFFu);
  }
}

// The four codes at p, of which the first `m` lie inside the payload (m <= 0:
// none); codes past the end read as 0 and are never stored.
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* p, int64_t m) {
  if (m >= 4) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  uint32_t w = 0;
  for (int j = 0; j < m; ++j) w |= (uint32_t)p[j] << (8 * j);
  return w;
}

// out[i] = fp32(fp32(sum over r = 0..R-1, in that order, of dec(q[r*stride + i])) * scale_inv).
// A wave takes chunks of 1024 consecutive elements: four pieces 256 elements
// apart, four elements per lane and piece.  Every load is then one 4-byte word
// per lane and rank (256 contiguous bytes per wave) and every store 16 (fp32)
// or 8 (bf16) contiguous bytes per lane, contiguous across the wave; up to
// kBatch ranks' words are in flight at once, all accesses nontemporal (each
// byte is touched once).  Sixteen consecutive elements per lane (one 16-byte
// load per rank) ran 22 % slower on MI355X: each of its 16-byte stores
// covered only a quarter of the 64 bytes between neighbouring lanes.
constexpr int kBatch = 8, kChunk = 1024;

template <int FMT, int OUT>
__global__ __launch_bounds__(256) void dequant_sum_kernel(const uint8_t* __restrict__ q, int R, int64_t n,
                                                          int64_t stride, const float* __restrict__ scale_inv,
                                                          void* __restrict__ out) {
  const float si = scale_inv[0];
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  for (int64_t c = wave; c < nchunks; c += nwaves) {
    const int64_t e0 = c * kChunk + lane * 4;  // piece k covers [e0 + 256k, e0 + 256k + 4)
    v4f acc[4];
    for (int r0 = 0; r0 < R; r0 += kBatch) {
      uint32_t w[kBatch][4];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (r0 + b < R) {
          const uint8_t* row = q + (int64_t)(r0 + b) * stride;
#pragma unroll
          for (int k = 0; k < 4; ++k) w[b][k] = load_codes4(row + e0 + 256 * k, n - (e0 + 256 * k));
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (r0 + b >= R) break;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const v4f d = decode4<FMT>(w[b][k]);
          acc[k] = r0 + b == 0 ? d : acc[k] + d;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t e = e0 + 256 * k;
      const v4f o = acc[k] * si;
      if (e + 4 <= n) {
        store_out4<OUT>(out, e, o);
      } else {
        for (int j = 0; j < 4; ++j)
          if (e + j < n) store_out1<OUT>(out, e + j, o[j]);
      }
    }
  }
}

template <int FMT, int OUT>
hipError_t run_sum(const uint8_t* q, int R, int64_t n, int64_t stride, const float* si, void* out, hipStream_t st) {
  const int cus = persistent_groups(1);
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  int64_t blocks = (nchunks + 3) / 4;  // four waves per workgroup, one chunk each
  const int64_t cap = (int64_t)cus * 8;
  blocks = blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
  hipLaunchKernelGGL((dequant_sum_kernel<FMT, OUT>), dim3((unsigned)blocks), dim3(256), 0, st, q, R, n, stride, si,
                     out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shared_scale(const float* amaxes, int R, int fmt, float* scale, float* scale_inv,
                               hipStream_t stream) {
  if (fmt == kE4M3)
    hipLaunchKernelGGL(shared_scale_kernel<kE4M3>, dim3(1), dim3(64), 0, stream, amaxes, R, scale, scale_inv);
  else
    hipLaunchKernelGGL(shared_scale_kernel<kE5M2>, dim3(1), dim3(64), 0, stream, amaxes, R, scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_dequant_sum(const uint8_t* q, int R, int64_t n, int64_t stride, int fmt, const float* scale_inv,
                              void* out, int otype, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (fmt == kE4M3) {
    if (otype == kBF16) return run_sum<kE4M3, kBF16>(q, R, n, stride, scale_inv, out, stream);
    return run_sum<kE4M3, kF32>(q, R, n, stride, scale_inv, out, stream);
  }
  if (otype == kBF16) return run_sum<kE5M2, kBF16>(q, R, n, stride, scale_inv, out, stream);
  return run_sum<kE5M2, kF32>(q, R, n, stride, scale_inv, out, stream);
}

}  // namespace fp8mi
