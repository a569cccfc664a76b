// Fused amax + scaled saturating FP8 cast (optionally with a transposed copy),
// and per-block current-scaling quantisation.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the FP8 tensor is
// round_to_fp8(tensor × scale) with scale ≈ FP8_MAX / amax; delayed scaling
// lets the cast use a scale known before the pass, so amax of this step and
// the cast come out of ONE read of the tensor.  "FP8 and low-precision
// formats", "Deep dive": scale factors are per tensor or per block.
//
// The per-tensor kernels are HBM-bound: per element they read 2 B (bf16) or
// 4 B (fp32) and write 1 B (2 B with the transposed copy).  Loads and stores are
// 16-B vectors; amax is an integer max over |bits| (exact and order-free),
// reduced across the wavefront with cross-lane shuffles, across the workgroup
// through LDS, and across workgroups with one atomicMax per workgroup.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

constexpr int kThreads = 256;

__global__ void zero_outputs_kernel(uint32_t* amax_bits, unsigned long long* sat) {
  if (threadIdx.x == 0) {
    if (amax_bits) *amax_bits = 0u;
    if (sat) *sat = 0ull;
  }
}

// Reduce (amax, count) over the workgroup and fold into the global outputs.
__device__ __forceinline__ void block_finish(uint32_t amx, uint32_t cnt, uint32_t* amax_bits,
                                             unsigned long long* sat) {
  __shared__ uint32_t s_max[kThreads / 64];
  __shared__ uint32_t s_cnt[kThreads / 64];
  amx = wave_max_u32(amx);
  cnt = wave_sum_u32(cnt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_max[wave] = amx;
    s_cnt[wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_max[0];
    unsigned long long c = s_cnt[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      m = m > s_max[w] ? m : s_max[w];
      c += s_cnt[w];
    }
    if (amax_bits) atomicMax(amax_bits, m);
    if (sat && c) atomicAdd(sat, c);
  }
}

// Load 8 consecutive input elements (16 B of bf16 or 32 B of fp32) as fp32.
template <int XT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t elem, float v[8]) {
  if constexpr (XT == kBF16) {
    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + elem);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + elem);
    const uint4 a = p[0], b = p[1];
    v[0] = u2f(a.x); v[1] = u2f(a.y); v[2] = u2f(a.z); v[3] = u2f(a.w);
    v[4] = u2f(b.x); v[5] = u2f(b.y); v[6] = u2f(b.z); v[7] = u2f(b.w);
  }
}

template <int XT>
__device__ __forceinline__ float load1(const void* __restrict__ x, int64_t elem) {
  if constexpr (XT == kBF16)
    return u2f((uint32_t)reinterpret_cast<const uint16_t*>(x)[elem] << 16);
  else
    return reinterpret_cast<const float*>(x)[elem];
}

// amax / saturation / cast of 8 values held in registers; returns the 8 codes.
template <int FMT, bool SAT>
__device__ __forceinline__ uint2 cast8(const float v[8], float s, uint32_t& amx, uint32_t& cnt) {
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t m = f2u(v[i]) & 0x7FFFFFFFu;
    amx = amx > m ? amx : m;
    p[i] = v[i] * s;
    if constexpr (SAT) cnt += is_saturated<FMT>(p[i]);
  }
  return make_uint2(encode4<FMT>(p[0], p[1], p[2], p[3]), encode4<FMT>(p[4], p[5], p[6], p[7]));
}

// ---------------------------------------------------------------------------
// Flat kernel: q (row-major) and/or amax; each thread owns 16-element chunks.
// ---------------------------------------------------------------------------
template <int XT, int FMT, bool WQ, bool SAT>
__global__ __launch_bounds__(kThreads) void quantize_flat_kernel(
    const void* __restrict__ x, int64_t n, const float* __restrict__ scale, uint8_t* __restrict__ q,
    uint32_t* __restrict__ amax_bits, unsigned long long* __restrict__ sat) {
  const float s = (WQ || SAT) ? *scale : 1.0f;
  uint32_t amx = 0u, cnt = 0u;
  const int64_t nchunk = n >> 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // Two chunks per trip so that each thread keeps 4 (bf16) or 8 (fp32) 16-B loads in flight.
  for (; c + stride < nchunk; c += 2 * stride) {
    float v0[8], v1[8], v2[8], v3[8];
    load8<XT>(x, c * 16, v0);
    load8<XT>(x, c * 16 + 8, v1);
    load8<XT>(x, (c + stride) * 16, v2);
    load8<XT>(x, (c + stride) * 16 + 8, v3);
    const uint2 a = cast8<FMT, SAT>(v0, s, amx, cnt);
    const uint2 b = cast8<FMT, SAT>(v1, s, amx, cnt);
    const uint2 d = cast8<FMT, SAT>(v2, s, amx, cnt);
    const uint2 e = cast8<FMT, SAT>(v3, s, amx, cnt);
    if constexpr (WQ) {
      reinterpret_cast<uint4*>(q)[c] = make_uint4(a.x, a.y, b.x, b.y);
      reinterpret_cast<uint4*>(q)[c + stride] = make_uint4(d.x, d.y, e.x, e.y);
    }
  }
  if (c < nchunk) {
    float v0[8], v1[8];
    load8<XT>(x, c * 16, v0);
    load8<XT>(x, c * 16 + 8, v1);
    const uint2 a = cast8<FMT, SAT>(v0, s, amx, cnt);
    const uint2 b = cast8<FMT, SAT>(v1, s, amx, cnt);
    if constexpr (WQ) reinterpret_cast<uint4*>(q)[c] = make_uint4(a.x, a.y, b.x, b.y);
  }
  // Ragged tail (n % 16 elements), element by element.
  if (blockIdx.x == 0 && threadIdx.x < (int)(n & 15)) {
    const int64_t i = (nchunk << 4) + threadIdx.x;
    const float v = load1<XT>(x, i);
    const uint32_t m = f2u(v) & 0x7FFFFFFFu;
    amx = amx > m ? amx : m;
    const float p = v * s;
    if constexpr (SAT) cnt += is_saturated<FMT>(p);
    if constexpr (WQ) q[i] = encode1<FMT>(p);
  }
  block_finish(amx, cnt, amax_bits, sat);
}

// ---------------------------------------------------------------------------
// Cast-transpose kernel: one 128x128 input tile per workgroup; writes q_t
// (and q when asked).  Codes pass through LDS as a [128 col][128 row] byte
// tile whose 16-B granules are XOR-swizzled by (col / 8) % 8 so that both the
// byte scatter and the 16-B row reads spread over the LDS banks.
// Requires rows % 16 == 0 and cols % 16 == 0.
// ---------------------------------------------------------------------------
constexpr int kTile = 128;

__device__ __forceinline__ int lds_t_offset(int col, int row) {
  return col * kTile + ((((row >> 4) ^ (col >> 3)) & 7) << 4) + (row & 15);
}

template <int XT, int FMT, bool WQ, bool SAT>
__global__ __launch_bounds__(kThreads) void quantize_transpose_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ scale,
    uint8_t* __restrict__ q, uint8_t* __restrict__ q_t, uint32_t* __restrict__ amax_bits,
    unsigned long long* __restrict__ sat) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kTile];
  const float s = *scale;
  const int64_t row0 = (int64_t)blockIdx.y * kTile, col0 = (int64_t)blockIdx.x * kTile;
  const int t = threadIdx.x;
  const int cc8 = (t & 15) * 8;  // column offset of this thread's 8 elements
  uint32_t amx = 0u, cnt = 0u;
#pragma unroll 2
  for (int i = 0; i < kTile / 16; ++i) {
    const int rr = i * 16 + (t >> 4);
    const int64_t r = row0 + rr, c = col0 + cc8;
    if (r < rows && c < cols) {
      float v[8];
      load8<XT>(x, r * cols + c, v);
      const uint2 w = cast8<FMT, SAT>(v, s, amx, cnt);
      if constexpr (WQ) *reinterpret_cast<uint2*>(q + r * cols + c) = w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[lds_t_offset(cc8 + j, rr)] = (uint8_t)(w.x >> (8 * j));
        tile[lds_t_offset(cc8 + 4 + j, rr)] = (uint8_t)(w.y >> (8 * j));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTile / 32; ++i) {
    const int cc = i * 32 + (t >> 3), g = t & 7;
    const int64_t c = col0 + cc, r = row0 + g * 16;
    if (c < cols && r < rows) {
      const uint4 v = *reinterpret_cast<const uint4*>(&tile[lds_t_offset(cc, g * 16)]);
      *reinterpret_cast<uint4*>(q_t + c * rows + r) = v;
    }
  }
  block_finish(amx, cnt, amax_bits, sat);
}

// ---------------------------------------------------------------------------
// Per-block current scaling.
// 1 x 128 tiles: 16 lanes per tile, 8 elements per lane.
// ---------------------------------------------------------------------------
template <int XT, int FMT>
__global__ __launch_bounds__(kThreads) void quantize_rowtile_kernel(const void* __restrict__ x,
                                                                    int64_t rows, int64_t cols,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale_inv) {
  const int64_t ntc = (cols + 127) / 128;
  const int64_t ntiles = rows * ntc;
  const int sub = threadIdx.x & 15;
  const int64_t groups = (int64_t)gridDim.x * (kThreads / 16);
  for (int64_t tile = (int64_t)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4); tile < ntiles;
       tile += groups) {
    // All 16 lanes of a group share `tile`, so the loop trip count is uniform per group;
    // the shuffles below stay inside the group (xor offsets < 16).
    const int64_t r = tile / ntc, tc = tile - r * ntc;
    const int64_t c = tc * 128 + sub * 8;
    const bool valid = c < cols;
    float v[8];
    if (valid) {
      load8<XT>(x, r * cols + c, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = f2u(v[i]) & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
      m = m > o ? m : o;
    }
    float s = 1.0f, si = 1.0f;
    scale_from_amax_bits<FMT>(m, &s, &si);
    if (valid) {
      uint32_t dummy_a = 0u, dummy_c = 0u;
      const uint2 w = cast8<FMT, false>(v, s, dummy_a, dummy_c);
      *reinterpret_cast<uint2*>(q + r * cols + c) = w;
    }
    if (sub == 0) scale_inv[tile] = si;
  }
}

// 128 x 128 blocks: one workgroup per block, 64 elements per thread held in registers.
template <int XT, int FMT>
__global__ __launch_bounds__(kThreads) void quantize_block128_kernel(const void* __restrict__ x,
                                                                     int64_t rows, int64_t cols,
                                                                     uint8_t* __restrict__ q,
                                                                     float* __restrict__ scale_inv) {
  __shared__ uint32_t s_max[kThreads / 64];
  const int64_t row0 = (int64_t)blockIdx.y * 128, col0 = (int64_t)blockIdx.x * 128;
  const int t = threadIdx.x;
  const int64_t c = col0 + (t & 15) * 8;
  float v[8][8];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 16 + (t >> 4);
    if (r < rows && c < cols) {
      load8<XT>(x, r * cols + c, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t a = f2u(v[i][j]) & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
  }
  m = wave_max_u32(m);
  if ((t & 63) == 0) s_max[t >> 6] = m;
  __syncthreads();
  m = s_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = m > s_max[w] ? m : s_max[w];
  float s = 1.0f, si = 1.0f;
  scale_from_amax_bits<FMT>(m, &s, &si);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 16 + (t >> 4);
    if (r < rows && c < cols) {
      uint32_t dummy_a = 0u, dummy_c = 0u;
      *reinterpret_cast<uint2*>(q + r * cols + c) = cast8<FMT, false>(v[i], s, dummy_a, dummy_c);
    }
  }
  if (t == 0) scale_inv[blockIdx.y * gridDim.x + blockIdx.x] = si;
}

// ---------------------------------------------------------------------------
// Launch helpers (template dispatch).
// ---------------------------------------------------------------------------
int flat_grid(int64_t nchunk) {
  // Enough workgroups to cover the tensor in at most ~2 trips of the 2-chunk loop,
  // capped so that small tensors launch few groups.
  int64_t g = (nchunk + 2 * kThreads - 1) / (2 * kThreads);
  if (g < 1) g = 1;
  if (g > 16384) g = 16384;
  return (int)g;
}

template <int XT, int FMT, bool WQ, bool SAT>
void launch_flat_t(const void* x, int64_t n, const float* scale, uint8_t* q, uint32_t* amax_bits,
                   unsigned long long* sat, hipStream_t st) {
  hipLaunchKernelGGL((quantize_flat_kernel<XT, FMT, WQ, SAT>), dim3(flat_grid(n >> 4)),
                     dim3(kThreads), 0, st, x, n, scale, q, amax_bits, sat);
}

template <int XT, int FMT>
void launch_flat_f(const void* x, int64_t n, const float* scale, uint8_t* q, uint32_t* amax_bits,
                   unsigned long long* sat, hipStream_t st) {
  if (q && sat) launch_flat_t<XT, FMT, true, true>(x, n, scale, q, amax_bits, sat, st);
  else if (q) launch_flat_t<XT, FMT, true, false>(x, n, scale, q, amax_bits, sat, st);
  else if (sat) launch_flat_t<XT, FMT, false, true>(x, n, scale, q, amax_bits, sat, st);
  else launch_flat_t<XT, FMT, false, false>(x, n, scale, q, amax_bits, sat, st);
}

template <int XT, int FMT>
void launch_transpose_f(const void* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q,
                        uint8_t* q_t, uint32_t* amax_bits, unsigned long long* sat,
                        hipStream_t st) {
  const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
  if (q && sat)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, true, true>), grid, dim3(kThreads), 0, st,
                       x, rows, cols, scale, q, q_t, amax_bits, sat);
  else if (q)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, true, false>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat);
  else if (sat)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, false, true>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat);
  else
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, false, false>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat);
}

template <int XT>
void launch_quantize_x(const void* x, int64_t rows, int64_t cols, int fmt, const float* scale,
                       uint8_t* q, uint8_t* q_t, uint32_t* amax_bits, unsigned long long* sat,
                       hipStream_t st) {
  const int64_t n = rows * cols;
  if (q_t) {
    if (fmt == kE4M3) launch_transpose_f<XT, kE4M3>(x, rows, cols, scale, q, q_t, amax_bits, sat, st);
    else launch_transpose_f<XT, kE5M2>(x, rows, cols, scale, q, q_t, amax_bits, sat, st);
  } else {
    if (fmt == kE4M3) launch_flat_f<XT, kE4M3>(x, n, scale, q, amax_bits, sat, st);
    else launch_flat_f<XT, kE5M2>(x, n, scale, q, amax_bits, sat, st);
  }
}

template <int XT, int FMT>
void launch_blockwise_t(const void* x, int64_t rows, int64_t cols, int block_rows, uint8_t* q,
                        float* scale_inv, hipStream_t st) {
  if (block_rows == 1) {
    const int64_t ntiles = rows * ((cols + 127) / 128);
    int64_t g = (ntiles + (kThreads / 16) - 1) / (kThreads / 16);
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL((quantize_rowtile_kernel<XT, FMT>), dim3((unsigned)g), dim3(kThreads), 0, st,
                       x, rows, cols, q, scale_inv);
  } else {
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    hipLaunchKernelGGL((quantize_block128_kernel<XT, FMT>), grid, dim3(kThreads), 0, st, x, rows,
                       cols, q, scale_inv);
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int xtype, int64_t rows, int64_t cols, int fmt,
                           const float* scale, uint8_t* q, uint8_t* q_t, float* amax,
                           unsigned long long* sat, hipStream_t stream) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(amax);
  if (amax_bits || sat)
    hipLaunchKernelGGL(zero_outputs_kernel, dim3(1), dim3(64), 0, stream, amax_bits, sat);
  if (rows * cols > 0) {
    if (xtype == kBF16)
      launch_quantize_x<kBF16>(x, rows, cols, fmt, scale, q, q_t, amax_bits, sat, stream);
    else
      launch_quantize_x<kF32>(x, rows, cols, fmt, scale, q, q_t, amax_bits, sat, stream);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_blockwise(const void* x, int xtype, int64_t rows, int64_t cols,
                                     int block_rows, int fmt, uint8_t* q, float* scale_inv,
                                     hipStream_t stream) {
  if (rows * cols == 0) return hipSuccess;
  if (xtype == kBF16) {
    if (fmt == kE4M3) launch_blockwise_t<kBF16, kE4M3>(x, rows, cols, block_rows, q, scale_inv, stream);
    else launch_blockwise_t<kBF16, kE5M2>(x, rows, cols, block_rows, q, scale_inv, stream);
  } else {
    if (fmt == kE4M3) launch_blockwise_t<kF32, kE4M3>(x, rows, cols, block_rows, q, scale_inv, stream);
    else launch_blockwise_t<kF32, kE5M2>(x, rows, cols, block_rows, q, scale_inv, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8mi
