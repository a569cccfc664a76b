// MXFP8: FP8 elements with one power-of-two scale per 32 consecutive values of
// a row, and the GEMM on such operands.
//
// "FP8 and low-precision formats", "Deep dive": per-tensor or per-block scale
// factors keep values in FP8's usable range; MXFP8 goes further with shared
// micro-scaling blocks.  "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the
// scale is set from the amax so the values fit the format (MAX / amax).  Here a
// block's scale is 2^e with e the smallest integer such that amax <= MAX * 2^e
// (stored as the 8-bit exponent code e + 127), and each element is
// round_to_fp8(x * 2^-e) with the cast's rule.
//
// The quantiser gives four lanes to a block (8 values each: one 16-byte bf16
// load or two fp32 loads per lane and piece; a wave covers 16 consecutive
// blocks per piece, four pieces per iteration), takes
// the block amax with two lane exchanges, and writes 8 codes per lane and one
// scale byte per block, K-block major so that the GEMM's per-step scale loads
// are contiguous.  The GEMM is the dense kernel's FP8 path with the
// scaled matrix-core instruction: V_MFMA_SCALE_F32_16X16X128_F8F6F4 takes, per
// lane, the E8M0 byte of the 32-deep K block that lane's fragment covers, for
// each operand, and applies both powers of two to the products (measured on
// MI355X: the first operand's scale follows its rows and K blocks, the
// second's likewise).
#include "gemm_dispatch.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

// Smallest e with amax <= MAX * 2^e for a finite, non-zero amax given as bits
// (MAX = 1.75 * 2^EMAX for both formats), clamped to [-127, 127].
template <int FMT>
__device__ __forceinline__ int mx_exponent(uint32_t bits) {
  constexpr int kEmax = FMT == kE4M3 ? 8 : 15;
  int E;                 // amax = m * 2^E with m in [1, 2)
  bool above;            // m > 1.75
  const uint32_t ef = bits >> 23, mant = bits & 0x7FFFFFu;
  if (ef != 0) {
    E = (int)ef - 127;
    above = mant > 0x600000u;
  } else {               // subnormal: mant * 2^-149, leading bit at position p
    const int p = 31 - __builtin_clz(mant);
    E = p - 149;
    above = (mant << 2) > (7u << p);
  }
  int e = E - kEmax + (above ? 1 : 0);
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e;
}

// 2^-e as an fp32 value, e in [-127, 127] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_neg(int e) {
  return e <= 126 ? u2f((uint32_t)(127 - e) << 23) : u2f(0x00400000u);
}

// Scale bytes go K-block major, rows permuted within groups of 64 (block b of
// row r at b * ld + mx_scale_pos(r); ld = rows rounded up to 64), the layout
// the GEMM reads (gemm_kernel.hpp, MxScaleLoader).  Each lane takes kMxU
// eight-value pieces per iteration (a wave: kMxU runs of 16 consecutive
// blocks), all loaded before any is used; the input is read and the codes
// written with nontemporal accesses (streamed once).  With one 16-B load in
// flight per lane the kernel ran at 3.5 TB/s on MI355X.
constexpr int kMxU = 4;

typedef unsigned int mx_u4 __attribute__((ext_vector_type(4)));
typedef unsigned int mx_u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 mx_load16(const void* p, int64_t vi) {
  const mx_u4 r = __builtin_nontemporal_load(reinterpret_cast<const mx_u4*>(p) + vi);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int FMT, int XT>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const void* __restrict__ x, int64_t nblocks, int64_t nbr,
                                                          int64_t ld, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ scales) {
  const int64_t lanes = nblocks * 4;  // one lane-piece = 8 values; four pieces = one block
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  // The loop bound is uniform per wave: every lane runs the same iterations
  // (the lane exchanges need the whole quad).
  for (int64_t base = wave * (64 * kMxU); base < lanes; base += nwaves * (64 * kMxU)) {
    uint4 raw[kMxU][XT == kBF16 ? 1 : 2];
#pragma unroll
    for (int u = 0; u < kMxU; ++u) {
      const int64_t i = base + u * 64 + lane;  // this piece's 8 values: [8i, 8i + 8)
      if (i < lanes) {
        if constexpr (XT == kBF16) {
          raw[u][0] = mx_load16(x, i);
        } else {
          raw[u][0] = mx_load16(x, 2 * i);
          raw[u][1] = mx_load16(x, 2 * i + 1);
        }
      } else {
#pragma unroll
        for (int h = 0; h < (XT == kBF16 ? 1 : 2); ++h) raw[u][h] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < kMxU; ++u) {
      const int64_t i = base + u * 64 + lane;
      const bool live = i < lanes;
      float v[8];
      if constexpr (XT == kBF16) {
        const uint4 w = raw[u][0];
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
      } else {
        const uint4 a = raw[u][0], b = raw[u][1];
        v[0] = u2f(a.x); v[1] = u2f(a.y); v[2] = u2f(a.z); v[3] = u2f(a.w);
        v[4] = u2f(b.x); v[5] = u2f(b.y); v[6] = u2f(b.z); v[7] = u2f(b.w);
      }
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t bits = f2u(v[k]) & 0x7FFFFFFFu;
        m = bits > m ? bits : m;
      }
      // the block's four lanes are a quad (lane & ~3)
      uint32_t o = (uint32_t)__shfl_xor((int)m, 1, 64);
      m = o > m ? o : m;
      o = (uint32_t)__shfl_xor((int)m, 2, 64);
      m = o > m ? o : m;
      if (!live) continue;
      const bool finite = m < 0x7F800000u;
      const int e = (finite && m != 0u) ? mx_exponent<FMT>(m) : 0;
      const float s = pow2_neg(e);
      uint32_t c0, c1;
      if (finite) {
        c0 = encode4_finite<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
        c1 = encode4_finite<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
      } else {
        c0 = encode4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
        c1 = encode4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
      }
      mx_u2 cw;
      cw[0] = c0;
      cw[1] = c1;
      __builtin_nontemporal_store(cw, reinterpret_cast<mx_u2*>(q) + i);
      if ((i & 3) == 0) {
        const int64_t blk = i >> 2, r = blk / nbr;
        scales[(blk - r * nbr) * ld + mx_scale_pos(r)] = (uint8_t)(e + 127);
      }
    }
  }
}

template <int FMT, int XT>
hipError_t run_quantize_mx(const void* x, int64_t nblocks, int64_t nbr, int64_t ld, uint8_t* q, uint8_t* scales,
                           hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t lanes = nblocks * 4;
  int64_t blocks = (lanes + 256 * kMxU - 1) / (256 * kMxU);
  const int64_t cap = (int64_t)cus * 8;
  blocks = blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
  hipLaunchKernelGGL((quantize_mx_kernel<FMT, XT>), dim3((unsigned)blocks), dim3(256), 0, st, x, nblocks, nbr, ld, q,
                     scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mx(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                              uint8_t* scales, hipStream_t stream) {
  const int64_t nbr = cols / 32, nblocks = rows * nbr, ld = mx_scale_ld(rows);
  if (nblocks == 0) return hipSuccess;
  if (fmt == kE4M3) {
    if (xtype == kBF16) return run_quantize_mx<kE4M3, kBF16>(x, nblocks, nbr, ld, q, scales, stream);
    return run_quantize_mx<kE4M3, kF32>(x, nblocks, nbr, ld, q, scales, stream);
  }
  if (xtype == kBF16) return run_quantize_mx<kE5M2, kBF16>(x, nblocks, nbr, ld, q, scales, stream);
  return run_quantize_mx<kE5M2, kF32>(x, nblocks, nbr, ld, q, scales, stream);
}

hipError_t launch_gemm_mx(const uint8_t* A, int fa, const uint8_t* sa, const uint8_t* B, int fb, const uint8_t* sb,
                          int64_t M, int64_t N, int64_t K, void* C, int ctype, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const RequantArgs none{nullptr, nullptr, nullptr};
  const MxScales mxs{sa, sb};
  if (ctype == kBF16)
    return gemm_dispatch_fmt<kBF16, kAccumMx>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
  return gemm_dispatch_fmt<kF32, kAccumMx>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
}

}  // namespace fp8mi
