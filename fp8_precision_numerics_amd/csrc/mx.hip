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
// The quantiser works on tiles of 64 rows x 16 blocks (512 columns).  Four
// lanes share a block (8 values each: one 16-byte bf16 load or two fp32 loads
// per lane and row), so a wave covers the tile's 16 blocks of one row; each of
// eight waves takes eight rows, four rows' loads in flight at a time.  The
// block amax comes from two lane exchanges; each lane writes its 8 codes, and
// the scale bytes, K-block major so that the GEMM's per-step scale loads are
// contiguous, are gathered in LDS and leave as one 64-byte run per block.  The GEMM is the dense kernel's FP8 path with the
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
// the GEMM reads (gemm_kernel.hpp, MxScaleLoader).  A tile's 64 rows are one
// such group, so its scales for block b are the 64 bytes at b * ld + r0: they
// are collected in LDS at the permuted positions and written one dword per
// lane (bytes only in a group cut by the last row: positions of rows past the
// end stay unwritten).  Writing each block's byte straight from its lane
// scattered 16 single-byte stores over 16 lines per wave instruction, and the
// kernel ran at 3.8-4.0 TB/s against 5.3-5.7 TB/s now on MI355X, as fast as
// the same kernel with its scale stores removed.  The input is read and the
// codes written with nontemporal accesses (streamed once).
constexpr int kMxTileRows = 64, kMxTileBlocks = 16, kMxWaves = 8;
constexpr int kMxRowsPerWave = kMxTileRows / kMxWaves, kMxU = 4;  // rows in flight per wave

typedef unsigned int mx_u4 __attribute__((ext_vector_type(4)));
typedef unsigned int mx_u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 mx_load16(const void* p, int64_t vi) {
  const mx_u4 r = __builtin_nontemporal_load(reinterpret_cast<const mx_u4*>(p) + vi);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int FMT, int XT>
__global__ __launch_bounds__(64 * kMxWaves) void quantize_mx_kernel(const void* __restrict__ x, int64_t rows,
                                                                    int64_t cols, int64_t nbr, int64_t ld,
                                                                    uint8_t* __restrict__ q,
                                                                    uint8_t* __restrict__ scales, int64_t tiles_b,
                                                                    int64_t ntiles) {
  __shared__ uint32_t sc_words[kMxTileBlocks * 16];  // 16 blocks x 64 bytes
  uint8_t* const sc = reinterpret_cast<uint8_t*>(sc_words);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // Tile and row loops are uniform per workgroup: every lane reaches every
  // barrier and every lane exchange (a block's four lanes are a quad).
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / tiles_b) * kMxTileRows, b0 = (tile % tiles_b) * kMxTileBlocks;
    const bool col_ok = b0 + (lane >> 2) < nbr;
    const int64_t c0 = b0 * 32 + lane * 8;  // this lane's 8 values of a row: columns [c0, c0 + 8)
#pragma unroll 1
    for (int it = 0; it < kMxRowsPerWave; it += kMxU) {
      uint4 raw[kMxU][XT == kBF16 ? 1 : 2];
#pragma unroll
      for (int u = 0; u < kMxU; ++u) {
        const int64_t r = r0 + w * kMxRowsPerWave + it + u, e = r * cols + c0;
        if (col_ok && r < rows) {
          if constexpr (XT == kBF16) {
            raw[u][0] = mx_load16(x, e >> 3);
          } else {
            raw[u][0] = mx_load16(x, e >> 2);
            raw[u][1] = mx_load16(x, (e >> 2) + 1);
          }
        } else {
#pragma unroll
          for (int h = 0; h < (XT == kBF16 ? 1 : 2); ++h) raw[u][h] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < kMxU; ++u) {
        const int rr = w * kMxRowsPerWave + it + u;  // row within the tile
        const int64_t r = r0 + rr;
        const bool live = col_ok && r < rows;
        float v[8];
        if constexpr (XT == kBF16) {
          const uint4 wv = raw[u][0];
          v[0] = bf16_lo(wv.x); v[1] = bf16_hi(wv.x); v[2] = bf16_lo(wv.y); v[3] = bf16_hi(wv.y);
          v[4] = bf16_lo(wv.z); v[5] = bf16_hi(wv.z); v[6] = bf16_lo(wv.w); v[7] = bf16_hi(wv.w);
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
        uint32_t o = (uint32_t)__shfl_xor((int)m, 1, 64);
        m = o > m ? o : m;
        o = (uint32_t)__shfl_xor((int)m, 2, 64);
        m = o > m ? o : m;
        if (!live) continue;
        const bool finite = m < 0x7F800000u;
        const int e = (finite && m != 0u) ? mx_exponent<FMT>(m) : 0;
        const float s = pow2_neg(e);
        uint32_t cw0, cw1;
        if (finite) {
          cw0 = encode4_finite<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
          cw1 = encode4_finite<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
        } else {
          cw0 = encode4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
          cw1 = encode4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
        }
        mx_u2 cw;
        cw[0] = cw0;
        cw[1] = cw1;
        __builtin_nontemporal_store(cw, reinterpret_cast<mx_u2*>(q) + ((r * cols + c0) >> 3));
        if ((lane & 3) == 0) sc[(lane >> 2) * 64 + mx_scale_pos(rr)] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
    // Dword d of block b's run holds rows d, d+16, d+32, d+48 of the group.
    for (int t = threadIdx.x; t < kMxTileBlocks * 16; t += 64 * kMxWaves) {
      const int b = t >> 4, d = t & 15;
      if (b0 + b >= nbr) continue;
      uint8_t* dst = scales + (b0 + b) * ld + r0 + 4 * d;
      const uint32_t word = sc_words[t];
      if (r0 + kMxTileRows <= rows) {
        *reinterpret_cast<uint32_t*>(dst) = word;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (r0 + d + 16 * k < rows) dst[k] = (uint8_t)(word >> (8 * k));
      }
    }
    __syncthreads();  // the LDS run buffer is free for the next tile
  }
}

template <int FMT, int XT>
hipError_t run_quantize_mx(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int cus = persistent_groups(1);
  const int64_t nbr = cols / 32, ld = mx_scale_ld(rows);
  const int64_t tiles_b = (nbr + kMxTileBlocks - 1) / kMxTileBlocks;
  const int64_t ntiles = (rows + kMxTileRows - 1) / kMxTileRows * tiles_b;
  const int64_t cap = (int64_t)cus * 4;  // four workgroups of eight waves per CU
  const int64_t blocks = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL((quantize_mx_kernel<FMT, XT>), dim3((unsigned)blocks), dim3(64 * kMxWaves), 0, st, x, rows,
                     cols, nbr, ld, q, scales, tiles_b, ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mx(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                              uint8_t* scales, hipStream_t stream) {
  if (rows == 0 || cols < 32) return hipSuccess;
  if (fmt == kE4M3) {
    if (xtype == kBF16) return run_quantize_mx<kE4M3, kBF16>(x, rows, cols, q, scales, stream);
    return run_quantize_mx<kE4M3, kF32>(x, rows, cols, q, scales, stream);
  }
  if (xtype == kBF16) return run_quantize_mx<kE5M2, kBF16>(x, rows, cols, q, scales, stream);
  return run_quantize_mx<kE5M2, kF32>(x, rows, cols, q, scales, stream);
}

hipError_t launch_gemm_mx(const uint8_t* A, int fa, const uint8_t* sa, const uint8_t* B, int fb, const uint8_t* sb,
                          int64_t M, int64_t N, int64_t K, void* C, int ctype, int accum, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const RequantArgs none{nullptr, nullptr, nullptr};
  const MxScales mxs{sa, sb};
  if (accum == kAccumExact) {
    if (ctype == kBF16)
      return gemm_dispatch_fmt<kBF16, kAccumMxExact>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
    return gemm_dispatch_fmt<kF32, kAccumMxExact>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
  }
  if (ctype == kBF16)
    return gemm_dispatch_fmt<kBF16, kAccumMx>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
  return gemm_dispatch_fmt<kF32, kAccumMx>(A, fa, B, fb, M, N, K, nullptr, nullptr, C, none, stream, mxs);
}

}  // namespace fp8mi
