// Shared building blocks of the FP8 GEMM kernels (dense and grouped).
//
// Two ways to contract FP8 operands on gfx950 (selected per call):
//
// * kAccumExact — every product exact, sums in fp32.  The FP8 codes are
//   widened in registers to bf16 (exact for both E4M3 and E5M2, subnormals
//   included: V_CVT_SCALEF32_PK_BF16_FP8/BF8 with scale 1; bf16 keeps 8
//   significant bits and fp32's exponent range) and contracted with
//   V_MFMA_F32_32X32X16_BF16, whose products of such values are exact and whose
//   sums are fp32 (no loss was found).  This is "GEMM in FP8, FP32
//   accumulation" in the sense of "4.2 Hopper I — Transformer Engine·FP8"
//   §4.2.4: the result meets 1e-5·Σ|ab| for every input.  (The fp16
//   instruction, fed fp16-widened codes, returns the same bits; the bf16 one
//   measured 1-1.5 % faster on MI355X.)
//
// * kAccumMfma8 — the native FP8 matrix-core instruction
//   V_MFMA_F32_16X16X128_F8F6F4.  Measured on MI355X: it forms dot products of
//   8 consecutive K terms in fixed point whose last bit lies 13 bits below
//   the largest product of the 8, truncating the rest toward zero, and adds
//   those partials in fp32.  Twice the rate of the bf16 path; the per-group
//   truncation (at most 8·2^-13 of the group's largest product) is its
//   accuracy price.
//
// Operand lanes.  16x16x128 (FP8 path): lane l supplies row l % 16 of each
// operand and 32 bytes of the 128-deep K step: the instruction takes the first
// 16 bytes of lane group h = l / 16 as K 16h .. 16h+15 and the last 16 as
// K 64+16h .. 64+16h+15 (measured on MI355X), and in its block-scaled form
// (MXFP8) applies the E8M0 scale that lane group b supplies to K 32b .. 32b+31.
// Unscaled, the kernels simply give lane group h the 32-byte slice h; scaled,
// they give it the 16-byte pieces h and h + 4, so the hardware's K blocks are
// the operand's.  32x32x16
// (bf16 paths): lane l supplies row l % 32 and the 64-byte half l / 32 of the
// step, of which sub-step s (16 deep) takes bytes [8s, 8s+8).  Any assignment
// of K values to (lane, register) slots works as long as both operands use the
// same one.  The kernels feed the B tile (rows = n) as the instruction's first
// operand and the A tile (rows = m) as its second, so each lane's accumulators
// hold one output row m and runs of FOUR CONSECUTIVE columns n.
//
// Operand tiles live in LDS as rows of 128 bytes (one K step); the 16-byte
// granule g of row r sits at position g ^ swz(r) with
// swz(r) = (r & 6) | ((r >> 3) & 1).  A fragment read (16 lanes on 16
// consecutive rows, same granule; lanes 16..63 at granules +2, +4, +6) runs at
// full LDS rate under this map.  The map was chosen by timing ds_read_b128 on
// MI355X over every GF(2)-linear map from the row's low four bits to the
// position: the plain g ^ (r & 7) and g ^ ((r >> 1) & 7) maps run at half
// rate, an unswizzled tile at a quarter.  The direct-to-LDS loads write 1 KiB
// contiguous per wave instruction, which the swizzle does not affect.
#pragma once

#include "device_common.hpp"

namespace fp8mi {

constexpr int kBK = 128;  // K bytes per main-loop step
// kAccumMx: the FP8 instruction with a power-of-two (E8M0) scale per 32-deep K
// block of each operand row (MXFP8), applied by the instruction itself.
// kAccumMxExact: MXFP8 operands with every product exact and fp32 sums: the
// codes are widened to bf16 as in kAccumExact but with the block's power of
// two relative to the row's largest block exponent folded into the conversion
// (still exact: the value keeps at most 4 significant bits inside bf16's
// exponent range), contracted the same way, and the two rows' reference powers
// of two are applied in the epilogue.
enum : int { kAccumExact = 0, kAccumMfma8 = 1, kAccumMx = 2, kAccumMxExact = 3 };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lds_swz(int row) { return (row & 6) | ((row >> 3) & 1); }
__device__ __forceinline__ int lds_granule(int row, int g) { return row * kBK + (((g ^ lds_swz(row)) & 7) << 4); }

template <int FA, int FB>
__device__ __forceinline__ v4f mfma_fp8(const v8i& first, const v8i& second, const v4f& c) {
  // Scale operands are zero, which selects the plain (unscaled) instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, FA, FB, 0, 0, 0, 0);
}

// The block-scaled form: s1 / s2 hold E8M0 codes, byte sel1 / sel2 of each is
// the scale of this lane's K block of the first / second operand.  The byte
// selectors are instruction fields, so they must be compile-time constants:
// in the kernels' unrolled loops every call resolves to one case.
template <int F1, int F2>
__device__ __forceinline__ v4f mfma_fp8_scaled(const v8i& first, const v8i& second, const v4f& c, int sel1, int s1,
                                               int sel2, int s2) {
  switch (sel1 * 4 + sel2) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 0, s1, 0, s2);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 0, s1, 1, s2);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 0, s1, 2, s2);
    case 3: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 0, s1, 3, s2);
    case 4: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 1, s1, 0, s2);
    case 5: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 1, s1, 1, s2);
    case 6: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 1, s1, 2, s2);
    case 7: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 1, s1, 3, s2);
    case 8: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 2, s1, 0, s2);
    case 9: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 2, s1, 1, s2);
    case 10: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 2, s1, 2, s2);
    case 11: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 2, s1, 3, s2);
    case 12: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 3, s1, 0, s2);
    case 13: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 3, s1, 1, s2);
    case 14: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 3, s1, 2, s2);
    case 15: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, F1, F2, 3, s1, 3, s2);
    default: __builtin_unreachable();
  }
}

// Eight FP8 codes (bytes of w0 then w1) times `scale` (a power of two; 1 for
// the per-tensor path), converted to bf16.  Measured on MI355X: exact for
// every code of both formats at every power of two from 2^-90 to 2^90 (the
// product has at most 4 significant bits and stays inside bf16's normal range
// there); Inf and NaN codes stay Inf and NaN.
template <int F>
__device__ __forceinline__ v8bf widen8_scaled_bf16(uint32_t w0, uint32_t w1, float scale) {
  v2bf a, b, c, d;
  if constexpr (F == kE4M3) {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, scale, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, scale, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, scale, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, scale, true);
  }
  return (v8bf){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A ROWS x 128-byte slab (rows row0.. of a row-major byte matrix with row
// stride ld, column offset k0) staged into an LDS tile through registers, with
// zero fill for k >= K (the ragged last K step) and for rows past the edge.
template <int ROWS, int NT>
__device__ __forceinline__ void tile_load_zero_fill(const uint8_t* __restrict__ base, int64_t ld,
                                                    int64_t row0, int64_t rows_valid, int k0, int K,
                                                    uint8_t* lds_tile, int t) {
  constexpr int PER = ROWS * 8 / NT;
  const int g = t & 7;
  const int k = k0 + g * 16;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int row = (t >> 3) + j * (NT / 8);
    const int64_t r = row0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows_valid && k < K) v = *reinterpret_cast<const uint4*>(base + r * ld + k);
    *reinterpret_cast<uint4*>(lds_tile + lds_granule(row, g)) = v;
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Map a linear workgroup id to an output tile.  Workgroups are dealt to the
// 8 XCDs round-robin (id % 8); remap so each XCD receives a contiguous range
// of tile ids, then walk that range in column bands of `group_m` tile-rows so
// neighbouring workgroups on one XCD share A rows and B columns in its L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int group_m, int* tm,
                                            int* tn) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) {
    const int per_xcd = total >> 3;
    pid = (pid & 7) * per_xcd + (pid >> 3);
  }
  const int in_group = group_m * tiles_n;
  const int gid = pid / in_group;
  const int first_m = gid * group_m;
  const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int local = pid - gid * in_group;
  *tm = first_m + local % gsize;
  *tn = local / gsize;
}

}  // namespace fp8mi
