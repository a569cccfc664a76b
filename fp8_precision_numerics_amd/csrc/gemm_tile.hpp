// Shared building blocks of the FP8 GEMM kernels (dense and grouped).
//
// Matrix-core contraction: V_MFMA_F32_16X16X128_F8F6F4 (gfx950).  One
// instruction multiplies a 16x128 FP8 block by a 128x16 FP8 block and adds an
// fp32 16x16 block; the two operand formats (E4M3 / E5M2) are chosen per
// operand.  Lane l of the wave supplies row (l % 16) and the 32-byte K slice
// (l / 16) of each operand; the fp32 result lands in lane l as column (l % 16),
// rows 4*(l/16) .. 4*(l/16)+3.  The kernels feed the B tile (rows = n) as the
// instruction's first operand and the A tile (rows = m) as its second, so the
// result block is C^T: lane l holds row m = l % 16 and FOUR CONSECUTIVE
// columns n = 4*(l/16) .. +3 — a contiguous 8-B (bf16) / 16-B (fp32) store.
//
// Operand tiles live in LDS as rows of 128 bytes (one K step).  The 16-byte
// granule g of row r is stored at granule position g ^ (r & 7): the 16-B reads
// of a fragment (rows r..r+15, same granule) and the 16-B writes of a loaded
// row both touch eight different granule positions per eight lanes.
#pragma once

#include "device_common.hpp"

namespace fp8mi {

constexpr int kBK = 128;  // K bytes per main-loop step (one MFMA deep)

__device__ __forceinline__ int lds_granule(int row, int g) { return row * kBK + (((g ^ row) & 7) << 4); }

template <int FA, int FB>
__device__ __forceinline__ v4f mfma16(const v8i& first, const v8i& second, const v4f& c) {
  // Scale operands are zero, which selects the plain (unscaled) instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, c, FA, FB, 0, 0, 0, 0);
}

// Read the 32-byte K slice of one fragment row for this lane from an LDS tile.
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int lane) {
  const int kg = (lane >> 4) * 2;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + lds_granule(row, kg));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + lds_granule(row, kg + 1));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

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

template <int OUT>
__device__ __forceinline__ void store4(void* C, int64_t N, int64_t m, int64_t n, int64_t M,
                                       const v4f& v, bool vec_ok) {
  if (m >= M) return;
  if (OUT == kF32) {
    float* c = reinterpret_cast<float*>(C) + m * N + n;
    if (vec_ok && n + 3 < N) {
      *reinterpret_cast<v4f*>(c) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) c[j] = v[j];
    }
  } else {
    __bf16* c = reinterpret_cast<__bf16*>(C) + m * N + n;
    const v2bf lo = __builtin_convertvector((v2f){v[0], v[1]}, v2bf);
    const v2bf hi = __builtin_convertvector((v2f){v[2], v[3]}, v2bf);
    if (vec_ok && n + 3 < N) {
      uint2 w;
      w.x = __builtin_bit_cast(uint32_t, lo);
      w.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<uint2*>(c) = w;
    } else {
      if (n + 0 < N) c[0] = lo[0];
      if (n + 1 < N) c[1] = lo[1];
      if (n + 2 < N) c[2] = hi[0];
      if (n + 3 < N) c[3] = hi[1];
    }
  }
}

}  // namespace fp8mi
