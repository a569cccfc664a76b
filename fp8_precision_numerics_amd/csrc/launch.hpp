// Internal launchers behind the C ABI (include/fp8mi.h).  Arguments are
// already validated by api.hip; each launcher only enqueues kernels on the
// given stream and returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

// The delayed-scaling history step a cast may run right after itself
// (fp8_quantize_update); `history` null = none.
struct HistoryArgs {
  float* history;
  int len;
  int32_t* head;
  float* scale;
  float* scale_inv;
  int32_t* status;
  int fmt;
  float* sinv_used;  // receives *scale_inv as it was before the step (may be null)
};

// Workgroups of a grid with `per_cu` per compute unit of the current device
// (the count is queried once per device; 256 compute units if the query fails).
int persistent_groups(int per_cu);

hipError_t launch_quantize(const void* x, int xtype, int64_t rows, int64_t cols, int fmt,
                           const float* scale, uint8_t* q, uint8_t* q_t, float* amax,
                           unsigned long long* sat, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, HistoryArgs hs = HistoryArgs{nullptr, 0, nullptr, nullptr, nullptr,
                                                                           nullptr, 0, nullptr});

// Bytes of the library-owned scratch behind fp8_quantize_update_noalloc
// (FP8MI_NOALLOC_SCRATCH_BYTES): 4096 partial slots of 16 bytes, more than any
// cast grid uses (a grid is capped at the slots it is given).
constexpr size_t kNoallocScratchBytes = 65536;

// The device address of that scratch on the current device, looked up once
// per device (hipGetSymbolAddress) and cached; the library's set-up calls it
// when it first sees a device.
hipError_t noalloc_scratch(void** out);

// launch_quantize with the library-owned scratch as the workspace.
hipError_t launch_quantize_noalloc(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                   uint8_t* q_t, float* amax, unsigned long long* sat, hipStream_t stream,
                                   HistoryArgs hs);

hipError_t launch_quantize_blockwise(const void* x, int xtype, int64_t rows, int64_t cols,
                                     int block_rows, int fmt, uint8_t* q, float* scale_inv,
                                     hipStream_t stream);

hipError_t launch_amax_update(float* history, int history_len, int32_t* head, const float* amax,
                              int fmt, float* scale, float* scale_inv, int32_t* status,
                              hipStream_t stream);

hipError_t launch_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int b_trans, int64_t M, int64_t N,
                       int64_t K, const float* sinv_a, const float* sinv_b, void* C, int ctype,
                       int accum, hipStream_t stream);

hipError_t launch_gemm_requant(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                               int64_t K, const float* sinv_a, const float* sinv_b, int out_fmt,
                               const float* out_scale, uint8_t* Cq, float* amax, unsigned long long* sat,
                               int accum, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t* A, const float* sinv_a, const uint8_t* B,
                               const float* sinv_b, const int32_t* m_offsets, int G,
                               int64_t total_m, int64_t N, int64_t K, void* C, int ctype,
                               int accum, hipStream_t stream);

hipError_t launch_shared_scale(const float* amaxes, int R, int fmt, float* scale, float* scale_inv,
                               hipStream_t stream);

hipError_t launch_dequant_sum(const uint8_t* q, int R, int64_t n, int64_t stride, int fmt, const float* scale_inv,
                              void* out, int otype, hipStream_t stream);

hipError_t launch_quantize_mx(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                              uint8_t* scales, hipStream_t stream);

hipError_t launch_gemm_mx(const uint8_t* A, int fa, const uint8_t* sa, const uint8_t* B, int fb, const uint8_t* sb,
                          int64_t M, int64_t N, int64_t K, void* C, int ctype, int accum, hipStream_t stream);

}  // namespace fp8mi
