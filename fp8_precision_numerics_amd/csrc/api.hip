// extern "C" entry points of libfp8mi: argument validation, device check,
// and dispatch to the kernel launchers.  The contract of each function
// (arguments, layout, ownership, errors) is stated in include/fp8mi.h.
#include <stdint.h>

#include <atomic>

#include "fp8mi.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;             // kernels index rows/cols with 32-bit ints
constexpr int64_t kMaxGemmK = int64_t(1) << 23;     // 256 rows x K bytes of a tile slab in a 32-bit buffer offset
constexpr int64_t kMaxGroupedK = int64_t(1) << 22;  // 512 rows x K bytes (the grouped kernels' widest slab)
constexpr int64_t kMaxBufferBytes = 0x7FFFFFFF;     // any offset a buffer load carries in one 32-bit register
constexpr int64_t kMaxElems = (int64_t)1 << 40;     // sanity bound on any one tensor
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];         // 0 unknown, 1 gfx950, -1 not usable

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fmt_ok(int f) { return f == FP8MI_E4M3 || f == FP8MI_E5M2; }
bool dtype_ok(int d) { return d == FP8MI_F32 || d == FP8MI_BF16; }
bool accum_ok(int a) { return a == FP8MI_ACCUM_EXACT || a == FP8MI_ACCUM_MFMA_FP8; }

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8MI_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    state = -1;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      const char* a = prop.gcnArchName;
      if (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' && a[5] == '0')
        state = 1;
    }
    // Set-up on the first call that sees this device: the device address of
    // the library-owned scratch (fp8_quantize_update_noalloc), looked up while
    // the device is current.  A failure here is reported by that entry point,
    // which retries the lookup, and does not affect the others.
    if (state == 1) {
      void* scratch = nullptr;
      (void)fp8mi::noalloc_scratch(&scratch);
    }
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? FP8MI_OK : FP8MI_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? FP8MI_OK : FP8MI_ERR_LAUNCH; }

bool dims_ok(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || rows > kMaxElems || cols > kMaxElems) return false;
  if (rows != 0 && cols > kMaxElems / rows) return false;
  return true;
}

}  // namespace

extern "C" {

const char* fp8mi_status_string(int status) {
  switch (status) {
    case FP8MI_OK: return "ok";
    case FP8MI_ERR_NULL: return "a required pointer is NULL";
    case FP8MI_ERR_SHAPE: return "invalid or inconsistent size";
    case FP8MI_ERR_ALIGN: return "pointer or size breaks the alignment rule";
    case FP8MI_ERR_FORMAT: return "unknown FP8 format";
    case FP8MI_ERR_DTYPE: return "unknown data type";
    case FP8MI_ERR_LAUNCH: return "kernel launch failed";
    case FP8MI_ERR_DEVICE: return "no usable gfx950 device is current";
    case FP8MI_ERR_ACCUM: return "unknown accumulation mode";
    default: return "unknown status";
  }
}

int fp8mi_version(void) { return 800; }

int fp8_quantize(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, const float* scale,
                 uint8_t* q, uint8_t* q_t, float* amax, unsigned long long* sat, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!dtype_ok(xtype)) return FP8MI_ERR_DTYPE;
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!dims_ok(rows, cols)) return FP8MI_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (!q && !q_t && !amax) return FP8MI_ERR_NULL;
  if ((q || q_t || sat) && !scale) return FP8MI_ERR_NULL;
  if (n > 0 && !x) return FP8MI_ERR_NULL;
  if ((x && !aligned16(x)) || (q && !aligned16(q)) || (q_t && !aligned16(q_t))) return FP8MI_ERR_ALIGN;
  if (q_t && ((rows & 15) || (cols & 15))) return FP8MI_ERR_ALIGN;
  if (workspace && (!aligned16(workspace) || workspace_bytes < 16)) return FP8MI_ERR_ALIGN;
  if (q_t && (rows + 127) / 128 > 65535) return FP8MI_ERR_SHAPE;
  if ((cols + 127) / 128 > kMaxDim) return FP8MI_ERR_SHAPE;
  if (!amax && !sat && n == 0) return FP8MI_OK;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_quantize(x, xtype, rows, cols, fmt, scale, q, q_t, amax, sat, workspace,
                                         workspace_bytes, (hipStream_t)stream));
}

int fp8_quantize_update(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* q_t,
                        float* amax, unsigned long long* sat, void* workspace, size_t workspace_bytes, float* history,
                        int32_t history_len, int32_t* head, float* scale, float* scale_inv, int32_t* status,
                        float* scale_inv_used, void* stream) {
  if (!dtype_ok(xtype)) return FP8MI_ERR_DTYPE;
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!dims_ok(rows, cols)) return FP8MI_ERR_SHAPE;
  if (history_len < 1 || history_len > 4096) return FP8MI_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (!amax || !history || !head || !scale || !scale_inv) return FP8MI_ERR_NULL;
  if (n > 0 && !x) return FP8MI_ERR_NULL;
  if ((x && !aligned16(x)) || (q && !aligned16(q)) || (q_t && !aligned16(q_t))) return FP8MI_ERR_ALIGN;
  if (q_t && ((rows & 15) || (cols & 15))) return FP8MI_ERR_ALIGN;
  if (workspace && (!aligned16(workspace) || workspace_bytes < 16)) return FP8MI_ERR_ALIGN;
  if (q_t && (rows + 127) / 128 > 65535) return FP8MI_ERR_SHAPE;
  if ((cols + 127) / 128 > kMaxDim) return FP8MI_ERR_SHAPE;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  const fp8mi::HistoryArgs hs{history, history_len, head, scale, scale_inv, status, fmt, scale_inv_used};
  return launched(fp8mi::launch_quantize(x, xtype, rows, cols, fmt, scale, q, q_t, amax, sat, workspace,
                                         workspace_bytes, (hipStream_t)stream, hs));
}

int fp8_quantize_update_noalloc(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                uint8_t* q_t, float* amax, unsigned long long* sat, float* history,
                                int32_t history_len, int32_t* head, float* scale, float* scale_inv, int32_t* status,
                                float* scale_inv_used, void* stream) {
  if (!dtype_ok(xtype)) return FP8MI_ERR_DTYPE;
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!dims_ok(rows, cols)) return FP8MI_ERR_SHAPE;
  if (history_len < 1 || history_len > 4096) return FP8MI_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (!amax || !history || !head || !scale || !scale_inv) return FP8MI_ERR_NULL;
  if (n > 0 && !x) return FP8MI_ERR_NULL;
  if ((x && !aligned16(x)) || (q && !aligned16(q)) || (q_t && !aligned16(q_t))) return FP8MI_ERR_ALIGN;
  if (q_t && ((rows & 15) || (cols & 15))) return FP8MI_ERR_ALIGN;
  if (q_t && (rows + 127) / 128 > 65535) return FP8MI_ERR_SHAPE;
  if ((cols + 127) / 128 > kMaxDim) return FP8MI_ERR_SHAPE;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  const fp8mi::HistoryArgs hs{history, history_len, head, scale, scale_inv, status, fmt, scale_inv_used};
  const hipError_t e = fp8mi::launch_quantize_noalloc(x, xtype, rows, cols, fmt, q, q_t, amax, sat,
                                                      (hipStream_t)stream, hs);
  if (e == hipErrorInvalidSymbol || e == hipErrorInvalidDevice) return FP8MI_ERR_DEVICE;
  return launched(e);
}

int fp8_amax_update(float* history, int32_t history_len, int32_t* head, const float* amax, int fmt,
                    float* scale, float* scale_inv, int32_t* status, void* stream) {
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!history || !head || !amax || !scale || !scale_inv) return FP8MI_ERR_NULL;
  if (history_len < 1 || history_len > 4096) return FP8MI_ERR_SHAPE;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_amax_update(history, history_len, head, amax, fmt, scale, scale_inv,
                                            status, (hipStream_t)stream));
}

int fp8_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int b_trans, int64_t M, int64_t N, int64_t K,
             const float* sinv_a, const float* sinv_b, void* C, int ctype, int accum, void* stream) {
  if (!fmt_ok(fa) || !fmt_ok(fb)) return FP8MI_ERR_FORMAT;
  if (!dtype_ok(ctype)) return FP8MI_ERR_DTYPE;
  if (!accum_ok(accum)) return FP8MI_ERR_ACCUM;
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK) return FP8MI_ERR_SHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return FP8MI_ERR_SHAPE;
  if ((K & 15) != 0) return FP8MI_ERR_ALIGN;
  // [K x N] B: whole 16-byte granules per K row, and every offset into it within 31 bits.
  if (b_trans && (N & 15) != 0) return FP8MI_ERR_ALIGN;
  if (b_trans && K * N > kMaxBufferBytes) return FP8MI_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return FP8MI_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8MI_OK;
  if (!A || !B || !sinv_a || !sinv_b || !C) return FP8MI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_gemm(A, fa, B, fb, b_trans ? 1 : 0, M, N, K, sinv_a, sinv_b, C, ctype, accum,
                                     (hipStream_t)stream));
}

int fp8_gemm_requant(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N, int64_t K,
                     const float* sinv_a, const float* sinv_b, int out_fmt, const float* out_scale,
                     uint8_t* Cq, float* amax, unsigned long long* sat, int accum, void* stream) {
  if (!fmt_ok(fa) || !fmt_ok(fb) || !fmt_ok(out_fmt)) return FP8MI_ERR_FORMAT;
  if (!accum_ok(accum)) return FP8MI_ERR_ACCUM;
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK) return FP8MI_ERR_SHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return FP8MI_ERR_SHAPE;
  if ((K & 15) != 0) return FP8MI_ERR_ALIGN;
  if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return FP8MI_ERR_SHAPE;
  if (M > 0 && N > 0) {
    if (!A || !B || !sinv_a || !sinv_b || !out_scale || !Cq) return FP8MI_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(Cq)) return FP8MI_ERR_ALIGN;
  } else if (!amax && !sat) {
    return FP8MI_OK;
  }
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_gemm_requant(A, fa, B, fb, M, N, K, sinv_a, sinv_b, out_fmt, out_scale, Cq,
                                             amax, sat, accum, (hipStream_t)stream));
}

int fp8_shared_scale(const float* amaxes, int32_t R, int fmt, float* scale, float* scale_inv, void* stream) {
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (R < 1 || R > 65536) return FP8MI_ERR_SHAPE;
  if (!amaxes || !scale || !scale_inv) return FP8MI_ERR_NULL;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_shared_scale(amaxes, R, fmt, scale, scale_inv, (hipStream_t)stream));
}

int fp8_dequant_sum(const uint8_t* q, int32_t R, int64_t n, int64_t stride, int fmt, const float* scale_inv,
                    void* out, int otype, void* stream) {
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!dtype_ok(otype)) return FP8MI_ERR_DTYPE;
  if (R < 1 || R > 65536 || n < 0 || n > kMaxElems || stride < n) return FP8MI_ERR_SHAPE;
  if (stride > kMaxElems || (int64_t)(R - 1) > kMaxElems / (stride > 0 ? stride : 1)) return FP8MI_ERR_SHAPE;
  if ((stride & 15) != 0) return FP8MI_ERR_ALIGN;
  if (n == 0) return FP8MI_OK;
  if (!q || !scale_inv || !out) return FP8MI_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_dequant_sum(q, R, n, stride, fmt, scale_inv, out, otype, (hipStream_t)stream));
}

int fp8_quantize_mx(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* scales,
                    void* stream) {
  if (!dtype_ok(xtype)) return FP8MI_ERR_DTYPE;
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (!dims_ok(rows, cols)) return FP8MI_ERR_SHAPE;
  if ((cols & 31) != 0) return FP8MI_ERR_ALIGN;
  if (rows * cols == 0) return FP8MI_OK;
  if (!x || !q || !scales) return FP8MI_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_quantize_mx(x, xtype, rows, cols, fmt, q, scales, (hipStream_t)stream));
}

int fp8_gemm_mx(const uint8_t* A, int fa, const uint8_t* sa, const uint8_t* B, int fb, const uint8_t* sb, int64_t M,
                int64_t N, int64_t K, void* C, int ctype, int accum, void* stream) {
  if (!fmt_ok(fa) || !fmt_ok(fb)) return FP8MI_ERR_FORMAT;
  if (!dtype_ok(ctype)) return FP8MI_ERR_DTYPE;
  if (!accum_ok(accum)) return FP8MI_ERR_ACCUM;
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK) return FP8MI_ERR_SHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return FP8MI_ERR_SHAPE;
  if ((K & 127) != 0) return FP8MI_ERR_ALIGN;
  if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return FP8MI_ERR_SHAPE;
  // The scale loads address a whole scale matrix with one 32-bit offset.
  if ((K / 32) * FP8MI_MX_SCALE_LD(M) > kMaxBufferBytes || (K / 32) * FP8MI_MX_SCALE_LD(N) > kMaxBufferBytes)
    return FP8MI_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8MI_OK;
  if (!A || !sa || !B || !sb || !C) return FP8MI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || ((uintptr_t)sa & 3) || ((uintptr_t)sb & 3))
    return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_gemm_mx(A, fa, sa, B, fb, sb, M, N, K, C, ctype, accum, (hipStream_t)stream));
}

int fp8_quantize_blockwise(const void* x, int xtype, int64_t rows, int64_t cols, int32_t block_rows,
                           int fmt, uint8_t* q, float* scale_inv, void* stream) {
  if (!dtype_ok(xtype)) return FP8MI_ERR_DTYPE;
  if (!fmt_ok(fmt)) return FP8MI_ERR_FORMAT;
  if (block_rows != 1 && block_rows != 128) return FP8MI_ERR_SHAPE;
  if (!dims_ok(rows, cols)) return FP8MI_ERR_SHAPE;
  if ((cols & 15) != 0) return FP8MI_ERR_ALIGN;
  if (block_rows == 128 && ((rows + 127) / 128 > 65535 || (cols + 127) / 128 > kMaxDim))
    return FP8MI_ERR_SHAPE;
  if (rows * cols == 0) return FP8MI_OK;
  if (!x || !q || !scale_inv) return FP8MI_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_quantize_blockwise(x, xtype, rows, cols, block_rows, fmt, q,
                                                   scale_inv, (hipStream_t)stream));
}

int fp8_grouped_gemm(const uint8_t* A, const float* sinv_a, const uint8_t* B, const float* sinv_b,
                     const int32_t* m_offsets, int32_t G, int64_t total_m, int64_t N, int64_t K,
                     void* C, int ctype, int accum, void* stream) {
  if (!dtype_ok(ctype)) return FP8MI_ERR_DTYPE;
  if (!accum_ok(accum)) return FP8MI_ERR_ACCUM;
  if (G < 1 || G > 1024) return FP8MI_ERR_SHAPE;
  if (total_m < 0 || N < 0 || K <= 0 || total_m > kMaxDim || N > kMaxDim || K > kMaxGroupedK)
    return FP8MI_ERR_SHAPE;
  if (!dims_ok(total_m, K) || !dims_ok(N, K) || !dims_ok((int64_t)G * N, K) || !dims_ok(total_m, N))
    return FP8MI_ERR_SHAPE;
  if ((K & 15) != 0) return FP8MI_ERR_ALIGN;
  if (((total_m + 127) / 128 + G) * ((N + 127) / 128) > kMaxDim) return FP8MI_ERR_SHAPE;
  if (total_m == 0 || N == 0) return FP8MI_OK;
  if (!A || !sinv_a || !B || !sinv_b || !m_offsets || !C) return FP8MI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return FP8MI_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FP8MI_OK) return dev;
  return launched(fp8mi::launch_grouped_gemm(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C,
                                             ctype, accum, (hipStream_t)stream));
}

}  // extern "C"
