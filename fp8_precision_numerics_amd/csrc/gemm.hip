// Per-tensor-scaled FP8 GEMM: C = (A · Bᵀ) × sinv_a × sinv_b, FP32 accumulation.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the GEMM runs in FP8, the
// result is accumulated in FP32 and restored with ×(1/scale); accumulation is
// always high precision.  §4.2.6: HYBRID pairs E4M3 forward operands with E5M2
// gradients, so each operand carries its own format.
//
// Design (gfx950): a workgroup computes a BM x BN output tile with WM x WN
// wavefronts; each K step moves a BM x 128 slab of A and a BN x 128 slab of B
// from HBM/L2 into one of two LDS buffers (16-B loads staged through VGPRs,
// issued one step ahead), while the wavefronts run 16x16x128 FP8 MFMAs out of
// the other buffer into fp32 accumulators held in registers.  One barrier per
// K step.  The epilogue multiplies by sinv_a·sinv_b and stores bf16 or fp32
// directly from the accumulators.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
__global__ __launch_bounds__(64 * WM* WN) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int M, int N, int K,
    const float* __restrict__ sinv_a, const float* __restrict__ sinv_b, void* __restrict__ C,
    int tiles_m, int tiles_n, int group_m) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;  // 16-B granules per thread per K step
  constexpr int ROWS_PER_PASS = NT / 8;
  static_assert(LA >= 1 && LB >= 1 && FM >= 1 && FN >= 1, "tile shape");
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, &tm, &tn);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w / WN, wn = w % WN;
  const int64_t m_base = (int64_t)tm * BM, n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK;
  const int g = t & 7, row_in_pass = t >> 3;

  uint4 ra[LA], rb[LB];
  auto gload = [&](int kt) {
    const int k = kt * kBK + g * 16;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int64_t r = m_base + row_in_pass + j * ROWS_PER_PASS;
      ra[j] = (r < M && k < K) ? *reinterpret_cast<const uint4*>(A + r * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int64_t r = n_base + row_in_pass + j * ROWS_PER_PASS;
      rb[j] = (r < N && k < K) ? *reinterpret_cast<const uint4*>(B + r * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* sa = smem + stage * STAGE;
    uint8_t* sb = sa + BM * kBK;
#pragma unroll
    for (int j = 0; j < LA; ++j)
      *reinterpret_cast<uint4*>(sa + lds_granule(row_in_pass + j * ROWS_PER_PASS, g)) = ra[j];
#pragma unroll
    for (int j = 0; j < LB; ++j)
      *reinterpret_cast<uint4*>(sb + lds_granule(row_in_pass + j * ROWS_PER_PASS, g)) = rb[j];
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* sa = smem + cur * STAGE;
    const uint8_t* sb = sa + BM * kBK;
    v8i bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = lds_frag(sb, wn * WTN + j * 16 + (lane & 15), lane);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v8i af = lds_frag(sa, wm * WTM + i * 16 + (lane & 15), lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<FB, FA>(bf[j], af, acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  const float sc = sinv_a[0] * sinv_b[0];
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m_base + wm * WTM + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n_base + wn * WTN + j * 16 + 4 * (lane >> 4);
      store4<OUT>(C, N, m, n, M, acc[i][j] * sc, vec_ok);
    }
  }
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
hipError_t run(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K,
               const float* sa, const float* sb, void* C, hipStream_t st) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int group_m = 8;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, FA, FB, OUT>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * WM * WN), 0, st, A, B, (int)M, (int)N, (int)K, sa, sb, C, tiles_m,
                     tiles_n, group_m);
  return hipGetLastError();
}

template <int FA, int FB, int OUT>
hipError_t dispatch_shape(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K,
                          const float* sa, const float* sb, void* C, hipStream_t st) {
  if (M >= 1024 && N >= 1024)
    return run<256, 256, 2, 2, FA, FB, OUT>(A, B, M, N, K, sa, sb, C, st);
  return run<128, 128, 2, 2, FA, FB, OUT>(A, B, M, N, K, sa, sb, C, st);
}

template <int OUT>
hipError_t dispatch_fmt(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                        int64_t K, const float* sa, const float* sb, void* C, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) return dispatch_shape<kE4M3, kE4M3, OUT>(A, B, M, N, K, sa, sb, C, st);
  if (fa == kE5M2 && fb == kE4M3) return dispatch_shape<kE5M2, kE4M3, OUT>(A, B, M, N, K, sa, sb, C, st);
  if (fa == kE4M3 && fb == kE5M2) return dispatch_shape<kE4M3, kE5M2, OUT>(A, B, M, N, K, sa, sb, C, st);
  return dispatch_shape<kE5M2, kE5M2, OUT>(A, B, M, N, K, sa, sb, C, st);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                       int64_t K, const float* sinv_a, const float* sinv_b, void* C, int ctype,
                       hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (ctype == kBF16) return dispatch_fmt<kBF16>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
  return dispatch_fmt<kF32>(A, fa, B, fb, M, N, K, sinv_a, sinv_b, C, stream);
}

}  // namespace fp8mi
