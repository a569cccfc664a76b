// Fine-grained-scaled grouped FP8 GEMM for MoE experts, with two-level
// accumulation.
//
// "#fp8" tag page, DeepGEMM entry: a grouped GEMM for Mixture-of-Experts runs
// one GEMM per expert in a single launch, and FP8 partial sums are "promoted"
// into a higher-precision accumulator to offset FP8's low precision.  "FP8 and
// low-precision formats", "Deep dive": scale factors per tensor or per block.
//
// Each 128-deep K step yields an fp32 partial P for a 16x16 output block (from
// either accumulation mode of gemm_tile.hpp); it is promoted into the running
// fp32 accumulator as
//     acc += P * (sinv_a[m][kb] * sinv_b[g][n/128][kb]),
// so every 1x128 activation tile and 128x128 weight block keeps its own scale.
// The tile scheduler finds each workgroup's expert from the device-side row
// offsets, so the host never needs the token counts.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

template <int BM, int BN, int WM, int WN, int OUT, int MODE>
__global__ __launch_bounds__(64 * WM* WN) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sinv_a, const uint8_t* __restrict__ B,
    const float* __restrict__ sinv_b, const int32_t* __restrict__ m_offsets, int G, int total_m,
    int N, int K, void* __restrict__ C, int tiles_n) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  __shared__ int s_info[3];

  const int tn = blockIdx.x % tiles_n, mt = blockIdx.x / tiles_n;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) {
    // Expert intervals [lo, hi) made non-decreasing and clamped to [0, total_m].
    int acc_tiles = 0, prev = 0, found = -1, row0 = 0, row_end = 0;
    for (int g = 0; g < G; ++g) {
      int lo = m_offsets[g], hi = m_offsets[g + 1];
      lo = lo < prev ? prev : (lo > total_m ? total_m : lo);
      hi = hi < lo ? lo : (hi > total_m ? total_m : hi);
      prev = hi;
      const int tiles = (hi - lo + BM - 1) / BM;
      if (mt < acc_tiles + tiles) {
        found = g;
        row0 = lo + (mt - acc_tiles) * BM;
        row_end = hi;
        break;
      }
      acc_tiles += tiles;
    }
    s_info[0] = found;
    s_info[1] = row0;
    s_info[2] = row_end;
  }
  __syncthreads();
  const int gidx = s_info[0];
  if (gidx < 0) return;  // workgroup beyond the last expert's tiles (uniform exit)
  const int64_t row0 = s_info[1], row_end = s_info[2];

  const int wm = w / WN, wn = w % WN;
  const int64_t n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK;
  const int nbn = (N + 127) / 128;
  const bool ragged_k = (K % kBK) != 0;
  const uint8_t* Bg = B + (int64_t)gidx * N * K;
  const float* sbg = sinv_b + (int64_t)gidx * nbn * nk;

  auto stage_in = [&](int kt, int stage) {
    uint8_t* sa = smem + stage * STAGE;
    uint8_t* sb = sa + BM * kBK;
    if (ragged_k && kt == nk - 1) {
      tile_load_zero_fill<BM, NT>(A, K, row0, row_end, kt * kBK, K, sa, t);
      tile_load_zero_fill<BN, NT>(Bg, K, n_base, N, kt * kBK, K, sb, t);
    } else {
      tile_load_direct<BM, NW>(A, K, row0, row_end, kt * kBK, sa, w, lane);
      tile_load_direct<BN, NW>(Bg, K, n_base, N, kt * kBK, sb, w, lane);
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Rows of this lane in each 16-row block (clamped for the scale lookup).
  int64_t arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t r = row0 + wm * WTM + i * 16 + (lane & 15);
    arow[i] = r < row_end ? r : row0;
  }
  int64_t bblk[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t nb = (n_base + wn * WTN + j * 16) / 128;
    bblk[j] = nb < nbn ? nb : nbn - 1;
  }

  stage_in(0, 0);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    float sa_v[FM], sb_v[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa_v[i] = sinv_a[arow[i] * nk + kt];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb_v[j] = sbg[bblk[j] * nk + kt];
    if (kt + 1 < nk) stage_in(kt + 1, cur ^ 1);
    const uint8_t* sa = smem + cur * STAGE;
    v4f part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) part[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    wave_kstep<FM, FN, kE4M3, kE4M3, MODE>(sa, sa + BM * kBK, wm * WTM, wn * WTN, lane, part);
    // promotion of this 128-deep partial with its block scales
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j] * (sa_v[i] * sb_v[j]);
    wait_vmem();
    __syncthreads();
  }

  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = row0 + wm * WTM + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n_base + wn * WTN + j * 16 + 4 * (lane >> 4);
      store4<OUT>(C, N, m, n, row_end, acc[i][j], vec_ok);
    }
  }
}

template <int BM, int BN, int WM, int WN, int OUT, int MODE>
hipError_t run(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
               const int32_t* offs, int G, int64_t total_m, int64_t N, int64_t K, void* C,
               hipStream_t st) {
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int64_t tiles_m = (total_m + BM - 1) / BM + G;  // upper bound over any split into G experts
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, OUT, MODE>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * WM * WN), 0, st, A, sa, B, sb, offs, G, (int)total_m, (int)N, (int)K, C,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* A, const float* sinv_a, const uint8_t* B,
                               const float* sinv_b, const int32_t* m_offsets, int G,
                               int64_t total_m, int64_t N, int64_t K, void* C, int ctype,
                               int accum, hipStream_t stream) {
  if (total_m == 0 || N == 0) return hipSuccess;
  if (accum == kAccumMfma8) {
    if (ctype == kBF16)
      return run<128, 128, 2, 2, kBF16, kAccumMfma8>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
    return run<128, 128, 2, 2, kF32, kAccumMfma8>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
  }
  if (ctype == kBF16)
    return run<128, 128, 2, 2, kBF16, kAccumExact>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
  return run<128, 128, 2, 2, kF32, kAccumExact>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
}

}  // namespace fp8mi
