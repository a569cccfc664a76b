// Fine-grained-scaled grouped FP8 GEMM for MoE experts, with two-level
// accumulation.
//
// "#fp8" tag page, DeepGEMM entry: a grouped GEMM for Mixture-of-Experts runs
// one GEMM per expert in a single launch, and FP8 partial sums are "promoted"
// into a higher-precision accumulator to offset FP8's low precision.  "FP8 and
// low-precision formats", "Deep dive": scale factors per tensor or per block.
//
// Each 128-deep K step yields an fp32 MFMA partial P for a 16x16 output block;
// it is promoted into the running fp32 accumulator as
//     acc += P * (sinv_a[m][kb] * sinv_b[g][n/128][kb]),
// so every 1x128 activation tile and 128x128 weight block keeps its own scale.
// The tile scheduler finds each workgroup's expert from the device-side row
// offsets, so the host never needs the token counts.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

template <int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(64 * WM* WN) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sinv_a, const uint8_t* __restrict__ B,
    const float* __restrict__ sinv_b, const int32_t* __restrict__ m_offsets, int G, int total_m,
    int N, int K, void* __restrict__ C, int tiles_n) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;
  constexpr int ROWS_PER_PASS = NT / 8;
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
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
  const uint8_t* Bg = B + (int64_t)gidx * N * K;
  const float* sbg = sinv_b + (int64_t)gidx * nbn * nk;
  const int g = t & 7, row_in_pass = t >> 3;

  uint4 ra[LA], rb[LB];
  auto gload = [&](int kt) {
    const int k = kt * kBK + g * 16;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int64_t r = row0 + row_in_pass + j * ROWS_PER_PASS;
      ra[j] = (r < row_end && k < K) ? *reinterpret_cast<const uint4*>(A + r * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int64_t r = n_base + row_in_pass + j * ROWS_PER_PASS;
      rb[j] = (r < N && k < K) ? *reinterpret_cast<const uint4*>(Bg + r * K + k) : make_uint4(0, 0, 0, 0);
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

  // Rows of this lane in each 16-row block (clamped for the scale lookup).
  int64_t arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t r = row0 + wm * WTM + i * 16 + (lane & 15);
    arow[i] = r < row_end ? r : row0;
  }

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    float sa_v[FM], sb_v[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa_v[i] = sinv_a[arow[i] * nk + kt];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      int64_t nb = (n_base + wn * WTN + j * 16) / 128;
      nb = nb < nbn ? nb : nbn - 1;
      sb_v[j] = sbg[nb * nk + kt];
    }
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
      for (int j = 0; j < FN; ++j) {
        const v4f p = mfma16<kE4M3, kE4M3>(bf[j], af, (v4f){0.f, 0.f, 0.f, 0.f});
        const float sc = sa_v[i] * sb_v[j];
        acc[i][j] += p * sc;
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
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

template <int BM, int BN, int WM, int WN, int OUT>
hipError_t run(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
               const int32_t* offs, int G, int64_t total_m, int64_t N, int64_t K, void* C,
               hipStream_t st) {
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int64_t tiles_m = (total_m + BM - 1) / BM + G;  // upper bound over any split into G experts
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, OUT>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * WM * WN), 0, st, A, sa, B, sb, offs, G, (int)total_m, (int)N, (int)K, C,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* A, const float* sinv_a, const uint8_t* B,
                               const float* sinv_b, const int32_t* m_offsets, int G,
                               int64_t total_m, int64_t N, int64_t K, void* C, int ctype,
                               hipStream_t stream) {
  if (total_m == 0 || N == 0) return hipSuccess;
  if (ctype == kBF16)
    return run<128, 128, 2, 2, kBF16>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
  return run<128, 128, 2, 2, kF32>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
}

}  // namespace fp8mi
