// Fine-grained-scaled grouped FP8 GEMM for MoE experts, with two-level
// accumulation.
//
// "#fp8" tag page, DeepGEMM entry: a grouped GEMM for Mixture-of-Experts runs
// one GEMM per expert in a single launch, and FP8 partial sums are "promoted"
// into a higher-precision accumulator to offset FP8's low precision.  "FP8 and
// low-precision formats", "Deep dive": scale factors per tensor or per block.
//
// Each 128-deep K step yields an fp32 partial P per output block (from either
// accumulation mode, see gemm_tile.hpp); it is promoted into the running fp32
// accumulator as
//     acc += P * (sinv_a[m][kb] * sinv_b[g][n/128][kb]),
// so every 1x128 activation tile and 128x128 weight block keeps its own scale.
// The tile scheduler finds each workgroup's expert from the device-side row
// offsets, so the host never needs the token counts.
//
// Layout and data movement follow the dense kernel (gemm_kernel.hpp): 128x128
// output tiles, 4 wavefronts of 64x64, two LDS stages filled by buffer loads
// issued one step ahead (rows past the expert's last row fall outside the
// buffer resource and are never stored), the measured LDS swizzle, and the
// output tile written through LDS as whole rows.  Two workgroups share a CU.
#include "gemm_kernel.hpp"
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
  constexpr int BLK = MODE == kAccumMfma8 ? 16 : 32;
  constexpr int FM = WTM / BLK, FN = WTN / BLK;
  constexpr int LQA = BM / 8 / NW, LQB = BN / 8 / NW;
  static_assert(FM >= 1 && FN >= 1 && WTM % BLK == 0 && WTN % BLK == 0 && WTN <= 128, "wave tile shape");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && NW % 2 == 0, "load split");
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  __shared__ int s_info[3];

  const int tn = blockIdx.x % tiles_n, mt = blockIdx.x / tiles_n;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
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
  const int nk = (K + kBK - 1) / kBK, nfull = K / kBK;
  const int nbn = (N + 127) / 128;
  const uint8_t* Bg = B + (int64_t)gidx * N * K;
  const float* sbg = sinv_b + (int64_t)gidx * nbn * nk;

  // Operand slabs: buffer resources over this expert's rows of A and of B_g.
  const __amdgpu_buffer_rsrc_t ra = operand_rsrc(A + row0 * K, row_end - row0, K);
  const __amdgpu_buffer_rsrc_t rb = operand_rsrc(Bg + n_base * K, N - n_base, K);
  const int lrow = w * 8 + (lane >> 3);
  const int voff = lrow * K + (((lane & 7) ^ lds_swz(lrow)) & 7) * 16;
  auto fill = [&](uint8_t* st, int kt) {
    if (kt < nfull) {
      const int k0 = kt * kBK;
      const uint32_t la = lds_addr(st) + w * 1024, lb = lds_addr(st + BM * kBK) + w * 1024;
#pragma unroll
      for (int q = 0; q < LQA; ++q) dma_lds16(ra, la + q * NW * 1024, voff, q * NW * 8 * K + k0);
#pragma unroll
      for (int q = 0; q < LQB; ++q) dma_lds16(rb, lb + q * NW * 1024, voff, q * NW * 8 * K + k0);
    } else {  // ragged last K step: zero-filled through registers
      tile_load_zero_fill<BM, NT>(A, K, row0, row_end, kt * kBK, K, st, t);
      tile_load_zero_fill<BN, NT>(Bg, K, n_base, N, kt * kBK, K, st + BM * kBK, t);
    }
  };

  const int rr = lane & (BLK - 1), hh = lane / BLK;
  const int swz = lds_swz(rr);
  auto granule = [&](const uint8_t* tile, int row0_, int g) {
    return *reinterpret_cast<const uint4*>(tile + (row0_ + rr) * kBK + (((g ^ swz) & 7) << 4));
  };

  // Scale lookups: the lane's row in each A block (clamped inside the expert),
  // and the 128-column weight block of each B block.
  int64_t arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t r = row0 + wm * WTM + i * BLK + rr;
    arow[i] = r < row_end ? r : row0;
  }
  int bblk[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int nb = (int)((n_base + wn * WTN + j * BLK) / 128);
    bblk[j] = nb < nbn ? nb : nbn - 1;
  }

  using Acc = typename std::conditional<MODE == kAccumMfma8, v4f, v16f>::type;
  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

  uint8_t* const s0 = smem;
  uint8_t* const s1 = smem + STAGE;
  fill(s0, 0);
  wait_loads_and_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* cur = (kt & 1) ? s1 : s0;
    uint8_t* nxt = (kt & 1) ? s0 : s1;
    // This step's scales first (their loads then precede the slab loads).
    float sa_v[FM], sb_v[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa_v[i] = sinv_a[arow[i] * nk + kt];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb_v[j] = sbg[bblk[j] * nk + kt];
    if (kt + 1 < nk) fill(nxt, kt + 1);
    __builtin_amdgcn_sched_barrier(0);
    Acc part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) part[i][j] = Acc{};
    if constexpr (MODE == kAccumMfma8) {
      v8i af[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 lo = granule(cur, wm * WTM + i * 16, 2 * hh), hi = granule(cur, wm * WTM + i * 16, 2 * hh + 1);
        af[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint8_t* tb = cur + BM * kBK;
        const uint4 lo = granule(tb, wn * WTN + j * 16, 2 * hh), hi = granule(tb, wn * WTN + j * 16, 2 * hh + 1);
        const v8i bf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int i = 0; i < FM; ++i) part[i][j] = mfma_fp8<kE4M3, kE4M3>(bf, af[i], part[i][j]);
      }
    } else {
      uint4 ar[FM][4], br[FN][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < FM; ++i) ar[i][c] = granule(cur, wm * WTM + i * 32, 4 * hh + c);
#pragma unroll
        for (int j = 0; j < FN; ++j) br[j][c] = granule(cur + BM * kBK, wn * WTN + j * 32, 4 * hh + c);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        v8h bh[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint4 g = br[j][s >> 1];
          bh[j] = (s & 1) ? widen8<kE4M3>(g.z, g.w) : widen8<kE4M3>(g.x, g.y);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const uint4 g = ar[i][s >> 1];
          const v8h ah = (s & 1) ? widen8<kE4M3>(g.z, g.w) : widen8<kE4M3>(g.x, g.y);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bh[j], ah, part[i][j], 0, 0, 0);
        }
      }
    }
    // Promotion of this 128-deep partial with its block scales.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j] * (sa_v[i] * sb_v[j]);
    __builtin_amdgcn_sched_barrier(0);
    wait_loads_and_barrier();
  }

  // Output tile through LDS, whole rows; rows past the expert are not stored.
  using TW = TileWriter<OUT, BM, BN, NT>;
  constexpr int PASS = (2 * STAGE / TW::ROWB) < BM ? (2 * STAGE / TW::ROWB) : BM;
  static_assert(BM % PASS == 0, "output passes must tile the rows");
  TW tw{smem, PASS};
#pragma unroll 1
  for (int r0 = 0; r0 < BM; r0 += PASS) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * BLK + rr;
      if (r < r0 || r >= r0 + PASS) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (MODE == kAccumMfma8) {
          tw.put(r - r0, wn * WTN + j * 16 + 4 * (lane >> 4), acc[i][j]);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            tw.put(r - r0, wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5), v);
          }
        }
      }
    }
    __syncthreads();
    tw.flush(C, row_end, N, row0 + r0, n_base, t);
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
