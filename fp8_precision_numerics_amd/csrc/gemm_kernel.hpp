// The dense FP8 GEMM kernel template (see gemm.hip for the design notes and
// the host-side dispatch).
//
// Main loop of one workgroup, per 128-deep K step t (stage = t % 2):
//   * the direct-to-LDS loads of step t+1 into the other stage are issued
//     spread through the MFMA stream of step t (scheduling hints below);
//   * the wave's B fragments for step t are already in registers; its A
//     fragments are read one 16-row block ahead (af[(i+1)&1] while the MFMAs of
//     block i run), so LDS latency hides behind matrix-core time;
//   * at the end of the step: wait for this lane's loads, barrier, then read
//     the B fragments and the first A fragment of step t+1.
#pragma once

#include "gemm_tile.hpp"

namespace fp8mi {

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, int MODE>
__global__ __launch_bounds__(64 * WM* WN) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int M, int N, int K,
    const float* __restrict__ sinv_a, const float* __restrict__ sinv_b, void* __restrict__ C,
    int tiles_m, int tiles_n, int group_m) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int LQA = BM / 8 / NW, LQB = BN / 8 / NW;  // direct-load instructions per wave per step
  static_assert(FM >= 2 && FN >= 1 && BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile shape");
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, &tm, &tn);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;
  const int64_t m_base = (int64_t)tm * BM, n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK;
  const bool ragged_k = (K % kBK) != 0;

  // Per-lane source pointers of the direct loads (row clamped at the edge; the
  // granule index g is this lane's swizzled 16-B column of its row).
  const int r_in = lane >> 3, g = (lane & 7) ^ r_in;
  const uint8_t* pa[LQA];
  const uint8_t* pb[LQB];
#pragma unroll
  for (int q = 0; q < LQA; ++q) {
    int64_t r = m_base + (w + q * NW) * 8 + r_in;
    r = r < M ? r : M - 1;
    pa[q] = A + r * K + g * 16;
  }
#pragma unroll
  for (int q = 0; q < LQB; ++q) {
    int64_t r = n_base + (w + q * NW) * 8 + r_in;
    r = r < N ? r : N - 1;
    pb[q] = B + r * K + g * 16;
  }
  auto issue_direct = [&](int kt, int stage) {
    uint8_t* sa = smem + stage * STAGE;
    uint8_t* sb = sa + BM * kBK;
    const int k0 = kt * kBK;
#pragma unroll
    for (int q = 0; q < LQA; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(pa[q] + k0), (lds_void_t*)(sa + (w + q * NW) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < LQB; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(pb[q] + k0), (lds_void_t*)(sb + (w + q * NW) * 1024), 16, 0, 0);
  };
  // Zero-filled register path for a ragged last K step.
  auto stage_ragged = [&](int kt, int stage) {
    uint8_t* sa = smem + stage * STAGE;
    tile_load_zero_fill<BM, NT>(A, K, m_base, M, kt * kBK, K, sa, t);
    tile_load_zero_fill<BN, NT>(B, K, n_base, N, kt * kBK, K, sa + BM * kBK, t);
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int a_row = wm * WTM + (lane & 15), b_row = wn * WTN + (lane & 15);
  v8i bf[FN], af[2];

  // Contract the stage at `sa` (B fragments and the first A fragment already in registers).
  auto compute = [&](const uint8_t* sa) {
    if constexpr (MODE == kAccumMfma8) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) af[(i + 1) & 1] = lds_frag(sa, a_row + (i + 1) * 16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_fp8<FB, FA>(bf[j], af[i & 1], acc[i][j]);
      }
    } else {
      v8h bh[4][FN];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < FN; ++j) bh[s][j] = widen8<FB>((uint32_t)bf[j][2 * s], (uint32_t)bf[j][2 * s + 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) af[(i + 1) & 1] = lds_frag(sa, a_row + (i + 1) * 16, lane);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v8h ah = widen8<FA>((uint32_t)af[i & 1][2 * s], (uint32_t)af[i & 1][2 * s + 1]);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh[s][j], ah, acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  // Interleave hint for a step whose next-stage direct loads are in the same
  // block: per A block, its 2 LDS reads, half its MFMAs, a share of the loads,
  // the other half.
  auto interleave = [&]() {
    if constexpr (MODE == kAccumMfma8) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FN / 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (LQA + LQB + FM - 1) / FM, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FN - FN / 2, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * FN, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (LQA + LQB + FM - 1) / FM, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * FN, 0);
      }
    }
  };
  auto load_frags = [&](const uint8_t* sa) {
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = lds_frag(sa + BM * kBK, b_row + j * 16, lane);
    af[0] = lds_frag(sa, a_row, lane);
  };

  const int nfull = K / kBK;
  if (nfull > 0) issue_direct(0, 0); else stage_ragged(0, 0);
  wait_vmem();
  __syncthreads();
  load_frags(smem);
  // Full steps whose successor is also full: loads unconditional, interleaved.
  int kt = 0;
  for (; kt + 1 < nfull; ++kt) {
    const int cur = kt & 1;
    issue_direct(kt + 1, cur ^ 1);
    compute(smem + cur * STAGE);
    interleave();
    wait_vmem();
    __syncthreads();
    load_frags(smem + (cur ^ 1) * STAGE);
  }
  // Last full step (its successor, if any, is the ragged step), then the ragged step.
  if (kt < nfull) {
    const int cur = kt & 1;
    if (ragged_k) stage_ragged(kt + 1, cur ^ 1);
    compute(smem + cur * STAGE);
    ++kt;
    if (ragged_k) {
      wait_vmem();
      __syncthreads();
      load_frags(smem + (cur ^ 1) * STAGE);
    }
  }
  if (kt < nk) compute(smem + (kt & 1) * STAGE);

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

}  // namespace fp8mi
