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
// Output tiles are laid end to end over the experts' row ranges; each
// workgroup finds its expert from the device-side row offsets, so the host
// never needs the token counts.
//
// Both kernels use the dense kernel's data movement (gemm_kernel.hpp): two LDS
// stages filled by buffer loads issued one step ahead (rows past the expert's
// last row fall outside the buffer resource and are never stored), the
// measured LDS swizzle, and the output tile written through LDS as whole rows.
//
// * FP8 matrix-core mode: one V_MFMA_F32_16X16X128_F8F6F4 covers a whole
//   128-deep step of a 16x16 block, so its result IS the partial P and is
//   promoted right away; only the running accumulators stay live.  That allows
//   the dense kernel's wave tile (64x128, A fragments resident, B streamed) in
//   128x512 workgroup tiles: 128 rows because token counts come in multiples of
//   128, 512 columns so that each wave's 128 columns meet one weight block.
// * exact mode: the 16-deep bf16 instructions build P over eight sub-steps, so
//   P and the accumulator are both live; 128x128 tiles of four 64x64 waves,
//   two workgroups per CU.
//
// The A block scales (one per row and K step, rows far apart in memory) are
// never loaded per lane and step: the exact mode stages them through LDS eight
// steps at a time, the FP8 mode (whose LDS the slabs fill) has the four lanes
// of a row share them through ds_bpermute.
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

// Output tiles of BM rows are laid end to end over the experts' row intervals
// [m_offsets[g], m_offsets[g+1]) (made non-decreasing and clamped to
// [0, total_m]).  Finds the expert of M tile `mt` and the tile's first row and
// the expert's end row; false if `mt` lies past the last expert's tiles.  The
// arguments are uniform over the workgroup, so this runs on the scalar unit.
template <int BM>
__device__ __forceinline__ bool expert_tile(const int32_t* __restrict__ m_offsets, int G, int total_m, int mt,
                                            int* g_out, int64_t* row0, int64_t* row_end) {
  int acc_tiles = 0, prev = 0;
  for (int g = 0; g < G; ++g) {
    int lo = m_offsets[g], hi = m_offsets[g + 1];
    lo = lo < prev ? prev : (lo > total_m ? total_m : lo);
    hi = hi < lo ? lo : (hi > total_m ? total_m : hi);
    prev = hi;
    const int tiles = (hi - lo + BM - 1) / BM;
    if (mt < acc_tiles + tiles) {
      *g_out = g;
      *row0 = lo + (int64_t)(mt - acc_tiles) * BM;
      *row_end = hi;
      return true;
    }
    acc_tiles += tiles;
  }
  return false;
}

// Output tile (mt, tn) of workgroup `wg`.  GM == 0: consecutive workgroups
// walk the N tiles of one M tile (the round-robin deal of workgroups to the 8
// XCDs then gives each XCD a fixed set of columns).  GM > 0: each XCD takes a
// contiguous range of the real tiles (the M tiles the experts' rows fill, not
// the grid's upper bound, so the padding tiles do not pile up on one XCD),
// walked in bands of GM M tiles, so the workgroups resident on one XCD form a
// compact block of tiles.  False for a workgroup with no tile.  The grid must
// be a multiple of 8 workgroups at least as large as the tile count.
template <int BM, int GM>
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ m_offsets, int G, int total_m, int tiles_n,
                                             int wg, int* mt, int* tn) {
  if constexpr (GM == 0) {
    *tn = wg % tiles_n;
    *mt = wg / tiles_n;
    return true;
  } else {
    int real_m = 0, prev = 0;
    for (int g = 0; g < G; ++g) {
      int lo = m_offsets[g], hi = m_offsets[g + 1];
      lo = lo < prev ? prev : (lo > total_m ? total_m : lo);
      hi = hi < lo ? lo : (hi > total_m ? total_m : hi);
      prev = hi;
      real_m += (hi - lo + BM - 1) / BM;
    }
    const int total = real_m * tiles_n;
    const int per_xcd = (total + 7) >> 3;
    const int j = wg >> 3;
    if (j >= per_xcd) return false;
    const int pid = (wg & 7) * per_xcd + j;
    if (pid >= total) return false;
    const int in_group = GM * tiles_n;
    const int gid = pid / in_group;
    const int first_m = gid * GM;
    const int gsize = (real_m - first_m) < GM ? (real_m - first_m) : GM;
    const int local = pid - gid * in_group;
    *mt = first_m + local % gsize;
    *tn = local / gsize;
    return true;
  }
}

// ---------------------------------------------------------------------------
// FP8 matrix-core mode.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int OUT, int GM = 0>
__global__ __launch_bounds__(64 * WM* WN) void grouped_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sinv_a, const uint8_t* __restrict__ B,
    const float* __restrict__ sinv_b, const int32_t* __restrict__ m_offsets, int G, int total_m,
    int N, int K, void* __restrict__ C, int tiles_n) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(WTM % 16 == 0 && WTN == 128, "a wave's columns must be one 128-wide weight block");
  static_assert(FN >= kDmaGroups, "one load group per leading B block");
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  int mt, tn;
  if (!grouped_tile<BM, GM>(m_offsets, G, total_m, tiles_n, blockIdx.x, &mt, &tn)) return;  // uniform exit
  int gidx;
  int64_t row0, row_end;
  if (!expert_tile<BM>(m_offsets, G, total_m, mt, &gidx, &row0, &row_end)) return;  // uniform exit

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;
  const int64_t n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK, nfull = K / kBK;
  const bool ragged_k = (K % kBK) != 0;
  const int nbn = (N + 127) / 128;
  const uint8_t* Bg = B + (int64_t)gidx * N * K;

  const SlabLoader<BM, BN, NW> slabs(A, row0, row_end, Bg, n_base, N, K, w, lane);
  auto issue_direct = [&](uint8_t* dst, int kt, int g) { slabs.issue(dst, kt, g); };
  auto stage_ragged = [&](int kt, int stage) { slabs.ragged(smem + stage * STAGE, kt, t); };

  // 16x16x128 fragments: lane l takes row l & 15 of a 16-row block and the
  // 32-byte K slice l >> 4 (granules 2h, 2h+1).
  const int rr = lane & 15, hh = lane >> 4;
  const int swz = lds_swz(rr);
  auto frag = [&](const uint8_t* tile, int r0) {
    const uint8_t* p = tile + (r0 + rr) * kBK;
    const uint4 lo = *reinterpret_cast<const uint4*>(p + (((2 * hh) ^ swz) & 7) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + (((2 * hh + 1) ^ swz) & 7) * 16);
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // Block scales of the lane's output row in each A block and of the wave's
  // weight block, one step ahead: the values of step kt+1 are loaded while
  // step kt runs.  The four lanes of a row (hh = 0..3, one K slice each) share
  // its A scales: lane hh of block i holds step s + hh, for the last step
  // s <= kt with s % 4 == i, and each step takes its value from lane
  // rr + 16*((kt - i) % 4) with ds_bpermute.  Step kt refreshes only block
  // kt % 4, from the one load issued during step kt - 1 (16 rows x 16 bytes).
  // Loading every row's scale in every lane and step cost 13 % (MoE shape,
  // MI355X, identical output: 563.6 against 491.2 us for all four blocks
  // refreshed every fourth step, that form 1.8 % slower than this one); a
  // branch around those loads made the register allocator spill.  One buffer
  // resource covers the wave's rows inside the expert; rows past it read as
  // zero and are never stored.
  static_assert(FM == 4, "one A block refreshed per step of a 4-step group");
  const int64_t tile_rows = row_end - row0 < BM ? row_end - row0 : BM;
  const int64_t wave_rows = tile_rows - wm * WTM < 0 ? 0 : (tile_rows - wm * WTM < WTM ? tile_rows - wm * WTM : WTM);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(sinv_a + (row0 + wm * WTM) * nk), (short)0, (int)(uint32_t)(wave_rows * nk * 4),
      kBufferRsrcWord3);
  auto steps_voff = [&](int blk, int first) {  // block blk, steps first .. first+3 (clamped)
    int k = first + hh;
    k = k < 0 ? 0 : (k < nk ? k : nk - 1);
    return (uint32_t)(((blk * 16 + rr) * nk + k) * 4);
  };
  const int nb = (int)((n_base + wn * WTN) >> 7);
  const float* sb_blk = sinv_b + ((int64_t)gidx * nbn + (nb < nbn ? nb : nbn - 1)) * nk;
  float sa_q[FM], sa_next, sb_n;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    sa_q[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, steps_voff(i, i - 4), 0, 0));
  auto load_scales = [&](int kt) {
    sa_next = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, steps_voff(kt & 3, kt), 0, 0));
    sb_n = sb_blk[kt];
  };
  load_scales(0);
  int kstep = 0;

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  v8i af[FM], bf[2];
  auto load_frags = [&](const uint8_t* st) {
    bf[0] = frag(st + BM * kBK, wn * WTN);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = frag(st, wm * WTM + i * 16);
  };
  // One step.  Each MFMA's partial is promoted after the next MFMA has been
  // issued, so the promotion does not wait for the product it consumes.
  auto compute = [&](const uint8_t* st, auto&& dma) {
    float s[FM];
    {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        sa_q[i] = (kstep & 3) == i ? sa_next : sa_q[i];
        const int src = (rr + 16 * ((kstep - i) & 3)) * 4;
        s[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sa_q[i]))) * sb_n;
      }
    }
    ++kstep;
    load_scales(kstep < nk ? kstep : nk - 1);
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f p[2];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (j < kDmaGroups) dma(j);
      if (j + 1 < FN) bf[(j + 1) & 1] = frag(st + BM * kBK, wn * WTN + (j + 1) * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int c = j * FM + i;
        p[c & 1] = mfma_fp8<kE4M3, kE4M3>(bf[j & 1], af[i], zero);
        if (c > 0) {
          const int jp = (c - 1) / FM, ip = (c - 1) % FM;
          acc[ip][jp] += p[(c - 1) & 1] * s[ip];
        }
      }
    }
    acc[FM - 1][FN - 1] += p[(FM * FN - 1) & 1] * s[FM - 1];
  };
  auto interleave = [&]() {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM, 0);
    }
  };
  run_main_loop(smem, smem + STAGE, nfull, nk, ragged_k, issue_direct, stage_ragged, load_frags, compute,
                interleave);

  // Lane l holds row m = l & 15 of each 16x16 block (the A operand went
  // second) and columns n = 4(l >> 4) .. +3; rows past the expert are not stored.
  using TW = TileWriter<OUT, BM, BN, NT>;
  constexpr int PASS = pass_rows<BM>(2 * STAGE, TW::ROWB);
  TW tw{smem, PASS};
#pragma unroll 1
  for (int r0 = 0; r0 < BM; r0 += PASS) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 16 + rr;
      if (r < r0 || r >= r0 + PASS) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) tw.put(r - r0, wn * WTN + j * 16 + 4 * hh, acc[i][j]);
    }
    __syncthreads();
    tw.flush(C, row_end, N, row0 + r0, n_base, t);
  }
}

// ---------------------------------------------------------------------------
// Exact mode (FP8 widened to bf16, 32x32x16 instructions).
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(64 * WM* WN) void grouped_exact_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sinv_a, const uint8_t* __restrict__ B,
    const float* __restrict__ sinv_b, const int32_t* __restrict__ m_offsets, int G, int total_m,
    int N, int K, void* __restrict__ C, int tiles_n) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && WTN <= 128, "wave tile shape");
  constexpr int STAGE = (BM + BN) * kBK;
  // A scales in LDS, SCH steps at a time: two chunks of [BM rows][SCH steps] fp32.
  constexpr int SCH = 8, SCB = BM * SCH * 4;
  static_assert(BM == 16 * SCH && NW >= 2, "each step loads 16 rows of the next chunk, 8 per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + 2 * SCB];

  // The plain order (grouped_tile<BM, 0>): the banded ones measured 1 % slower here.
  int mt, tn;
  if (!grouped_tile<BM, 0>(m_offsets, G, total_m, tiles_n, blockIdx.x, &mt, &tn)) return;  // uniform exit
  int gidx;
  int64_t row0, row_end;
  if (!expert_tile<BM>(m_offsets, G, total_m, mt, &gidx, &row0, &row_end)) return;  // uniform exit

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;
  const int64_t n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK, nfull = K / kBK;
  const int nbn = (N + 127) / 128;
  const uint8_t* Bg = B + (int64_t)gidx * N * K;
  const float* sbg = sinv_b + (int64_t)gidx * nbn * nk;

  const SlabLoader<BM, BN, NW> slabs(A, row0, row_end, Bg, n_base, N, K, w, lane);
  auto fill = [&](uint8_t* st, int kt) {
    if (kt < nfull) {
#pragma unroll
      for (int g = 0; g < kDmaGroups; ++g) slabs.issue(st, kt, g);
    } else {
      slabs.ragged(st, kt, t);
    }
  };

  // 32x32x16 fragments (eight K sub-steps of 16): lane l takes row l & 31 of a
  // 32-row block and the 64-byte half l >> 5 of the step (granules 4h..4h+3);
  // sub-step s uses bytes [8s, 8s+8) of it, for both operands alike.
  const int rr = lane & 31, hh = lane >> 5;
  const int swz = lds_swz(rr);
  auto granule = [&](const uint8_t* tile, int r0, int g) {
    return *reinterpret_cast<const uint4*>(tile + (r0 + rr) * kBK + (((g ^ swz) & 7) << 4));
  };

  // The A scales of the tile's rows come through LDS in chunks of SCH steps,
  // loaded like the slabs (direct to LDS, published by the stage barrier): one
  // dword load covers 8 rows x SCH steps (lane l: row l >> 3, step l & 7), and
  // the next chunk's 16 rows per step are loaded while the current chunk is in
  // use.  Read straight from global memory, each wave's per-row loads touched
  // 32 cache lines per instruction, and the kernel ran 6 % slower (MoE shape,
  // MI355X, identical output: 830.6 against 783.1 us).  Rows past the expert
  // fall outside the buffer resource (the tile's rows inside the expert) and
  // read as zero; steps past the last read other rows' scales and are never
  // used.
  const int64_t tile_rows = row_end - row0 < BM ? row_end - row0 : BM;
  const int64_t sa_bytes = tile_rows * nk * 4 < 0xFFFFFFFFll ? tile_rows * nk * 4 : 0xFFFFFFFFll;
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(sinv_a + row0 * nk), (short)0, (int)(uint32_t)sa_bytes, kBufferRsrcWord3);
  const int sa_lane = ((lane >> 3) * nk + (lane & 7)) * 4;
  auto scale_rows = [&](int chunk, int rb) {  // rows rb .. rb+7 of chunk `chunk`
    dma_lds4(rsa, lds_addr(smem + 2 * STAGE + (chunk & 1) * SCB) + rb * SCH * 4,
             sa_lane + (rb * nk + chunk * SCH) * 4, 0);
  };
  const float* const sa_lds = reinterpret_cast<const float*>(smem + 2 * STAGE);
  // The 128-column weight block of each B block.
  int bblk[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int nb = (int)((n_base + wn * WTN + j * 32) / 128);
    bblk[j] = nb < nbn ? nb : nbn - 1;
  }

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (v16f){};

  uint8_t* const s0 = smem;
  uint8_t* const s1 = smem + STAGE;
  fill(s0, 0);
#pragma unroll
  for (int u = 0; u < BM / 8 / NW; ++u) scale_rows(0, 8 * (w + u * NW));
  wait_loads_and_barrier();
  // Each wave runs at raised priority (s_setprio) for the first half of a
  // step: the two waves of a SIMD (one per workgroup) then stop contending
  // for issue in lockstep.  MoE shape, MI355X, identical output: 812.9 against
  // 841.6 us (raised until sub-step 2, 3, 4, 5 or 6: -1.7, -2.6, -3.4, -2.2,
  // -2.4 %).
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* cur = (kt & 1) ? s1 : s0;
    uint8_t* nxt = (kt & 1) ? s0 : s1;
    float sa_v[FM], sb_v[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa_v[i] = sa_lds[((kt / SCH) & 1) * (BM * SCH) + (wm * WTM + i * 32 + rr) * SCH + kt % SCH];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb_v[j] = sbg[bblk[j] * nk + kt];
    if (kt + 1 < nk) fill(nxt, kt + 1);
    if (w < 2 && (kt / SCH + 1) * SCH < nk) scale_rows(kt / SCH + 1, (kt % SCH) * 16 + 8 * w);
    __builtin_amdgcn_sched_barrier(0);
    v16f part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) part[i][j] = (v16f){};
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
      if (s == 4) __builtin_amdgcn_s_setprio(0);
      v8bf bh[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 g = br[j][s >> 1];
        bh[j] = widen8_scaled_bf16<kE4M3>((s & 1) ? g.z : g.x, (s & 1) ? g.w : g.y, 1.0f);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 g = ar[i][s >> 1];
        const v8bf ah = widen8_scaled_bf16<kE4M3>((s & 1) ? g.z : g.x, (s & 1) ? g.w : g.y, 1.0f);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[j], ah, part[i][j], 0, 0, 0);
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

  // Lane l holds row m = l & 31 of each 32x32 block and columns
  // n = 8g + 4(l >> 5) + 0..3 in registers 4g..4g+3; rows past the expert are
  // not stored.
  using TW = TileWriter<OUT, BM, BN, NT>;
  constexpr int PASS = pass_rows<BM>(2 * STAGE, TW::ROWB);
  TW tw{smem, PASS};
#pragma unroll 1
  for (int r0 = 0; r0 < BM; r0 += PASS) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + rr;
      if (r < r0 || r >= r0 + PASS) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v4f v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          tw.put(r - r0, wn * WTN + j * 32 + 8 * g + 4 * hh, v);
        }
    }
    __syncthreads();
    tw.flush(C, row_end, N, row0 + r0, n_base, t);
  }
}

// Grid: N tiles times an upper bound on the M tiles over any split of total_m
// rows into G experts (each expert adds at most one partial tile), rounded up
// to a multiple of the 8 XCDs (grouped_tile); workgroups past the real tiles
// exit at once.
template <int BM, int BN>
dim3 grouped_grid(int64_t total_m, int G, int64_t N, int* tiles_n) {
  *tiles_n = (int)((N + BN - 1) / BN);
  const int64_t tiles_m = (total_m + BM - 1) / BM + G;
  return dim3((unsigned)((tiles_m * *tiles_n + 7) / 8 * 8));
}

template <int BM, int BN, int WM, int WN, int OUT>
hipError_t run_fp8(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb, const int32_t* offs,
                   int G, int64_t total_m, int64_t N, int64_t K, void* C, hipStream_t st) {
  int tiles_n;
  const dim3 grid = grouped_grid<BM, BN>(total_m, G, N, &tiles_n);
  // Bands of 4 M tiles (MoE shape, MI355X, identical output): 5 % faster than
  // the plain order launched back to back, level with it (0.4 %) right after
  // the block quantisers and the exact kernel.
  hipLaunchKernelGGL((grouped_fp8_kernel<BM, BN, WM, WN, OUT, 4>), grid, dim3(64 * WM * WN), 0, st, A, sa, B, sb,
                     offs, G, (int)total_m, (int)N, (int)K, C, tiles_n);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int OUT>
hipError_t run_exact(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb, const int32_t* offs,
                     int G, int64_t total_m, int64_t N, int64_t K, void* C, hipStream_t st) {
  int tiles_n;
  const dim3 grid = grouped_grid<BM, BN>(total_m, G, N, &tiles_n);
  hipLaunchKernelGGL((grouped_exact_kernel<BM, BN, WM, WN, OUT>), grid, dim3(64 * WM * WN), 0, st, A, sa, B, sb,
                     offs, G, (int)total_m, (int)N, (int)K, C, tiles_n);
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
      return run_fp8<128, 512, 2, 4, kBF16>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
    return run_fp8<128, 512, 2, 4, kF32>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
  }
  if (ctype == kBF16)
    return run_exact<128, 128, 2, 2, kBF16>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
  return run_exact<128, 128, 2, 2, kF32>(A, sinv_a, B, sinv_b, m_offsets, G, total_m, N, K, C, stream);
}

}  // namespace fp8mi
