// The dense FP8 GEMM kernel template (see gemm.hip for the design notes and
// the host-side dispatch).
//
// Main loop of one workgroup, per 128-deep K step t (stage = t % 2):
//   * the direct-to-LDS loads of step t+1 into the other stage are issued in
//     groups between the first MFMA blocks of step t and only waited for at
//     the end of the step, so their latency overlaps the step;
//   * FP8 path: the wave's A fragments for step t are in registers; its B
//     fragments are read one 16-row block ahead (bf[(j+1)&1] while the MFMAs
//     of block j run).  bf16 paths: the raw FP8 fragments of the step are read
//     one 16-byte granule ahead of the sub-steps that use them and widened to
//     bf16 per 16-deep sub-step;
//   * at the end of the step: wait for this lane's loads, barrier, then read
//     the fragments of step t+1.
//
// Operand slabs are fetched with buffer loads: one buffer resource per tile
// covers the rows [tile start, M) (or N) of the operand.  The hardware range
// check compares only the per-lane (VGPR) offset with the resource's size; the
// scalar offset is added after the check.  So each load carries its whole row
// position in the VGPR offset and only the K offset of the step (which stays
// inside a row that passed the check) in the scalar one: rows past the edge
// then fail the check, read as zero without touching memory, and only feed
// output rows or columns that are not stored.
#pragma once

#include <type_traits>

#include "gemm_tile.hpp"

namespace fp8mi {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Output kinds of the epilogue besides fp32 and bf16 (kF32, kBF16): FP8 codes
// of the result re-quantised with a caller-supplied scale.
enum : int { kOutE4M3 = 2, kOutE5M2 = 3 };
template <int OUT>
constexpr int out_bytes() {
  return OUT == kF32 ? 4 : (OUT == kBF16 ? 2 : 1);
}

// Where a re-quantising epilogue sends its by-products: the scale to apply,
// the amax of the unscaled result (as fp32 bits) and the saturation count
// (either pointer may be null).  Unused by the fp32 / bf16 outputs.
struct RequantArgs {
  const float* out_scale;
  uint32_t* amax_bits;
  unsigned long long* sat;
};

// E8M0 block-scale matrices of an MXFP8 GEMM (one byte per 32 K values of a
// row of A and of B); unused by the other modes.
struct MxScales {
  const uint8_t* a;
  const uint8_t* b;
};

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;

// dword 3 of a raw (untyped, stride 0) buffer resource on gfx9: 32-bit data format.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint8_t* base, int64_t rows_left, int64_t ld) {
  int64_t bytes = rows_left * ld;
  bytes = bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)(uint32_t)bytes, kBufferRsrcWord3);
}

// Buffer loads with the LDS as destination, written as inline assembly so that
// the compiler does not track them: it cannot tell the stages apart and would
// otherwise wait for every such load before any later LDS read it cannot prove
// disjoint, i.e. right after issuing them.  The kernel waits for them itself (vmcnt) before the
// barrier that publishes a stage.  Lane i writes `bytes` at LDS address
// lds + i*bytes; M0 carries the LDS base (one wait state after it is written).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
__device__ __forceinline__ void dma_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ void dma_lds4(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
               : "memory");
}

// The next stage's loads are issued in this many groups within a step.
constexpr int kDmaGroups = 4;

// The operand slabs of one output tile: rows [m0, m_end) of A and [n0, n_end)
// of B, both row-major with K bytes per row, fetched 128 K bytes per step.
// Direct loads: load q of wave w fills tile rows (w + q*NW)*8 .. +7; lane i
// fills position i & 7 of row i >> 3 of that group with the granule stored
// there under the swizzle (which depends on the row's low 4 bits only, i.e. not
// on q since NW is even).  One buffer resource per operand covers its rows
// from the tile start to the edge.  The lane's row offset of load q,
// voff + q*NW*8*K, is a VGPR operand, so the range check sees the row: rows
// past the edge read as zero without touching memory.  Only k0 (< K, and the
// 16 bytes at k0 + granule stay inside the row) is a scalar offset.
//
// BT (B stored [K x N], N contiguous, as the operand of C = A B): the B slab of
// a step is 128 K rows of BN bytes in its natural orientation, the 16-byte
// granule q of K row r at position q ^ (r & 7) (see bt_lds_offset).  Wave
// load e fills K rows e*RPB .. +RPB-1 (RPB = 1024 / BN rows per instruction);
// lane i fills position i % (BN/16) of row i / (BN/16) with the granule that
// belongs there.  Since NW is even, the parity of e and so the lane's source
// granule is the same for every load of the wave: one VGPR offset serves them
// all.  Columns at or past N get an offset above the resource's size, so they
// read as zero without touching memory; rows at or past K can only occur in a
// ragged last step, whose loads carry the row in the VGPR offset as well.
template <int BN>
__device__ __forceinline__ int bt_lds_offset(int krow, int col) {
  return krow * BN + ((((col >> 4) ^ (krow & 7)) << 4) | (col & 15));
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // above any operand size these loads allow (< 2^31 bytes)

template <int BM, int BN, int NW, bool BT = false>
struct SlabLoader {
  static constexpr int LQA = BM / 8 / NW, LQB = BN / 8 / NW;  // direct-load instructions per wave per step
  static constexpr int PER = (LQA + LQB + kDmaGroups - 1) / kDmaGroups;
  static constexpr int RPB = 1024 / BN;                       // BT: K rows per load instruction
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split evenly over the wavefronts");
  static_assert(NW % 2 == 0, "the swizzle of a lane's load must not depend on its row group");
  static_assert(!BT || (BN >= 128 && BN <= 1024 && 128 % (RPB * NW) == 0), "BT slab shape");
  const uint8_t* A;
  const uint8_t* B;
  int64_t m0, m_end, n0, n_end;
  int K, w, voff;
  int ldb;            // BT: bytes per K row of B (= N)
  uint32_t voff_bt;   // BT: the lane's offset in the first K row group, or kOutOfRange
  __amdgpu_buffer_rsrc_t ra, rb;

  __device__ __forceinline__ SlabLoader(const uint8_t* A_, int64_t m0_, int64_t m_end_, const uint8_t* B_,
                                        int64_t n0_, int64_t n_end_, int K_, int w_, int lane)
      : A(A_), B(B_), m0(m0_), m_end(m_end_), n0(n0_), n_end(n_end_), K(K_), w(w_) {
    ra = operand_rsrc(A + m0 * K, m_end - m0, K);
    const int lrow = w * 8 + (lane >> 3);
    voff = lrow * K + (((lane & 7) ^ lds_swz(lrow)) & 7) * 16;
    if constexpr (BT) {
      ldb = (int)n_end;
      rb = operand_rsrc(B, K, ldb);  // the whole [K x N] matrix
      const int r = w * RPB + lane / (BN / 16);                  // K row of load 0 (same parity for every load)
      const int q = (lane % (BN / 16)) ^ (r & 7);                // source granule of the lane
      const int64_t col = n0 + 16 * q;
      voff_bt = col < n_end ? (uint32_t)(r * ldb + col) : kOutOfRange;
    } else {
      ldb = K;
      voff_bt = 0;
      rb = operand_rsrc(B + n0 * K, n_end - n0, K);
    }
  }
  // Group g of the loads of step kt into the stage at `dst`: loads
  // d = g*PER .. of the wave's LQA + LQB (A first).  A group is pinned where it
  // is issued.
  __device__ __forceinline__ void issue(uint8_t* dst, int kt, int g) const {
    const int k0 = kt * kBK;
    const uint32_t la = lds_addr(dst) + w * 1024, lb = lds_addr(dst + BM * kBK) + w * 1024;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = g * PER + e;
      if (d >= LQA + LQB) break;
      if (d < LQA) dma_lds16(ra, la + d * NW * 1024, voff + d * NW * 8 * K, k0);
      else if constexpr (BT)  // a full step: every K row exists, only the column needs the range check
        dma_lds16(rb, lb + (d - LQA) * NW * 1024, (int)voff_bt, ((d - LQA) * NW * RPB + k0) * ldb);
      else dma_lds16(rb, lb + (d - LQA) * NW * 1024, voff + (d - LQA) * NW * 8 * K, k0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // A ragged last K step (all threads of the workgroup): A zero-filled through
  // registers; B likewise, or (BT) by direct loads whose VGPR offset carries
  // the row, so K rows past the end read as zero.
  __device__ __forceinline__ void ragged(uint8_t* dst, int kt, int t) const {
    tile_load_zero_fill<BM, 64 * NW>(A, K, m0, m_end, kt * kBK, K, dst, t);
    if constexpr (BT) {
      const uint32_t lb = lds_addr(dst + BM * kBK) + w * 1024;
#pragma unroll
      for (int d = 0; d < LQB; ++d)
        dma_lds16(rb, lb + d * NW * 1024, (int)(voff_bt + (uint32_t)((d * NW * RPB + kt * kBK) * ldb)), 0);
    } else {
      tile_load_zero_fill<BN, 64 * NW>(B, K, n0, n_end, kt * kBK, K, dst + BM * kBK, t);
    }
  }
};

// The K loop shared by both accumulation modes.  `step` handles one full step
// whose successor is also full: load step kt+1 into `nxt` while contracting
// `cur`.  Two steps per iteration keep each stage pointer fixed at compile
// time.
//
// The end of a step waits for this wave's loads and LDS reads, then meets the
// other wavefronts at a plain barrier: after it, every wave's slab of the next
// stage is in the LDS and no wave still reads the stage about to be refilled.
// (An L2 prefetch of the step after next, one dword per line, was measured
// slower: it only added L2 traffic.)
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

template <class Issue, class Ragged, class Frags, class Compute, class Hint>
__device__ __forceinline__ void run_main_loop(uint8_t* s0, uint8_t* s1, int nfull, int nk, bool ragged_k,
                                              Issue& issue_direct, Ragged& stage_ragged, Frags& load_frags,
                                              Compute& compute, Hint& interleave, bool first_issued = false) {
  // The loads of step kt+1 go out in groups between the first MFMA blocks of
  // step kt (the hook `dma(g)`): issued all at once they back up the wave's
  // memory-instruction queue and stall its MFMAs.  The MFMAs stay inside their
  // step (sched_barrier): the scheduler would otherwise sink them below the
  // barrier, where they no longer hide the loads.
  auto step = [&](uint8_t* nxt, const uint8_t* cur, int kt_next) {
    compute(cur, [&](int g) { issue_direct(nxt, kt_next, g); });
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    wait_loads_and_barrier();
    load_frags(nxt);
  };
  auto no_dma = [](int) {};
  if (nfull > 0) {
    if (!first_issued)
      for (int g = 0; g < kDmaGroups; ++g) issue_direct(s0, 0, g);
    wait_loads_and_barrier();
    load_frags(s0);
  } else {
    stage_ragged(0, 0);
    wait_vmem();
    __syncthreads();
  }
  int kt = 0;
  for (; kt + 2 < nfull; kt += 2) {
    step(s1, s0, kt + 1);
    step(s0, s1, kt + 2);
  }
  if (kt + 1 < nfull) {
    step(s1, s0, kt + 1);
    ++kt;
  }
  // Last full step (its successor, if any, is the ragged step), then the
  // ragged step, which reads its own fragments: loaded inside the branch on
  // ragged_k and merged with the registers of the other path, they made the
  // FP8-core kernel with MX scales spill at the join.  Each step keeps the
  // loop body's scheduling hint, or its fragment reads are all hoisted ahead
  // of its MFMAs.
  if (kt < nfull) {
    uint8_t* cur = (kt & 1) ? s1 : s0;
    if (ragged_k) stage_ragged(kt + 1, (kt & 1) ^ 1);
    compute(cur, no_dma);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    ++kt;
    if (ragged_k) {
      wait_vmem();
      __syncthreads();
    }
  }
  if (kt < nk) {
    uint8_t* cur = (kt & 1) ? s1 : s0;
    load_frags(cur);
    compute(cur, no_dma);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmem();  // no load may still be writing the LDS when the epilogue reuses it
}

// Epilogue: the scaled output tile goes through LDS (free once the K loop is
// done) so that global stores are whole contiguous rows: each lane stores 16
// bytes, consecutive lanes consecutive addresses.  Storing straight from the
// matrix-core layout writes 8-16 byte pieces of many rows per instruction,
// which costs several times the output's size in memory traffic.  Tile rows
// are BN*sizeof(out) bytes (1 per FP8 code); the 16-byte granule q of row r sits at position
// q ^ (r mod min(granules per row, 32)).  A tile that does not fit the LDS goes
// out in row passes.
template <int OUT, int BM, int BN, int NT>
struct TileWriter {
  static constexpr int CB = out_bytes<OUT>();              // bytes per output element
  static constexpr int ROWB = BN * CB;                     // bytes per tile row
  static constexpr int GR = ROWB / 16;                     // granules per row
  static constexpr int SWZ = (GR < 32 ? GR : 32) - 1;
  static_assert(GR >= 8 && (GR & (GR - 1)) == 0, "tile row must be a power-of-two number of granules");
  uint8_t* lds;
  int pass_rows;
  __device__ __forceinline__ int pos(int r, int byte) const {
    return r * ROWB + ((((byte >> 4) ^ (r & SWZ)) & (GR - 1)) << 4) + (byte & 15);
  }
  // Four consecutive outputs (n_local multiple of 4) of tile row r_local, already scaled.
  __device__ __forceinline__ void put(int r_local, int n_local, const v4f& v) const {
    uint8_t* p = lds + pos(r_local, n_local * CB);
    if constexpr (OUT == kF32) {
      *reinterpret_cast<v4f*>(p) = v;
    } else {
      const v2bf lo = __builtin_convertvector((v2f){v[0], v[1]}, v2bf);
      const v2bf hi = __builtin_convertvector((v2f){v[2], v[3]}, v2bf);
      *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  }
  // Four FP8 codes (byte i = column n_local + i) of tile row r_local.
  __device__ __forceinline__ void put_codes(int r_local, int n_local, uint32_t codes) const {
    *reinterpret_cast<uint32_t*>(lds + pos(r_local, n_local)) = codes;
  }
  // Copy rows [0, pass_rows) of the staged pass to C rows m0.. (all threads).
  __device__ __forceinline__ void flush(void* C, int64_t M, int64_t N, int64_t m0, int64_t n0, int t) const {
    const bool full_cols = n0 + BN <= N && ((N * CB) & 15) == 0;
    for (int idx = t; idx < pass_rows * GR; idx += NT) {
      const int r = idx / GR, q = idx % GR;
      const int64_t m = m0 + r;
      if (m >= M) break;  // rows are visited in order
      const uint4 v = *reinterpret_cast<const uint4*>(lds + pos(r, q * 16));
      uint8_t* dst = reinterpret_cast<uint8_t*>(C) + (m * N + n0) * CB + q * 16;
      if (full_cols) {
        // Nontemporal: the output is not read again by this kernel, and
        // streaming it past the caches made the FC1 GEMM 5 % faster on MI355X.
        u32x4 vv;
        vv[0] = v.x;
        vv[1] = v.y;
        vv[2] = v.z;
        vv[3] = v.w;
        __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(dst));
      } else {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(&v);
        const int64_t nq = n0 + q * (16 / CB);
        for (int e = 0; e < 16 / CB; ++e)
          if (nq + e < N) {
            if constexpr (CB == 4) reinterpret_cast<float*>(dst)[e] = reinterpret_cast<const float*>(src)[e];
            else if constexpr (CB == 2) reinterpret_cast<uint16_t*>(dst)[e] = reinterpret_cast<const uint16_t*>(src)[e];
            else dst[e] = src[e];
          }
      }
    }
  }
};

// Rows of one output pass through the LDS: the largest power of two that fits
// `bytes` and divides a tile of BM rows.
template <int BM>
constexpr int pass_rows(int bytes, int row_bytes) {
  int p = BM;
  while (p > 1 && p * row_bytes > bytes) p >>= 1;
  return p;
}

// Fold one lane's amax bits and the wave's saturation count of the
// re-quantised output into the global results: a wave-wide reduction, then one
// device-scope atomic per wave, skipped when the wave's maximum does not exceed
// `seen` (the global value read before the epilogue began: the global maximum
// only grows after it is cleared, so an older value is a safe lower bound) or
// its count is 0.
__device__ __forceinline__ void publish_requant_stats(uint32_t amax_bits_lane, uint32_t sat_wave, uint32_t seen,
                                                      const RequantArgs& rq, int lane) {
  const uint32_t m = wave_max_u32(amax_bits_lane);
  if (lane == 0) {
    if (rq.amax_bits && m > seen) atomicMax(rq.amax_bits, m);
    if (rq.sat && sat_wave) atomicAdd(rq.sat, (unsigned long long)sat_wave);
  }
}

// Block scales of one MXFP8 step.  The scale matrices are stored K-block
// major, rows permuted within groups of 64: byte (row r, block b) at
// b * ld + mx_scale_pos(r), ld = rows rounded up to 64 (mx_scale_ld).  One K
// block's scales of a 64-row group are then contiguous, and the four rows
// c, c+16, c+32, c+48 of a group sit in one dword: the four 16-row fragments of
// a 64-row wave tile take their scales from one LDS dword (the instruction
// picks the byte).  A step needs blocks 4kt .. 4kt+3 of the tile's BM rows of A and
// BN rows of B: BM + BN dwords of 4 rows each, one per lane of the workgroup
// (entry e = 64 w + lane: A entries first, entry e of A covers block
// e / (BM/4) and positions 4 (e % (BM/4)) .. +3), fetched with one dword load
// to LDS per wave.  In the stage's scale area the byte of A row r, block b
// sits at b * BM + mx_scale_pos(r), that of B row r at 4 BM + b * BN +
// mx_scale_pos(r) (tile starts are multiples of 64).  Rows past the edge only
// feed outputs that are not stored.  The step's block offset kt * 4 * ld is
// part of the VGPR offset, so the range check covers the whole address: in an
// edge tile the positions past ld belong to the next block's rows (in bounds,
// feeding only outputs that are not stored), and past the last block they read
// as zero without touching memory.
__host__ __device__ constexpr int64_t mx_scale_ld(int64_t rows) { return (rows + 63) / 64 * 64; }
__host__ __device__ constexpr int64_t mx_scale_pos(int64_t r) { return (r & ~int64_t(63)) | ((r & 15) << 2) | ((r >> 4) & 3); }

// With fewer lanes than dwords (4-wave tiles: 256 lanes for 512 dwords) each
// lane issues PER loads, entry e + u * 64 * NW for u < PER.  BM is a multiple
// of 64, so each wave's load u is all A or all B (a wave-uniform choice).
template <int BM, int BN, int NW>
struct MxScaleLoader {
  static constexpr int PER = (BM + BN) / (64 * NW);
  static_assert(PER >= 1 && BM + BN == PER * 64 * NW && BM % 64 == 0, "whole dwords of scales per lane");
  __amdgpu_buffer_rsrc_t r[PER];
  int voff[PER], step[PER];
  int w;
  __device__ __forceinline__ MxScaleLoader(const MxScales& sx, int64_t m0, int64_t M, int64_t n0, int64_t N, int K,
                                           int w_, int lane)
      : w(w_) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = w * 64 + lane + u * 64 * NW;
      if ((w + u * NW) * 64 < BM) {  // uniform over the wave
        const int64_t ld = mx_scale_ld(M);
        r[u] = operand_rsrc(sx.a, K / 32, ld);
        voff[u] = (int)((e / (BM / 4)) * ld + m0 + 4 * (e % (BM / 4)));
        step[u] = (int)(4 * ld);
      } else {
        const int64_t ld = mx_scale_ld(N);
        const int f = e - BM;
        r[u] = operand_rsrc(sx.b, K / 32, ld);
        voff[u] = (int)((f / (BN / 4)) * ld + n0 + 4 * (f % (BN / 4)));
        step[u] = (int)(4 * ld);
      }
    }
  }
  __device__ __forceinline__ void issue(uint8_t* scale_area, int kt) const {
#pragma unroll
    for (int u = 0; u < PER; ++u)
      dma_lds4(r[u], lds_addr(scale_area) + (w + u * NW) * 256, voff[u] + kt * step[u], 0);
  }
};

// kAccumMxExact: the reference exponent of every row of the tile and whether
// the row's block exponents fit the exact path.  Scale codes c (2^(c - 127))
// are scanned over all K/32 blocks; R = the row's largest code.  A block of
// code c is widened with the factor 2^(c - R), so the smallest nonzero value
// of the row becomes at least 2^-16 (the smallest E5M2 subnormal) times
// 2^-(span), span = R - (the row's smallest code); with span <= kMxExactSpan
// for both operands every nonzero product is at least 2^-126 (an fp32 normal
// number) and at most 57344^2, so the fp32 accumulation sees exact products.
// Rows outside that window get a NaN factor: their outputs are NaN rather than
// silently inexact.  Output in LDS (refs): bytes [0, BM) and [BM, BM + BN) the
// codes R of the A and B rows, floats at refs + 512: 2^(R - 127) or NaN.
constexpr int kMxExactSpan = 47;
constexpr int kMxRefBytes = 512 + 4 * 512 + 16 * 512;  // codes, factors, reduction scratch (up to 512 threads)

template <int BM, int BN, int NT>
__device__ __forceinline__ void mx_row_refs(const MxScales& sx, int64_t m0, int64_t M, int64_t n0, int64_t N, int K,
                                            int t, uint8_t* scratch, uint8_t* refs) {
  static_assert(BM + BN <= 512, "reference area");
  constexpr int DW = (BM + BN) / 4;  // dwords of one K block's codes for the tile (A then B)
  static_assert(NT % DW == 0, "whole blocks per pass");
  constexpr int LANES = NT / DW;     // blocks scanned side by side
  const int nb = K / 32;
  const int d = t % DW, b0 = t / DW;
  const bool is_a = d < BM / 4;
  const int64_t ld = is_a ? mx_scale_ld(M) : mx_scale_ld(N);
  const __amdgpu_buffer_rsrc_t r = operand_rsrc(is_a ? sx.a : sx.b, nb, ld);
  const int voff0 = (int)(is_a ? m0 + 4 * d : n0 + 4 * (d - BM / 4));
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mx_lo = {0, 0}, mx_hi = {0, 0}, mn_lo = {255, 255}, mn_hi = {255, 255};
  // U loads in flight per thread before any is used: each is a round trip to
  // L2 or beyond, and one at a time they dominated the tile's start.
  constexpr int U = 32;
  for (int b = b0; b < nb; b += LANES * U) {
    uint32_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bb = b + u * LANES;
      w[u] = bb < nb ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff0 + (int)(bb * ld), 0, 0) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b + u * LANES >= nb) break;
      const u16x2 lo = __builtin_bit_cast(u16x2, w[u] & 0x00FF00FFu);
      const u16x2 hi = __builtin_bit_cast(u16x2, (w[u] >> 8) & 0x00FF00FFu);
      mx_lo = __builtin_elementwise_max(mx_lo, lo);
      mx_hi = __builtin_elementwise_max(mx_hi, hi);
      mn_lo = __builtin_elementwise_min(mn_lo, lo);
      mn_hi = __builtin_elementwise_min(mn_hi, hi);
    }
  }
  // combine the LANES partial results of each dword through LDS
  static_assert(NT * 16 <= 16 * 512, "reduction scratch");
  uint32_t* part = reinterpret_cast<uint32_t*>(scratch);
  part[4 * t + 0] = __builtin_bit_cast(uint32_t, mx_lo);
  part[4 * t + 1] = __builtin_bit_cast(uint32_t, mx_hi);
  part[4 * t + 2] = __builtin_bit_cast(uint32_t, mn_lo);
  part[4 * t + 3] = __builtin_bit_cast(uint32_t, mn_hi);
  __syncthreads();
  if (t < DW) {
    uint32_t mxb[4] = {0, 0, 0, 0}, mnb[4] = {255, 255, 255, 255};
    for (int l = 0; l < LANES; ++l) {
      const uint32_t* p = part + 4 * (t + l * DW);
      const uint32_t v[4] = {p[0] & 0xFFu, p[1] & 0xFFu, p[0] >> 16, p[1] >> 16};      // max of bytes 0, 1, 2, 3
      const uint32_t u[4] = {p[2] & 0xFFu, p[3] & 0xFFu, p[2] >> 16, p[3] >> 16};      // min of bytes 0, 1, 2, 3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mxb[i] = v[i] > mxb[i] ? v[i] : mxb[i];
        mnb[i] = u[i] < mnb[i] ? u[i] : mnb[i];
      }
    }
    // byte i of the dword at tile position 4 d' holds the row whose position
    // within its 64-row group is 4 (d' % 16) + i: row (pos & ~63) | (i << 4) | (d' % 16)
    const bool a_side = t < BM / 4;
    const int dd = a_side ? t : t - BM / 4;
    const int64_t rows_valid = a_side ? M - m0 : N - n0;
    float* fac = reinterpret_cast<float*>(refs + 512);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 4 * dd + i;
      const int row = (pos & ~63) | (i << 4) | ((pos >> 2) & 15);
      const int slot = (a_side ? 0 : BM) + row;
      refs[slot] = (uint8_t)mxb[i];
      const bool ok = row >= rows_valid || (int)(mxb[i] - mnb[i]) <= kMxExactSpan;
      fac[slot] = ok ? (mxb[i] ? __builtin_bit_cast(float, mxb[i] << 23) : __builtin_bit_cast(float, 0x00400000u))
                     : __builtin_nanf("");
    }
  }
  __syncthreads();
}

// LDS transpose read (ds_read_b64_tr_b8), measured lane layout on MI355X:
// within each group of 16 lanes, lane 8h + c receives byte c of the 8-byte
// pieces addressed by lanes 2j + h, j = 0..7, as its bytes j.  So when lane
// 2j + h of a group addresses K row (r0 + j) at column c0 + 8h of a K-major
// tile, lane 8h + c gets the eight values of column c0 + 8h + c in K rows
// r0 .. r0 + 7: the K-contiguous fragment a matrix-core operand wants.
typedef int v2i_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) v2i_t lds_v2i;
  const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_v2i*)(__attribute__((address_space(3))) uint8_t*)const_cast<uint8_t*>(p));
  return make_uint2((uint32_t)r[0], (uint32_t)r[1]);
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, int MODE, bool BT = false>
__global__ __launch_bounds__(64 * WM* WN) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int M, int N, int K,
    const float* __restrict__ sinv_a, const float* __restrict__ sinv_b, void* __restrict__ C,
    int tiles_m, int tiles_n, int group_m, RequantArgs rq, MxScales mxs) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  // Output block of one matrix-core instruction: 16x16 (FP8 paths), 32x32 (bf16 paths).
  constexpr bool MX = MODE == kAccumMx;
  constexpr bool MXE = MODE == kAccumMxExact;
  constexpr bool MXS = MX || MXE;  // stages carry the step's E8M0 block scales
  constexpr int BLK = (MODE == kAccumExact || MXE) ? 32 : 16;
  constexpr int FM = WTM / BLK, FN = WTN / BLK;
  static_assert(FM >= 1 && FN >= 1 && WTM % BLK == 0 && WTN % BLK == 0, "wave tile shape");
  // A stage: the A slab, the B slab, and (MXFP8) their block scales.
  constexpr int SLABS = (BM + BN) * kBK;
  constexpr int STAGE = SLABS + (MXS ? (BM + BN) * 4 : 0);
  static_assert(STAGE % 1024 == 0, "stages keep the slabs' 1 KiB alignment");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + (MXE ? kMxRefBytes : 0)];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, &tm, &tn);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;
  const int64_t m_base = (int64_t)tm * BM, n_base = (int64_t)tn * BN;
  const int nk = (K + kBK - 1) / kBK;
  const bool ragged_k = (K % kBK) != 0;

  const SlabLoader<BM, BN, NW, BT> slabs(A, m_base, M, B, n_base, N, K, w, lane);
  static_assert(!BT || !MXS, "MXFP8 operands are K-contiguous");
  auto issue_direct = [&](uint8_t* dst, int kt, int g) {
    slabs.issue(dst, kt, g);
    if constexpr (MXS) {
      if (g == 0) MxScaleLoader<BM, BN, NW>(mxs, m_base, M, n_base, N, K, w, lane).issue(dst + SLABS, kt);
    }
  };
  auto stage_ragged = [&](int kt, int stage) { slabs.ragged(smem + stage * STAGE, kt, t); };

  // Fragment reads.  FP8 path (16x16x128): lane l takes row l & 15 of a
  // 16-row block and the 32-byte K slice l >> 4 (granules 2h, 2h+1).  bf16
  // paths (32x32x16, eight K sub-steps of 16): lane l takes row l & 31 of a
  // 32-row block and the 64-byte half l >> 5 of the K step (granules 4h..4h+3);
  // sub-step s uses bytes [8s, 8s+8) of it, for both operands alike.  Block
  // starts are multiples of 16 rows, so the swizzle of a lane's row is fixed.
  const int rr = lane & (BLK - 1), hh = lane / BLK;
  const int swz = lds_swz(rr);
  auto granule = [&](const uint8_t* tile, int row0, int g) {
    return *reinterpret_cast<const uint4*>(tile + (row0 + rr) * kBK + (((g ^ swz) & 7) << 4));
  };
  // BT: the lane's role as an address provider of the transpose read (K row
  // offset jt in 0..7, column half ht) and its 16-lane group gt.
  const int gt = lane >> 4, jt = (lane & 15) >> 1, ht = lane & 1;
  // Eight K values of the B tile (BT layout) for the fragment whose 16 columns
  // start at col0: K rows krow0 + 0..7 of this lane's column.
  auto bt_piece = [&](const uint8_t* st, int krow0, int col0) {
    return lds_read_tr8(st + BM * kBK + bt_lds_offset<BN>(krow0 + jt, col0 + 8 * ht));
  };

  uint8_t* const s0 = smem;
  uint8_t* const s1 = smem + STAGE;
  const int nfull = K / kBK;

  // Four outputs c (already x sinv_a x sinv_b) of tile row r, columns n..n+3,
  // into the staged pass (row r - r_lo).  The FP8 outputs are round_to_fp8 of
  // fp32(c x out_scale), exactly as the cast kernels encode.  The amax of the
  // unscaled c and the saturation count cover only outputs inside M x N;
  // `mask` (a std::integral_constant) is false for tiles wholly inside C,
  // which skips the bounds tests.  Saturation is |p| > max as a float
  // comparison (false for NaN, true for Inf), counted per lane and summed over
  // the wave once, when the tile is done.
  // Common case (no NaN among the four scaled values, tested through their
  // sum, which an Inf - Inf also sends down the other path): the short
  // encoder and a float maximum of |c|.  Otherwise the full rule and
  // bit-pattern maxima (NaN above Inf).
  float rq_maxf = 0.0f;
  uint32_t rq_max = 0, rq_sat_lane = 0;
  float rq_scale = 1.0f;
  if constexpr (OUT == kOutE4M3 || OUT == kOutE5M2) rq_scale = rq.out_scale[0];
  const int rows_left = (int)((M - m_base) < BM ? (M - m_base) : BM);
  const int cols_left = (int)((N - n_base) < BN ? (N - n_base) : BN);
  auto emit4 = [&](auto& tw, int r, int r_lo, int n, const v4f& c, auto mask) {
    if constexpr (OUT == kF32 || OUT == kBF16) {
      tw.put(r - r_lo, n, c);
    } else {
      constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
      constexpr float kMax = Fp8Traits<F>::max_value;
      const v4f p = c * rq_scale;
      bool ok[4] = {true, true, true, true};
      if constexpr (decltype(mask)::value) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ok[e] = r < rows_left && n + e < cols_left;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rq_sat_lane += (ok[e] && __builtin_fabsf(p[e]) > kMax) ? 1u : 0u;
      const float t = (p[0] + p[1]) + (p[2] + p[3]);
      uint32_t codes;
      if (__builtin_expect(t == t, 1)) {
        codes = encode4_finite<F>(p[0], p[1], p[2], p[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = ok[e] ? __builtin_fabsf(c[e]) : 0.0f;
          rq_maxf = a > rq_maxf ? a : rq_maxf;
        }
      } else {
        codes = encode4<F>(p[0], p[1], p[2], p[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t mb = ok[e] ? (f2u(c[e]) & 0x7FFFFFFFu) : 0u;
          rq_max = mb > rq_max ? mb : rq_max;
        }
      }
      tw.put_codes(r - r_lo, n, codes);
    }
  };

  // Stage the output tile through LDS in passes of as many rows as fit;
  // `emit(r_lo, r_hi, writer)` puts this lane's outputs of rows [r_lo, r_hi).
  auto write_tile = [&](auto&& emit) {
    using TW = TileWriter<OUT, BM, BN, NT>;
    constexpr int PASS = pass_rows<BM>(2 * STAGE, TW::ROWB);
    static_assert(PASS == BM || OUT == kF32 || OUT == kBF16, "FP8 tiles go out in one pass");
    TW tw{smem, PASS};
#pragma unroll 1
    for (int r0 = 0; r0 < BM; r0 += PASS) {
      __syncthreads();  // the LDS is free: K loop or previous pass done
      emit(r0, r0 + PASS, tw);
      __syncthreads();
      tw.flush(C, M, N, m_base + r0, n_base, t);
    }
  };
  // `rows(r_lo, r_hi, writer, mask)`: write_tile with the bounds tests of the
  // FP8 epilogue switched on only for tiles that cross the edge of C.
  uint32_t rq_seen = 0;
  auto write_tile_checked = [&](auto&& rows) {
    auto with = [&](auto mask) { write_tile([&](int r_lo, int r_hi, auto& tw) { rows(r_lo, r_hi, tw, mask); }); };
    if constexpr (OUT == kOutE4M3 || OUT == kOutE5M2) {
      if (rq.amax_bits) rq_seen = __hip_atomic_load(rq.amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rows_left == BM && cols_left == BN) with(std::false_type{});
      else with(std::true_type{});
    } else {
      with(std::false_type{});
    }
  };

  if constexpr (MODE == kAccumMfma8 || MODE == kAccumMx) {
    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    // The instruction reads lane group h's first 16 bytes as K 16h .. 16h+15 and
    // its last 16 as K 64+16h .. (measured).  Unscaled, any consistent K order
    // gives the same sum, and granules 2h, 2h+1 are used; with block scales the
    // hardware's K blocks must be the operand's, so granules h and h + 4.
    auto frag = [&](const uint8_t* tile, int row0) {
      const uint4 lo = granule(tile, row0, MX ? hh : 2 * hh), hi = granule(tile, row0, MX ? hh + 4 : 2 * hh + 1);
      return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // B fragment of 16 columns starting at col0: the same K order as `frag`
    // (lane group hh holds K 32hh .. 32hh+31 in register order), taken from the
    // BT layout as four transpose reads of 8 K rows each.
    auto frag_b = [&](const uint8_t* st, int col0) {
      if constexpr (BT) {
        v8i f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint2 p = bt_piece(st, 32 * gt + 8 * r, col0);
          f[2 * r] = (int)p.x;
          f[2 * r + 1] = (int)p.y;
        }
        return f;
      } else {
        return frag(st + BM * kBK, col0);
      }
    };
    static_assert(FN >= kDmaGroups, "one load group per leading B block");
    // A fragments of the step stay in registers; B fragments stream one
    // 16-row block ahead (bf[(j+1)&1] is read while the MFMAs of block j run).
    // MXFP8: each fragment comes with its lane's E8M0 byte (row l & 15, K block
    // l >> 4 of the step), passed to the instruction as that operand's scale.
    static_assert(!MX || (WTM % 64 == 0 && WTN % 64 == 0 && FM == 4), "MX scales: 64-row groups per wave tile");
    v8i af[FM], bf[2];
    int sca = 0, scb[FN / 4 > 0 ? FN / 4 : 1] = {};
    // The dword holding the scales of rows g64 + c + 16 i (i = 0..3, c = lane & 15)
    // of the lane's K block; fragment i selects byte i.
    auto scales4 = [&](const uint8_t* st, int area, int rows_in_area, int g64) {
      return *reinterpret_cast<const int*>(st + SLABS + area + (lane >> 4) * rows_in_area + g64 + 4 * (lane & 15));
    };
    auto load_frags = [&](const uint8_t* st) {
      bf[0] = frag_b(st, wn * WTN);
      if constexpr (MX) {
        sca = scales4(st, 0, BM, wm * WTM);
#pragma unroll
        for (int h = 0; h < FN / 4; ++h) scb[h] = scales4(st, 4 * BM, BN, wn * WTN + 64 * h);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        af[i] = frag(st, wm * WTM + i * 16);
      }
    };
    // Contract the stage at `st` (A fragments and the first B fragment already in registers).
    // The wave runs at raised priority (s_setprio) while it issues the next
    // stage's load groups with its first MFMA blocks: the two waves of a SIMD,
    // which meet at every barrier, then no longer issue in lockstep, and the
    // FC1 GEMM runs 3.4 % faster (414 against 428 us on MI355X, identical
    // output; raised for the whole step: no gain, for the first 1, 2, 3, 5 or 6
    // of the 8 blocks: 1.2-3.4 %).
    auto compute = [&](const uint8_t* st, auto&& dma) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (j == kDmaGroups) __builtin_amdgcn_s_setprio(0);
        if (j < kDmaGroups) dma(j);
        if (j + 1 < FN) {
          bf[(j + 1) & 1] = frag_b(st, wn * WTN + (j + 1) * 16);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if constexpr (MX)
            acc[i][j] = mfma_fp8_scaled<FB, FA>(bf[j & 1], af[i], acc[i][j], j & 3, scb[j >> 2], i, sca);
          else
            acc[i][j] = mfma_fp8<FB, FA>(bf[j & 1], af[i], acc[i][j]);
        }
      }
      if constexpr (FN == kDmaGroups) __builtin_amdgcn_s_setprio(0);
    };
    // Scheduling hint: per B block, its two LDS reads ahead of its MFMAs.
    auto interleave = [&]() {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM, 0);
      }
    };
    run_main_loop(s0, s1, nfull, nk, ragged_k, issue_direct, stage_ragged, load_frags, compute, interleave);

    // Lane l holds row m = l & 15 of each 16x16 block (the A operand went
    // second) and columns n = 4(l >> 4) .. +3.  MXFP8 carries its scales in
    // the instruction: no per-tensor factor.
    const float sc = MX ? 1.0f : sinv_a[0] * sinv_b[0];
    write_tile_checked([&](int r_lo, int r_hi, auto& tw, auto mask) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 16 + (lane & 15);
        if (r < r_lo || r >= r_hi) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) emit4(tw, r, r_lo, wn * WTN + j * 16 + 4 * (lane >> 4), acc[i][j] * sc, mask);
      }
    });
  } else {
    // bf16 paths: per-tensor (kAccumExact) or with block scales (kAccumMxExact)
    using H8 = v8bf;
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = (v16f){};
    uint8_t* const refs = smem + 2 * STAGE;  // kAccumMxExact: the rows' reference codes and factors
    // kAccumMxExact: the conversion factors 2^(c - R) of the lane's rows for
    // block 2 hh + h of the current step (c from the stage's scale bytes, R
    // the row's reference code).  Sub-steps 4h .. 4h + 3 lie in that block.
    // The lane's rows are 32 apart: rows i and i + 1 (i even) of a 64-row
    // group share one scale dword (bytes l >> 4 and 2 + (l >> 4), l = lane & 31),
    // so a half-step's codes take FM / 2 + FN / 2 dword reads.  The reference
    // codes do not change over the tile: kept packed, one byte per row.
    static_assert(!MXE || (FM % 2 == 0 && FN % 2 == 0 && WTM % 64 == 0 && WTN % 64 == 0), "row pairs per dword");
    float fa[FM], fb[FN];
    uint32_t ref_a = 0, ref_b = 0;
    const int sel = 8 * ((lane >> 4) & 1);
    if constexpr (MXE) {
      // the first step's slabs and scales load while the rows' references are
      // found (K is a multiple of 128 here, so step 0 is a full step)
      for (int g = 0; g < kDmaGroups; ++g) issue_direct(s0, 0, g);
      mx_row_refs<BM, BN, NT>(mxs, m_base, M, n_base, N, K, t, refs + 512 + 4 * 512, refs);
#pragma unroll
      for (int i = 0; i < FM; ++i) ref_a |= (uint32_t)refs[wm * WTM + i * 32 + (lane & 31)] << (8 * i);
#pragma unroll
      for (int j = 0; j < FN; ++j) ref_b |= (uint32_t)refs[BM + wn * WTN + j * 32 + (lane & 31)] << (8 * j);
    }
    auto codes_dword = [&](const uint8_t* st, int area, int rows_in_area, int h, int row0) {
      return *reinterpret_cast<const uint32_t*>(st + SLABS + area + (2 * hh + h) * rows_in_area + row0 +
                                                4 * (lane & 15));
    };
    auto to_factor = [&](uint32_t code, uint32_t ref) {
      return __builtin_bit_cast(float, (code - ref + 127u) << 23);
    };
    auto load_fa = [&](const uint8_t* st, int h) {
#pragma unroll
      for (int i = 0; i < FM; i += 2) {
        const uint32_t d = codes_dword(st, 0, BM, h, wm * WTM + i * 32);
        fa[i] = to_factor((d >> sel) & 0xFFu, (ref_a >> (8 * i)) & 0xFFu);
        fa[i + 1] = to_factor((d >> (sel + 16)) & 0xFFu, (ref_a >> (8 * i + 8)) & 0xFFu);
      }
    };
    auto load_fb = [&](const uint8_t* st, int h) {
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
        const uint32_t d = codes_dword(st, 4 * BM, BN, h, wn * WTN + j * 32);
        fb[j] = to_factor((d >> sel) & 0xFFu, (ref_b >> (8 * j)) & 0xFFu);
        fb[j + 1] = to_factor((d >> (sel + 16)) & 0xFFu, (ref_b >> (8 * j + 8)) & 0xFFu);
      }
    };
    auto widen_a = [&](uint32_t w0, uint32_t w1, int i) -> H8 {
      return widen8_scaled_bf16<FA>(w0, w1, MXE ? fa[i] : 1.0f);
    };
    auto widen_b = [&](uint32_t w0, uint32_t w1, int j) -> H8 {
      return widen8_scaled_bf16<FB>(w0, w1, MXE ? fb[j] : 1.0f);
    };
    auto mfma = [&](const H8& b, const H8& a, const v16f& c) {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
    };
    // Raw FP8 fragments of the whole step: 4 granules (64 bytes) per block.
    // Only granule 0 is read right after the barrier; granule c + 1 is read
    // while the MFMAs of granule c run (sub-steps 2c, 2c + 1), so the four
    // waves' LDS reads no longer arrive as one burst that every wave's first
    // MFMA waits behind (1-3 % faster on FC1, identical results).
    // BT: the B pieces of sub-steps 2c and 2c + 1 come from two transpose reads
    // (K rows 64 hh + 8s + 0..7 of the lane's column, hh = gt >> 1; lanes
    // 16 (gt & 1) + 0..15 of each half cover the block's 32 columns).
    uint4 ar[FM][4], br[FN][4];
    auto read_granule = [&](const uint8_t* st, int c) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BT) {
          const int col0 = wn * WTN + j * 32 + 16 * (gt & 1);
          const uint2 p0 = bt_piece(st, 64 * (gt >> 1) + 16 * c, col0);
          const uint2 p1 = bt_piece(st, 64 * (gt >> 1) + 16 * c + 8, col0);
          br[j][c] = make_uint4(p0.x, p0.y, p1.x, p1.y);
        } else {
          br[j][c] = granule(st + BM * kBK, wn * WTN + j * 32, 4 * hh + c);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) ar[i][c] = granule(st, wm * WTM + i * 32, 4 * hh + c);
    };
    auto load_frags = [&](const uint8_t* st) { read_granule(st, 0); };
    // The wave issues in order, so conversions written after a sub-step's
    // MFMAs wait until the last of them has issued: with all 32 conversions of
    // a sub-step ahead of its 16 MFMAs the matrix core idled while the next
    // sub-step was being converted.  Here the B operands are converted one
    // sub-step ahead, and the scheduling groups place two conversions (the
    // remaining A blocks', then the next sub-step's B blocks') after each
    // MFMA, inside its shadow (2-3 % faster on FC1, identical results).
    auto cvt_b = [&](int s, H8* out) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 g = br[j][s >> 1];
        out[j] = (s & 1) ? widen_b(g.z, g.w, j) : widen_b(g.x, g.y, j);
      }
    };
    auto compute = [&](const uint8_t* st, auto&& dma) {
      H8 bb[2][FN];
      if constexpr (MXE) {
        load_fa(st, 0);
        load_fb(st, 0);
      }
      cvt_b(0, bb[0]);
      // Raised wave priority for the first six sub-steps: with two waves per
      // SIMD (8-wave tiles), one of them is favoured while both leave the
      // step's barrier, so they stop issuing in lockstep.  FC1 on MI355X,
      // identical output: 8 waves of 128x64 with this window 716.8 us, against
      // 733.4 us for 4 waves of 128x128; windows of 5 or 7 sub-steps 720.3 and
      // 721.4 us.  A lone wave per SIMD is unaffected.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s == 6) __builtin_amdgcn_s_setprio(0);
        if (s < kDmaGroups) dma(s);
        if ((s & 1) == 0 && (s >> 1) + 1 < 4) {
          read_granule(st, (s >> 1) + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        const H8* bh = bb[s & 1];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const uint4 g = ar[i][s >> 1];
          const H8 ah = (s & 1) ? widen_a(g.z, g.w, i) : widen_a(g.x, g.y, i);
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma(bh[j], ah, acc[i][j]);
        }
        if constexpr (MXE) {
          // the second block's factors: after the last use of the first's
          // (sub-step 3's A conversions), before cvt_b(4); the LDS reads are
          // free to move up over this sub-step's MFMAs
          if (s == 3) {
            load_fa(st, 1);
            load_fb(st, 1);
          }
        }
        if (s + 1 < 8) cvt_b(s + 1, bb[(s + 1) & 1]);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
#pragma unroll
        for (int k = 0; k < FM * FN; ++k) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto interleave = [&]() {};
    run_main_loop(s0, s1, nfull, nk, ragged_k, issue_direct, stage_ragged, load_frags, compute, interleave, MXE);

    // Lane l holds row m = l & 31 of each 32x32 block (the A operand went
    // second) and columns n = 8g + 4(l >> 5) + 0..3 in registers 4g..4g+3.
    // kAccumMxExact: the result is acc * 2^(R_a - 127) * 2^(R_b - 127), in
    // that order (each step exact unless the result leaves fp32's range).
    const float sc = MXE ? 1.0f : sinv_a[0] * sinv_b[0];
    const float* fac = reinterpret_cast<const float*>(refs + 512);
    write_tile_checked([&](int r_lo, int r_hi, auto& tw, auto mask) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + (lane & 31);
        if (r < r_lo || r >= r_hi) continue;
        const float fr = MXE ? fac[r] : sc;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
            const v4f v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            if constexpr (MXE) {
              const v4f fc = *reinterpret_cast<const v4f*>(fac + BM + n);
              emit4(tw, r, r_lo, n, (v * fr) * fc, mask);
            } else {
              emit4(tw, r, r_lo, n, v * sc, mask);
            }
          }
      }
    });
  }
  if constexpr (OUT == kOutE4M3 || OUT == kOutE5M2) {
    // |c| of the common path as bits (non-negative floats order as their bit patterns)
    const uint32_t mf = f2u(rq_maxf);
    publish_requant_stats(mf > rq_max ? mf : rq_max, wave_sum_u32(rq_sat_lane), rq_seen, rq, lane);
  }
}

}  // namespace fp8mi
