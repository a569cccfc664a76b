// Fused amax + scaled saturating FP8 cast (optionally with a transposed copy),
// and per-block current-scaling quantisation.
//
// "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the FP8 tensor is
// round_to_fp8(tensor × scale) with scale ≈ FP8_MAX / amax; delayed scaling
// lets the cast use a scale known before the pass, so this step's amax and
// the cast come out of ONE read of the tensor.  "FP8 and low-precision
// formats", "Deep dive": scale factors are per tensor or per block.
//
// The per-tensor kernels are HBM-bound: per element they read 2 B (bf16) or
// 4 B (fp32) and write 1 B (2 B with both layouts).  Every wave instruction
// moves one contiguous 1 KiB of input (16 B per lane).  Per element the work
// is: widen, multiply by the scale, half a packed conversion, and an integer
// max of |bits| for amax (exact and order-free).  The clamp (V_MED3_F32), the
// saturation count and the NaN rule only change codes whose scaled value
// exceeds max or is NaN, so the flat cast applies them only to wave chunks
// whose largest |x| times the scale exceeds max (or is NaN); NaN codes are
// fixed on a separate path taken only when a NaN is present.  amax is reduced
// across the wavefront with shuffles, across the workgroup in LDS, and across
// workgroups through per-workgroup partials (or one atomicMax per workgroup
// without a workspace); the saturation count is a wave ballot + popcount.
#include <atomic>
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__global__ void zero_outputs_kernel(uint32_t* amax_bits, unsigned long long* sat) {
  if (threadIdx.x == 0) {
    if (amax_bits) *amax_bits = 0u;
    if (sat) *sat = 0ull;
  }
}

// Fold (per-lane amax bits, per-wave saturation count) into the global outputs:
// either one partial per workgroup (`partials` non-null: slot blockIdx.x gets
// {amax bits, 0, count lo, count hi}, reduced afterwards by
// reduce_partials_kernel) or device-scope atomics on the outputs.  The atomics
// on one address are serialised across the chip (about 4 ns each on MI355X,
// ~4 us for a 512-workgroup grid); the partials cost one tiny extra kernel.
__device__ __forceinline__ void block_finish(uint32_t amx, uint32_t wave_cnt, uint32_t* amax_bits,
                                             unsigned long long* sat, uint4* partials) {
  __shared__ uint32_t s_max[kWaves];
  __shared__ uint32_t s_cnt[kWaves];
  amx = wave_max_u32(amx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_max[wave] = amx;
    s_cnt[wave] = wave_cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_max[0];
    unsigned long long c = s_cnt[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      m = m > s_max[w] ? m : s_max[w];
      c += s_cnt[w];
    }
    if (partials) {
      partials[blockIdx.x] = make_uint4(m, 0u, (uint32_t)c, (uint32_t)(c >> 32));
    } else {
      if (amax_bits) atomicMax(amax_bits, m);
      if (sat && c) atomicAdd(sat, c);
    }
  }
}

// Reduce `count` workgroup partials into the outputs (one workgroup) and,
// when `hs.history` is set, run the delayed-scaling history step on the
// reduced amax in the same launch (the rule of amax_update.hip: push it into
// the ring at *head, advance the head, scale = MAX / max(ring) when that max
// is finite and non-zero, else hold the scale and set status bit 0; a head
// outside [0, len) is treated as 0 and sets status bit 1).  The ring, the
// head and the old inverse scale do not depend on the partials, so they are
// loaded first and their latency overlaps the partials' loads; the ring's
// max (without the slot being replaced) rides in the same reduction.
__global__ __launch_bounds__(kThreads) void reduce_partials_kernel(const uint4* __restrict__ partials, int count,
                                                                  uint32_t* __restrict__ amax_bits,
                                                                  unsigned long long* __restrict__ sat,
                                                                  HistoryArgs hs) {
  __shared__ uint32_t s_max[kWaves];
  __shared__ uint32_t s_hmax[kWaves];
  __shared__ unsigned long long s_cnt[kWaves];
  int h = 0, flags = 0;
  uint32_t hm = 0u;
  float sinv_old = 0.0f;
  if (hs.history) {  // uniform
    h = *hs.head;
    if (h < 0 || h >= hs.len) {
      h = 0;
      flags |= 2;
    }
    for (int i = threadIdx.x; i < hs.len; i += kThreads) {
      const uint32_t b = f2u(hs.history[i]) & 0x7FFFFFFFu;  // loaded whatever h is; slot h dropped below
      const uint32_t bb = (i == h) ? 0u : b;
      hm = hm > bb ? hm : bb;
    }
    if (threadIdx.x == 0 && hs.sinv_used) sinv_old = *hs.scale_inv;
  }
  // Up to eight partials per thread, all loads issued before any is used:
  // they were just written by workgroups on every XCD, so each one is a
  // round trip past the local L2, and a loop that waited for each load in
  // turn paid those round trips one after another.  Slots past `count` read
  // as zero, which changes neither the maximum nor the sum.
  constexpr int kPer = 8;
  uint32_t m = 0u;
  unsigned long long c = 0ull;
  for (int base = threadIdx.x; base < count; base += kThreads * kPer) {
    uint4 p[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = base + u * kThreads;
      p[u] = i < count ? partials[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      m = m > p[u].x ? m : p[u].x;
      c += (unsigned long long)p[u].z | ((unsigned long long)p[u].w << 32);
    }
  }
  m = wave_max_u32(m);
  hm = wave_max_u32(hm);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_max[wave] = m;
    s_hmax[wave] = hm;
    s_cnt[wave] = c;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // Thread 0 holds wave 0's totals.
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    m = m > s_max[w] ? m : s_max[w];
    hm = hm > s_hmax[w] ? hm : s_hmax[w];
    c += s_cnt[w];
  }
  if (amax_bits) *amax_bits = m;
  if (sat) *sat = c;
  if (!hs.history) return;
  hm = hm > m ? hm : m;  // the ring after the push
  if (hs.sinv_used) *hs.sinv_used = sinv_old;
  hs.history[h] = u2f(m);
  *hs.head = (h + 1 == hs.len) ? 0 : h + 1;
  float sc, si;
  const bool ok = hs.fmt == kE4M3 ? scale_from_amax_bits<kE4M3>(hm, &sc, &si) : scale_from_amax_bits<kE5M2>(hm, &sc, &si);
  if (ok) {
    *hs.scale = sc;
    *hs.scale_inv = si;
  } else {
    flags |= 1;
  }
  if (hs.status && flags) *hs.status |= flags;
}

// One fp32 value copied on the device (stream-ordered, capturable).
__global__ void copy_scalar_kernel(const float* __restrict__ src, float* __restrict__ dst) {
  if (threadIdx.x == 0) *dst = *src;
}

// With a finite non-zero scale, x * s is NaN exactly where x is NaN.
__device__ __forceinline__ bool scale_is_regular(float s) {
  const uint32_t m = f2u(s) & 0x7FFFFFFFu;
  return m != 0u && m < 0x7F800000u;
}

// One 16-B input vector: 8 bf16 or 4 fp32 elements.
template <int XT>
struct Vec {
  static constexpr int EPV = XT == kBF16 ? 8 : 4;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16-B load; NT marks it nontemporal (streamed data that is read once: on
// MI355X the flat cast ran 9 % faster with its loads and stores marked so).
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* __restrict__ x, int64_t vi) {
  if constexpr (NT) {
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + vi);
    return make_uint4(r[0], r[1], r[2], r[3]);
  } else {
    return reinterpret_cast<const uint4*>(x)[vi];
  }
}

// Nontemporal code stores (8 B or 4 B per lane).
__device__ __forceinline__ void store_nt(uint8_t* __restrict__ q, int64_t vi, uint32_t c0, uint32_t c1) {
  u32x2 r;
  r[0] = c0;
  r[1] = c1;
  __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(q) + vi);
}
__device__ __forceinline__ void store_nt(uint8_t* __restrict__ q, int64_t vi, uint32_t c0) {
  __builtin_nontemporal_store(c0, reinterpret_cast<uint32_t*>(q) + vi);
}

// A 16-B input vector as fp32 values (exact widening of bf16).
template <int XT>
__device__ __forceinline__ void widen_vec(const uint4& a, float* v) {
  if constexpr (XT == kBF16) {
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  } else {
    v[0] = u2f(a.x); v[1] = u2f(a.y); v[2] = u2f(a.z); v[3] = u2f(a.w);
  }
}

// The largest magnitude bit pattern of a 16-B input vector, as fp32 bits.
template <int XT>
__device__ __forceinline__ uint32_t vec_max_bits(const uint4& a) {
  if constexpr (XT == kBF16) {
    const us2 m0 = __builtin_bit_cast(us2, a.x & 0x7FFF7FFFu), m1 = __builtin_bit_cast(us2, a.y & 0x7FFF7FFFu);
    const us2 m2 = __builtin_bit_cast(us2, a.z & 0x7FFF7FFFu), m3 = __builtin_bit_cast(us2, a.w & 0x7FFF7FFFu);
    const us2 m = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1), __builtin_elementwise_max(m2, m3));
    return (uint32_t)(m[0] > m[1] ? m[0] : m[1]) << 16;
  } else {
    const uint32_t m01 = (a.x & 0x7FFFFFFFu) > (a.y & 0x7FFFFFFFu) ? (a.x & 0x7FFFFFFFu) : (a.y & 0x7FFFFFFFu);
    const uint32_t m23 = (a.z & 0x7FFFFFFFu) > (a.w & 0x7FFFFFFFu) ? (a.z & 0x7FFFFFFFu) : (a.w & 0x7FFFFFFFu);
    return m01 > m23 ? m01 : m23;
  }
}

// Load vector `vi` as fp32 values and the max of its magnitude bit patterns.
template <int XT, bool NT = false>
__device__ __forceinline__ void load_vec(const void* __restrict__ x, int64_t vi, float* v, uint32_t& vmax) {
  const uint4 a = load16<NT>(x, vi);
  widen_vec<XT>(a, v);
  vmax = vec_max_bits<XT>(a);
}

template <int XT>
__device__ __forceinline__ float load1(const void* __restrict__ x, int64_t elem) {
  if constexpr (XT == kBF16)
    return u2f((uint32_t)reinterpret_cast<const uint16_t*>(x)[elem] << 16);
  else
    return reinterpret_cast<const float*>(x)[elem];
}

// Scale and encode 4 values; `finite` = no NaN can appear in the products.
// When SAT, adds the wave's count of |p| > max (NaN never counts) to wave_cnt.
template <int FMT, bool SAT>
__device__ __forceinline__ uint32_t scale_encode4(const float* v, float s, bool finite, uint32_t& wave_cnt) {
  const float p0 = v[0] * s, p1 = v[1] * s, p2 = v[2] * s, p3 = v[3] * s;
  if constexpr (SAT) {
    constexpr float mx = Fp8Traits<FMT>::max_value;
    wave_cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(p0) > mx)) +
                __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(p1) > mx)) +
                __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(p2) > mx)) +
                __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(p3) > mx));
  }
  if (__builtin_expect(finite, 1)) return encode4_finite<FMT>(p0, p1, p2, p3);
  return encode4<FMT>(p0, p1, p2, p3);
}

// Scale and encode 4 values known to give products of magnitude <= max (so
// no clamp, no NaN, nothing saturates): on such values the conversion
// instruction alone is the encoding rule.
template <int FMT>
__device__ __forceinline__ uint32_t scale_encode4_inrange(const float* v, float s) {
  const uint32_t w = cvt_pk<FMT, false>(v[0] * s, v[1] * s, 0u);
  return cvt_pk<FMT, true>(v[2] * s, v[3] * s, w);
}

// True when fp32(|x| * s) <= max for the largest magnitude `m_bits` of a
// chunk: rounding is monotone, so it then holds for every element of the
// chunk.  False when m_bits is NaN or s is NaN (the comparison fails).
template <int FMT>
__device__ __forceinline__ bool chunk_in_range(uint32_t m_bits, float s) {
  return __builtin_fabsf(u2f(m_bits) * s) <= Fp8Traits<FMT>::max_value;
}

// ---------------------------------------------------------------------------
// Flat kernel: q (row-major) and/or amax.  Each lane casts U vectors; vector u
// of a wave covers one contiguous 1 KiB (64 lanes x 16 B).
// ---------------------------------------------------------------------------
constexpr int kVecPerLane = 4;

template <int XT, int FMT, bool WQ, bool SAT>
__global__ __launch_bounds__(kThreads) void quantize_flat_kernel(
    const void* __restrict__ x, int64_t n, const float* __restrict__ scale, uint8_t* __restrict__ q,
    uint32_t* __restrict__ amax_bits, unsigned long long* __restrict__ sat, uint4* __restrict__ partials) {
  constexpr int EPV = Vec<XT>::EPV, U = kVecPerLane;
  const float s = (WQ || SAT) ? *scale : 1.0f;
  const bool regular = scale_is_regular(s);
  const int64_t nvec = n / EPV;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t amx = 0u, wcnt = 0u;
  float v[U][EPV];
  uint32_t vm[U];
  auto cast_store = [&](int u, int64_t vi) {
    amx = amx > vm[u] ? amx : vm[u];
    if constexpr (WQ || SAT) {
      const bool finite = regular && vm[u] <= 0x7F800000u;
      const uint32_t c0 = scale_encode4<FMT, SAT>(&v[u][0], s, finite, wcnt);
      if constexpr (EPV == 8) {
        const uint32_t c1 = scale_encode4<FMT, SAT>(&v[u][4], s, finite, wcnt);
        if constexpr (WQ) store_nt(q, vi, c0, c1);
      } else {
        if constexpr (WQ) store_nt(q, vi, c0);
      }
    }
  };
  // Grid-stride over wave chunks of 64*U vectors: a persistent grid of a few
  // workgroups per CU keeps the number of cross-workgroup partials small.
  const int64_t wave_stride = (int64_t)gridDim.x * kWaves * (64 * U);
  for (int64_t wave_base = ((int64_t)blockIdx.x * kWaves + wave) * (64 * U); wave_base < nvec;
       wave_base += wave_stride) {
    if (wave_base + U * 64 <= nvec) {
      // Whole chunk in range: every load issued before any use.
#pragma unroll
      for (int u = 0; u < U; ++u) load_vec<XT, true>(x, wave_base + u * 64 + lane, v[u], vm[u]);
      if constexpr (WQ || SAT) {
        // When no product of the wave's chunk can exceed max (the common
        // case), the clamp, the saturation count and the NaN rule are no-ops.
        uint32_t cm = vm[0];
#pragma unroll
        for (int u = 1; u < U; ++u) cm = cm > vm[u] ? cm : vm[u];
        if (__builtin_amdgcn_ballot_w64(!chunk_in_range<FMT>(cm, s)) == 0) {
          amx = amx > cm ? amx : cm;
          if constexpr (WQ) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const int64_t vi = wave_base + u * 64 + lane;
              const uint32_t c0 = scale_encode4_inrange<FMT>(&v[u][0], s);
              if constexpr (EPV == 8)
                store_nt(q, vi, c0, scale_encode4_inrange<FMT>(&v[u][4], s));
              else
                store_nt(q, vi, c0);
            }
          }
          continue;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) cast_store(u, wave_base + u * 64 + lane);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t vi = wave_base + u * 64 + lane;
        vm[u] = 0u;
        if (vi < nvec) load_vec<XT>(x, vi, v[u], vm[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t vi = wave_base + u * 64 + lane;
        if (vi < nvec) cast_store(u, vi);
      }
    }
  }
  // Ragged tail (n % EPV elements), element by element, in workgroup 0.
  const int rem = (int)(n - nvec * EPV);
  if (blockIdx.x == 0 && (int)threadIdx.x < rem) {
    const int64_t i = nvec * EPV + threadIdx.x;
    const float xv = load1<XT>(x, i);
    const uint32_t m = f2u(xv) & 0x7FFFFFFFu;
    amx = amx > m ? amx : m;
    const float p = xv * s;
    if constexpr (SAT) {
      wcnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(p) > Fp8Traits<FMT>::max_value));
    }
    if constexpr (WQ) q[i] = encode1<FMT>(p);
  }
  block_finish(amx, wcnt, amax_bits, sat, partials);
}

// ---------------------------------------------------------------------------
// Cast-transpose kernel: one 128x128 input tile per workgroup; writes q_t (and
// q when asked).  Phase 1 casts the tile and writes the codes row-major into
// LDS (row pitch 132 B); phase 2 gives each lane 4 columns x 16 rows: 16 LDS
// words, a 4x4 byte transpose per 4 rows with V_PERM_B32, and four 16-B
// stores into 4 rows of q_t (eight lanes cover 128 contiguous bytes of one
// q_t row).  Requires rows % 16 == 0 and cols % 16 == 0.
// ---------------------------------------------------------------------------
constexpr int kTile = 128;
constexpr int kPitch = 132;

__device__ __forceinline__ void transpose4x4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t& c0,
                                             uint32_t& c1, uint32_t& c2, uint32_t& c3) {
  // w_r holds columns 0..3 of row r (byte k = column k); c_k gets rows 0..3 of column k.
  const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);  // w2.b0 w3.b0 w2.b1 w3.b1
  const uint32_t t2 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);  // w2.b2 w3.b2 w2.b3 w3.b3
  c0 = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
  c1 = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
  c2 = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
  c3 = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

template <int XT, int FMT, bool WQ, bool SAT>
__global__ __launch_bounds__(kThreads) void quantize_transpose_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, const float* __restrict__ scale,
    uint8_t* __restrict__ q, uint8_t* __restrict__ q_t, uint32_t* __restrict__ amax_bits,
    unsigned long long* __restrict__ sat, uint4* __restrict__ partials) {
  constexpr int EPV = Vec<XT>::EPV;
  constexpr int VPR = kTile / EPV;          // vectors per tile row
  constexpr int RPP = kThreads / VPR;       // tile rows per pass
  constexpr int PASSES = kTile / RPP;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kPitch];
  const float s = *scale;
  const bool regular = scale_is_regular(s);
  const int t = threadIdx.x;
  const int vi = t % VPR, rr0 = t / VPR;
  const int64_t vecs_per_row = cols / EPV;
  const int64_t tiles_c = (cols + kTile - 1) / kTile, tiles = tiles_c * ((rows + kTile - 1) / kTile);
  uint32_t amx = 0u, wcnt = 0u;
  // Persistent grid: each workgroup walks tiles blockIdx.x, +gridDim.x, ...
  for (int64_t tile_id = blockIdx.x; tile_id < tiles; tile_id += gridDim.x) {
  const int64_t row0 = (tile_id / tiles_c) * kTile, col0 = (tile_id % tiles_c) * kTile;
  // Raw 16-B vectors (widened one pass at a time, which keeps the register
  // footprint, and with it the occupancy, down) and their magnitude maxima.
  uint4 raw[PASSES];
  uint32_t vm[PASSES];
  auto cast_pass = [&](int i, bool in_range) {
    const int rr = rr0 + i * RPP;
    const int64_t r = row0 + rr, c = col0 + vi * EPV;
    float v[EPV];
    widen_vec<XT>(raw[i], v);
    uint32_t c0, c1 = 0u;
    if (in_range) {
      c0 = scale_encode4_inrange<FMT>(&v[0], s);
      if constexpr (EPV == 8) c1 = scale_encode4_inrange<FMT>(&v[4], s);
    } else {
      const bool finite = regular && vm[i] <= 0x7F800000u;
      c0 = scale_encode4<FMT, SAT>(&v[0], s, finite, wcnt);
      if constexpr (EPV == 8) c1 = scale_encode4<FMT, SAT>(&v[4], s, finite, wcnt);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + rr * kPitch + vi * EPV);
    dst[0] = c0;
    if constexpr (EPV == 8) {
      dst[1] = c1;
      if constexpr (WQ) *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(c0, c1);
    } else {
      if constexpr (WQ) *reinterpret_cast<uint32_t*>(q + r * cols + c) = c0;
    }
  };
  if (row0 + kTile <= rows && col0 + kTile <= cols) {
    // Interior tile: every load issued before any use; when no product of the
    // wave's part of the tile can exceed max, the clamp, the count and the NaN
    // rule are no-ops (as in the flat cast).
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      raw[i] = load16<false>(x, (row0 + rr0 + i * RPP) * vecs_per_row + (col0 + vi * EPV) / EPV);
    uint32_t cm = 0u;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      vm[i] = vec_max_bits<XT>(raw[i]);
      cm = cm > vm[i] ? cm : vm[i];
    }
    amx = amx > cm ? amx : cm;
    const bool in_range = __builtin_amdgcn_ballot_w64(!chunk_in_range<FMT>(cm, s)) == 0;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) cast_pass(i, in_range);
  } else {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int64_t r = row0 + rr0 + i * RPP, c = col0 + vi * EPV;
      raw[i] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows && c < cols) raw[i] = load16<false>(x, r * vecs_per_row + c / EPV);
      vm[i] = vec_max_bits<XT>(raw[i]);
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int64_t r = row0 + rr0 + i * RPP, c = col0 + vi * EPV;
      if (r < rows && c < cols) {
        amx = amx > vm[i] ? amx : vm[i];
        cast_pass(i, false);
      }
    }
  }
  __syncthreads();
  {
    const int rg = t & 7, cq = t >> 3;
    const int64_t c = col0 + cq * 4, r = row0 + rg * 16;
    if (c < cols && r < rows) {
      uint32_t w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = *reinterpret_cast<const uint32_t*>(tile + (rg * 16 + j) * kPitch + cq * 4);
      uint32_t o[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        transpose4x4(w[4 * b], w[4 * b + 1], w[4 * b + 2], w[4 * b + 3], o[b][0], o[b][1], o[b][2], o[b][3]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<uint4*>(q_t + (c + k) * rows + r) = make_uint4(o[0][k], o[1][k], o[2][k], o[3][k]);
    }
  }
  __syncthreads();  // the LDS tile is rewritten by the next iteration
  }
  block_finish(amx, wcnt, amax_bits, sat, partials);
}

// ---------------------------------------------------------------------------
// Per-block current scaling.
// ---------------------------------------------------------------------------
// Load 8 consecutive elements (one or two 16-B vectors) and their magnitude max.
template <int XT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t elem, float v[8], uint32_t& vmax) {
  if constexpr (XT == kBF16) {
    load_vec<XT>(x, elem / 8, v, vmax);
  } else {
    uint32_t m1;
    load_vec<XT>(x, elem / 4, v, vmax);
    load_vec<XT>(x, elem / 4 + 1, v + 4, m1);
    vmax = vmax > m1 ? vmax : m1;
  }
}

// 1 x 128 tiles: 16 lanes per tile, 8 elements per lane.
template <int XT, int FMT>
__global__ __launch_bounds__(kThreads) void quantize_rowtile_kernel(const void* __restrict__ x,
                                                                    int64_t rows, int64_t cols,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale_inv) {
  const int64_t ntc = (cols + 127) / 128;
  const int64_t ntiles = rows * ntc;
  const int sub = threadIdx.x & 15;
  const int64_t groups = (int64_t)gridDim.x * (kThreads / 16);
  for (int64_t tile = (int64_t)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4); tile < ntiles;
       tile += groups) {
    // All 16 lanes of a group share `tile`, so the trip count is uniform per
    // group and the shuffles below (xor offsets < 16) stay inside the group.
    const int64_t r = tile / ntc, tc = tile - r * ntc;
    const int64_t c = tc * 128 + sub * 8;
    const bool valid = c < cols;
    float v[8];
    uint32_t m = 0u;
    if (valid) load8<XT>(x, r * cols + c, v, m);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
      m = m > o ? m : o;
    }
    float s = 1.0f, si = 1.0f;
    scale_from_amax_bits<FMT>(m, &s, &si);
    if (valid) {
      const bool finite = m <= 0x7F800000u;
      uint32_t unused = 0u;
      const uint32_t c0 = scale_encode4<FMT, false>(&v[0], s, finite, unused);
      const uint32_t c1 = scale_encode4<FMT, false>(&v[4], s, finite, unused);
      *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(c0, c1);
    }
    if (sub == 0) scale_inv[tile] = si;
  }
}

// 128 x 128 blocks: one workgroup per block, 64 elements per thread held in
// registers as the raw 16-B input vectors and widened row by row when they are
// encoded.  Held as fp32 values they took 100 registers (five waves per SIMD);
// raw, bf16 input takes half as many, so more blocks are in flight per CU.
template <int XT, int FMT>
__global__ __launch_bounds__(kThreads) void quantize_block128_kernel(const void* __restrict__ x,
                                                                     int64_t rows, int64_t cols,
                                                                     uint8_t* __restrict__ q,
                                                                     float* __restrict__ scale_inv) {
  __shared__ uint32_t s_max[kWaves];
  constexpr int NV = XT == kBF16 ? 1 : 2;  // 16-B vectors per 8 elements
  const int64_t row0 = (int64_t)blockIdx.y * 128, col0 = (int64_t)blockIdx.x * 128;
  const int t = threadIdx.x;
  const int64_t c = col0 + (t & 15) * 8;
  uint4 raw[8][NV];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 16 + (t >> 4);
#pragma unroll
    for (int h = 0; h < NV; ++h) {
      raw[i][h] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows && c < cols) raw[i][h] = load16<false>(x, (r * cols + c) / (8 / NV) + h);
      const uint32_t vm = vec_max_bits<XT>(raw[i][h]);
      m = m > vm ? m : vm;
    }
  }
  m = wave_max_u32(m);
  if ((t & 63) == 0) s_max[t >> 6] = m;
  __syncthreads();
  m = s_max[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = m > s_max[w] ? m : s_max[w];
  float s = 1.0f, si = 1.0f;
  scale_from_amax_bits<FMT>(m, &s, &si);
  const bool finite = m <= 0x7F800000u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 16 + (t >> 4);
    if (r < rows && c < cols) {
      float v[8];
#pragma unroll
      for (int h = 0; h < NV; ++h) widen_vec<XT>(raw[i][h], v + 4 * h);
      uint32_t unused = 0u;
      const uint32_t c0 = scale_encode4<FMT, false>(&v[0], s, finite, unused);
      const uint32_t c1 = scale_encode4<FMT, false>(&v[4], s, finite, unused);
      *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(c0, c1);
    }
  }
  if (t == 0) scale_inv[blockIdx.y * gridDim.x + blockIdx.x] = si;
}

// ---------------------------------------------------------------------------
// Launch helpers (template dispatch).
// ---------------------------------------------------------------------------
}  // namespace

// Workgroups of a persistent cast grid: `per_cu` per compute unit.  With
// workspace partials each workgroup costs one 16-B slot.  Without them each
// workgroup ends with device-scope atomics on single words, serialised across
// the chip (about 10 ns each on MI355X), so that path keeps two per CU.
int persistent_groups(int per_cu) {
  // Compute units per device, queried once per device (relaxed atomics: every
  // thread that races here stores the same value).
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * per_cu;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus * per_cu;
}

namespace {

// Workgroups of a cast grid with `partials` slots available (0: no partials,
// atomics path).  The flat cast streams at the same rate with 2 or 4
// workgroups per CU; the cast-transpose, which alternates a load phase and
// an LDS/store phase per tile, runs 13 % faster with 8 (measured on MI355X).
int cast_groups(int64_t units, int64_t per_group, int64_t slots, int per_cu = 2) {
  int64_t g = (units + per_group - 1) / per_group;
  const int cap = persistent_groups(slots > 0 ? per_cu : 2);
  if (g > cap) g = cap;
  if (slots > 0 && g > slots) g = slots;
  return g < 1 ? 1 : (int)g;
}

template <int XT, int FMT, bool WQ, bool SAT>
int launch_flat_t(const void* x, int64_t n, const float* scale, uint8_t* q, uint32_t* amax_bits,
                  unsigned long long* sat, uint4* partials, int64_t slots, hipStream_t st) {
  constexpr int EPV = Vec<XT>::EPV;
  const int g = cast_groups(n / EPV, (int64_t)kThreads * kVecPerLane, partials ? slots : 0);
  hipLaunchKernelGGL((quantize_flat_kernel<XT, FMT, WQ, SAT>), dim3((unsigned)g), dim3(kThreads), 0, st, x, n,
                     scale, q, amax_bits, sat, partials);
  return g;
}

template <int XT, int FMT>
int launch_flat_f(const void* x, int64_t n, const float* scale, uint8_t* q, uint32_t* amax_bits,
                  unsigned long long* sat, uint4* partials, int64_t slots, hipStream_t st) {
  if (q && sat) return launch_flat_t<XT, FMT, true, true>(x, n, scale, q, amax_bits, sat, partials, slots, st);
  if (q) return launch_flat_t<XT, FMT, true, false>(x, n, scale, q, amax_bits, sat, partials, slots, st);
  if (sat) return launch_flat_t<XT, FMT, false, true>(x, n, scale, q, amax_bits, sat, partials, slots, st);
  return launch_flat_t<XT, FMT, false, false>(x, n, scale, q, amax_bits, sat, partials, slots, st);
}

template <int XT, int FMT>
int launch_transpose_f(const void* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q, uint8_t* q_t,
                       uint32_t* amax_bits, unsigned long long* sat, uint4* partials, int64_t slots,
                       hipStream_t st) {
  const int64_t tiles = ((cols + kTile - 1) / kTile) * ((rows + kTile - 1) / kTile);
  const dim3 grid((unsigned)cast_groups(tiles, 1, partials ? slots : 0, 8));
  if (q && sat)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, true, true>), grid, dim3(kThreads), 0, st,
                       x, rows, cols, scale, q, q_t, amax_bits, sat, partials);
  else if (q)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, true, false>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat, partials);
  else if (sat)
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, false, true>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat, partials);
  else
    hipLaunchKernelGGL((quantize_transpose_kernel<XT, FMT, false, false>), grid, dim3(kThreads), 0,
                       st, x, rows, cols, scale, q, q_t, amax_bits, sat, partials);
  return (int)grid.x;
}

template <int XT>
int launch_quantize_x(const void* x, int64_t rows, int64_t cols, int fmt, const float* scale, uint8_t* q,
                      uint8_t* q_t, uint32_t* amax_bits, unsigned long long* sat, uint4* partials, int64_t slots,
                      hipStream_t st) {
  const int64_t n = rows * cols;
  if (q_t) {
    if (fmt == kE4M3) return launch_transpose_f<XT, kE4M3>(x, rows, cols, scale, q, q_t, amax_bits, sat, partials, slots, st);
    return launch_transpose_f<XT, kE5M2>(x, rows, cols, scale, q, q_t, amax_bits, sat, partials, slots, st);
  }
  if (fmt == kE4M3) return launch_flat_f<XT, kE4M3>(x, n, scale, q, amax_bits, sat, partials, slots, st);
  return launch_flat_f<XT, kE5M2>(x, n, scale, q, amax_bits, sat, partials, slots, st);
}

template <int XT, int FMT>
void launch_blockwise_t(const void* x, int64_t rows, int64_t cols, int block_rows, uint8_t* q,
                        float* scale_inv, hipStream_t st) {
  if (block_rows == 1) {
    const int64_t ntiles = rows * ((cols + 127) / 128);
    int64_t g = (ntiles + (kThreads / 16) - 1) / (kThreads / 16);
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL((quantize_rowtile_kernel<XT, FMT>), dim3((unsigned)g), dim3(kThreads), 0, st,
                       x, rows, cols, q, scale_inv);
  } else {
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    hipLaunchKernelGGL((quantize_block128_kernel<XT, FMT>), grid, dim3(kThreads), 0, st, x, rows,
                       cols, q, scale_inv);
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int xtype, int64_t rows, int64_t cols, int fmt,
                           const float* scale, uint8_t* q, uint8_t* q_t, float* amax,
                           unsigned long long* sat, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, HistoryArgs hs) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(amax);
  const bool reduce = amax_bits || sat;
  // With a workspace: per-workgroup partials, then one small reduction kernel.
  // Without: clear the outputs, then device-scope atomics per workgroup.
  uint4* partials = (reduce && workspace) ? reinterpret_cast<uint4*>(workspace) : nullptr;
  const int64_t slots = (int64_t)(workspace_bytes / sizeof(uint4));
  if (reduce && !partials) hipLaunchKernelGGL(zero_outputs_kernel, dim3(1), dim3(64), 0, stream, amax_bits, sat);
  int groups = 0;
  if (rows * cols > 0) {
    if (xtype == kBF16)
      groups = launch_quantize_x<kBF16>(x, rows, cols, fmt, scale, q, q_t, amax_bits, sat, partials, slots, stream);
    else
      groups = launch_quantize_x<kF32>(x, rows, cols, fmt, scale, q, q_t, amax_bits, sat, partials, slots, stream);
  }
  if (partials) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(1), dim3(kThreads), 0, stream, partials, groups, amax_bits, sat,
                       hs);
  } else if (hs.history) {
    if (hs.sinv_used) hipLaunchKernelGGL(copy_scalar_kernel, dim3(1), dim3(64), 0, stream, hs.scale_inv, hs.sinv_used);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_amax_update(hs.history, hs.len, hs.head, amax, hs.fmt, hs.scale, hs.scale_inv, hs.status, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The library's own scratch for callers that cannot allocate
// (fp8_quantize_update_noalloc): the per-workgroup partials of one cast, in a
// file-scope device array instead of a caller workspace.  Each GPU holds its
// own copy until the process ends.  Host code never uses the array's name as
// an address (on the host it names a stand-in, not device memory): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept in g_scratch_ptr.  Every workgroup of a cast writes
// its own slot and the reduction reads only the slots of that grid, so the
// contents a previous call left behind never need clearing.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_quantize_noalloc(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                   uint8_t* q_t, float* amax, unsigned long long* sat, hipStream_t stream,
                                   HistoryArgs hs) {
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_quantize(x, xtype, rows, cols, fmt, hs.scale, q, q_t, amax, sat, ws, kNoallocScratchBytes, stream,
                         hs);
}

hipError_t launch_quantize_blockwise(const void* x, int xtype, int64_t rows, int64_t cols,
                                     int block_rows, int fmt, uint8_t* q, float* scale_inv,
                                     hipStream_t stream) {
  if (rows * cols == 0) return hipSuccess;
  if (xtype == kBF16) {
    if (fmt == kE4M3) launch_blockwise_t<kBF16, kE4M3>(x, rows, cols, block_rows, q, scale_inv, stream);
    else launch_blockwise_t<kBF16, kE5M2>(x, rows, cols, block_rows, q, scale_inv, stream);
  } else {
    if (fmt == kE4M3) launch_blockwise_t<kF32, kE4M3>(x, rows, cols, block_rows, q, scale_inv, stream);
    else launch_blockwise_t<kF32, kE5M2>(x, rows, cols, block_rows, q, scale_inv, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8mi
