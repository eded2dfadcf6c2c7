// Stable global top-K select over gathered DCP candidates, gfx950.
//
// vLLM PR #47348 ("[Kernel] Optimize CuTeDSL DCP top-k merge", Summary): the
// selector finds the K-th best 32-bit score key by radix selection instead of
// sorting 64-bit (score key, complemented id) keys, and runs a token-id
// tie-break pass only when that score threshold ties.  The review comment on
// the same page describes the race this design avoids: the threshold was
// broadcast through shared memory that was then cleared for the next phase
// with no barrier in between, so late waves read a zero threshold and lost
// every tied candidate.  Here every pass broadcasts through its own LDS slot,
// histograms alternate between two buffers, and a buffer is cleared only after
// the barrier that ends its last read.
//
// One workgroup of 1024 threads (16 wave64s) owns one row.  Thread t keeps the
// candidates at positions v*VEC*1024 + VEC*t + j (v < NV, j < VEC) in VGPRs
// for the whole kernel, so the row is read from HBM exactly once; with VEC = 2
// every wave reads 1 KiB of contiguous candidates per 16-byte load.
//
// Per row:
//   1. score key  key = bits ^ (negative ? 0xFFFFFFFF : 0x80000000), an
//      order-preserving uint32 (IEEE totalOrder).
//   2. radix select on the key, MSB first, digits of 11, 11 and 10 bits.  Each
//      pass histograms the digit of the candidates that still match the prefix
//      (LDS atomics), then a suffix scan over the bins (DPP wave scan plus one
//      cross-wave step) finds the digit holding the K-th best key.  When the
//      chosen bin holds exactly the candidates still needed, the remaining
//      passes are skipped.
//   3. only if more candidates share the threshold key than are still needed:
//      the same radix select on u = ~id among the tied candidates (largest u =
//      lowest id first).  If even (key, id) ties at the boundary, candidate
//      position decides (lowest first).
//   4. stable compaction: selected flags -> wave ballots -> mbcnt prefix ->
//      one cross-wave scan in (chunk, wave, lane) order, which is candidate
//      position order -> each selected candidate is stored at its rank.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dcptopk {
namespace {

constexpr int kBlock = 1024;
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;
constexpr int kBins = 2048;       // widest digit: 11 bits
constexpr int kMaxPasses = 6;     // 3 score passes + 3 id passes
constexpr int kMaxSegments = 16 * kWaves;  // (chunk, wave) pairs, chunks <= 16

struct alignas(16) SelectLds {
  uint32_t hist[2][kBins];            // digit histograms, alternating by pass
  uint32_t wave_total[2][kWaves];     // cross-wave step of the bin scan
  uint32_t slot[kMaxPasses][4];       // per-pass broadcast: digit, above, count
  uint32_t segment[2][kMaxSegments];  // per (chunk, wave) flag counts
};

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its
// outstanding global loads, so the row's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

__device__ __forceinline__ uint32_t lane_of(uint32_t x, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), lane));
}

// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele inside
// each row of 16 lanes with DPP row shifts, then the row totals are added in
// from lanes 15, 31 and 47.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  const uint32_t r0 = lane_of(v, 15);
  const uint32_t r1 = lane_of(v, 31);
  const uint32_t r2 = lane_of(v, 47);
  v += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
  return v;
}

// Number of set bits of a wave ballot in lanes below this one.
__device__ __forceinline__ uint32_t ballot_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u));
}

__device__ __forceinline__ uint32_t score_key(uint32_t bits) {
  return bits ^ (static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t key_to_bits(uint32_t key) {
  return key ^ (static_cast<uint32_t>(static_cast<int32_t>(~key) >> 31) | 0x80000000u);
}

struct Digit {
  uint32_t digit;  // bin holding the K-th best value among the matching ones
  uint32_t above;  // matching values in higher bins
  uint32_t count;  // matching values in that bin
};

// Suffix scan of an NB-bin histogram: returns the bin d with
// above(d) < need <= above(d) + hist[d], where above(d) counts higher bins.
// Requires 1 <= need <= total.  Thread t reads the NB/1024 bins just below
// NB - (NB/1024)*t, so thread order is descending bin order.
template <int NB>
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, uint32_t need, uint32_t* wave_total,
                                            uint32_t* slot, int t, int lane, int w) {
  constexpr int kPer = NB / kBlock;
  static_assert(kPer == 1 || kPer == 2, "1024 or 2048 bins");
  const int lo = NB - kPer * (t + 1);
  uint32_t h[kPer];  // h[0] is this thread's highest bin
  if constexpr (kPer == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(hist + lo);
    h[0] = x.y;
    h[1] = x.x;
  } else {
    h[0] = hist[lo];
  }
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) sum += h[i];
  const uint32_t incl = wave_inclusive_scan(sum, lane);
  if (lane == kWave - 1) wave_total[w] = incl;
  lds_barrier();
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) before += (i < w) ? wave_total[i] : 0u;
  uint32_t above = before + incl - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (above < need && need <= above + h[i]) {
      slot[0] = static_cast<uint32_t>(lo + kPer - 1 - i);
      slot[1] = above;
      slot[2] = h[i];
    }
    above += h[i];
  }
  lds_barrier();
  Digit d;
  d.digit = uniform(slot[0]);
  d.above = uniform(slot[1]);
  d.count = uniform(slot[2]);
  return d;
}

// Clear the bins find_digit<NB> read in this thread.
template <int NB>
__device__ __forceinline__ void clear_bins(uint32_t* hist, int t) {
  constexpr int kPer = NB / kBlock;
  const int lo = NB - kPer * (t + 1);
  if constexpr (kPer == 2) {
    *reinterpret_cast<uint2*>(hist + lo) = make_uint2(0u, 0u);
  } else {
    hist[lo] = 0u;
  }
}

// Radix-select state of one value stream (score keys, or complemented ids).
struct Radix {
  uint32_t prefix;  // digits fixed so far
  uint32_t mask;    // bits covered by prefix
  uint32_t need;    // values still to take among those matching prefix
  uint32_t count;   // values matching prefix after the last pass
};

// One MSB-first pass over the digit at SHIFT (BITS wide) of the eligible
// values that match the prefix.
template <int SHIFT, int BITS, int N>
__device__ __forceinline__ void radix_pass(SelectLds& lds, int pass, const uint32_t (&val)[N], uint32_t eligible,
                                           Radix& st, int t, int lane, int w) {
  constexpr int NB = 1 << BITS;
  constexpr uint32_t kDigitMask = NB - 1;
  uint32_t* hist = lds.hist[pass & 1];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (((eligible >> i) & 1u) && (val[i] & st.mask) == st.prefix) {
      __hip_atomic_fetch_add(hist + ((val[i] >> SHIFT) & kDigitMask), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  lds_barrier();
  const Digit d = find_digit<NB>(hist, st.need, lds.wave_total[pass & 1], lds.slot[pass], t, lane, w);
  clear_bins<NB>(hist, t);  // reused two passes later, after at least one barrier
  st.prefix |= d.digit << SHIFT;
  st.mask |= kDigitMask << SHIFT;
  st.need -= d.above;
  st.count = d.count;
}

// Up to three passes (11, 11, 10 bits); stops early once the chosen bin holds
// exactly the values still needed.  Returns the number of passes run.
template <int N>
__device__ __forceinline__ int radix_select(SelectLds& lds, int pass, const uint32_t (&val)[N], uint32_t eligible,
                                            Radix& st, int t, int lane, int w) {
  radix_pass<21, 11>(lds, pass, val, eligible, st, t, lane, w);
  if (st.count == st.need) return 1;
  radix_pass<10, 11>(lds, pass + 1, val, eligible, st, t, lane, w);
  if (st.count == st.need) return 2;
  radix_pass<0, 10>(lds, pass + 2, val, eligible, st, t, lane, w);
  return 3;
}

// Exclusive prefix count of `flags` (bit i = item i) in candidate-position
// order (chunk v, thread t, slot j).  Needs one barrier; `segment` must not be
// read by any other phase between the two barriers around this call.
template <int VEC, int NV>
__device__ __forceinline__ void position_scan(uint32_t flags, uint32_t* segment, uint32_t (&rank)[VEC * NV],
                                              int lane, int w) {
  constexpr int kEntries = NV * kWaves;
  constexpr int kPerLane = (kEntries + kWave - 1) / kWave;
  uint32_t below[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const uint64_t b = __ballot((flags >> (v * VEC + j)) & 1u);
      before += ballot_below(b);
      total += static_cast<uint32_t>(__popcll(b));
    }
    below[v] = before;
    if (lane == 0) segment[v * kWaves + w] = total;
  }
  lds_barrier();
  // every wave scans all (chunk, wave) totals itself: no second barrier
  uint32_t x[kPerLane];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) {
    const int idx = lane * kPerLane + e;
    x[e] = idx < kEntries ? segment[idx] : 0u;
    sum += x[e];
  }
  const uint32_t incl = wave_inclusive_scan(sum, lane);
  uint32_t ex[kPerLane];
  ex[0] = incl - sum;
#pragma unroll
  for (int e = 1; e < kPerLane; ++e) ex[e] = ex[e - 1] + x[e - 1];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int entry = v * kWaves + w;
    uint32_t base = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const uint32_t b = lane_of(ex[e], entry / kPerLane);
      base = (entry % kPerLane == e) ? b : base;
    }
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      rank[v * VEC + j] = base + below[v] + own;
      own += (flags >> (v * VEC + j)) & 1u;
    }
  }
}

template <int VEC, int NV>
__global__ __launch_bounds__(kBlock) void stable_topk_select_kernel(const dcp_topk_cand* __restrict__ cand,
                                                                    int32_t num_cand, int32_t k,
                                                                    dcp_topk_cand* __restrict__ out) {
  constexpr int N = VEC * NV;
  static_assert(N <= 32, "flags are 32-bit masks");
  static_assert(NV * kWaves <= kMaxSegments, "segment table");
  __shared__ SelectLds lds;

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int w = static_cast<int>(uniform(static_cast<uint32_t>(t >> 6)));
  const int64_t row = blockIdx.x;
  const int C = num_cand;
  const uint32_t* in = reinterpret_cast<const uint32_t*>(cand + row * C);
  uint2* o = reinterpret_cast<uint2*>(out + row * static_cast<int64_t>(k));

  // k >= C: every candidate is selected, in place, then padding
  if (k >= C) {
    const uint2* src = reinterpret_cast<const uint2*>(in);
    for (int s = t; s < C; s += kBlock) o[s] = src[s];
    const uint2 pad = make_uint2(0xFF800000u, 0x7FFFFFFFu);
    for (int s = C + t; s < k; s += kBlock) o[s] = pad;
    return;
  }

  // 1. issue every load of the row before touching LDS.  Here C > k >= 1, so
  // clamping a position past the row to the last full vector keeps every
  // load in bounds without a branch; such items are masked out by `valid`.
  uint32_t key[N], idv[N];
  uint32_t valid = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int q = v * VEC * kBlock + VEC * t;
    const int qc = q < C ? q : C - VEC;
    if constexpr (VEC == 2) {
      const uint4 x = *reinterpret_cast<const uint4*>(in + 2 * static_cast<int64_t>(qc));
      key[2 * v] = x.x;
      idv[2 * v] = x.y;
      key[2 * v + 1] = x.z;
      idv[2 * v + 1] = x.w;
      if (q < C) valid |= 3u << (2 * v);  // C is even on this path
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(in + 2 * static_cast<int64_t>(qc));
      key[v] = x.x;
      idv[v] = x.y;
      if (q < C) valid |= 1u << v;
    }
  }

  // clear both histogram buffers while the loads are in flight; the key
  // transform stays after the barrier so that pass 1 starts on the first
  // chunk while later chunks are still arriving
  *reinterpret_cast<uint2*>(&lds.hist[0][2 * t]) = make_uint2(0u, 0u);
  *reinterpret_cast<uint2*>(&lds.hist[1][2 * t]) = make_uint2(0u, 0u);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) key[i] = score_key(key[i]);

  // 2. radix select on the score keys
  Radix sk{0u, 0u, static_cast<uint32_t>(k), 0u};
  int pass = radix_select(lds, 0, key, valid, sk, t, lane, w);

  // 3. id tie-break, only when the threshold key ties beyond what is needed
  const bool tie = sk.count > sk.need;  // implies all three score passes ran
  Radix ik{0u, 0u, sk.need, 0u};
  uint32_t tied = 0;
  uint32_t u[N];
#pragma unroll
  for (int i = 0; i < N; ++i) u[i] = ~idv[i];
  bool dup = false;
  uint32_t duprank[N];
  if (tie) {
#pragma unroll
    for (int i = 0; i < N; ++i) tied |= (((valid >> i) & 1u) && key[i] == sk.prefix) ? (1u << i) : 0u;
    pass += radix_select(lds, pass, u, tied, ik, t, lane, w);
    dup = ik.count > ik.need;  // identical (key, id) pairs straddle the boundary
    if (dup) {
      uint32_t same = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) same |= (((tied >> i) & 1u) && u[i] == ik.prefix) ? (1u << i) : 0u;
      position_scan<VEC, NV>(same, lds.segment[0], duprank, lane, w);
    }
  }

  // 4. stable compaction
  uint32_t sel = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t kp = key[i] & sk.mask;
    bool s = kp > sk.prefix;
    if (kp == sk.prefix) {
      if (!tie) {
        s = true;
      } else {
        const uint32_t up = u[i] & ik.mask;
        s = up > ik.prefix || (up == ik.prefix && (!dup || duprank[i] < ik.need));
      }
    }
    sel |= (s && ((valid >> i) & 1u)) ? (1u << i) : 0u;
  }
  uint32_t rank[N];
  position_scan<VEC, NV>(sel, lds.segment[1], rank, lane, w);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (((sel >> i) & 1u) && rank[i] < static_cast<uint32_t>(k)) o[rank[i]] = make_uint2(key_to_bits(key[i]), idv[i]);
  }
}

template <int VEC, int NV>
hipError_t launch(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, dcp_topk_cand* out,
                  hipStream_t stream) {
  void* args[] = {const_cast<dcp_topk_cand**>(&cand), &num_cand, &k, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stable_topk_select_kernel<VEC, NV>), dim3(rows),
                         dim3(kBlock), args, 0, stream);
}

}  // namespace

hipError_t launch_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, dcp_topk_cand* out,
                         hipStream_t stream) {
  const bool vec2 = (num_cand % 2 == 0) && (reinterpret_cast<uintptr_t>(cand) % 16 == 0);
  if (vec2) {
    if (num_cand <= 2 * kBlock) return launch<2, 1>(cand, rows, num_cand, k, out, stream);
    if (num_cand <= 4 * kBlock) return launch<2, 2>(cand, rows, num_cand, k, out, stream);
    if (num_cand <= 8 * kBlock) return launch<2, 4>(cand, rows, num_cand, k, out, stream);
    return launch<2, 8>(cand, rows, num_cand, k, out, stream);
  }
  if (num_cand <= 2 * kBlock) return launch<1, 2>(cand, rows, num_cand, k, out, stream);
  if (num_cand <= 4 * kBlock) return launch<1, 4>(cand, rows, num_cand, k, out, stream);
  if (num_cand <= 8 * kBlock) return launch<1, 8>(cand, rows, num_cand, k, out, stream);
  return launch<1, 16>(cand, rows, num_cand, k, out, stream);
}

}  // namespace dcptopk
