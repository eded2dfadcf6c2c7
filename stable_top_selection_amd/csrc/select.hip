// Stable global top-K select over gathered DCP candidates, gfx950.
//
// vLLM PR #47348 ("[Kernel] Optimize CuTeDSL DCP top-k merge", Summary): the
// selector finds the K-th best 32-bit score key by radix selection instead of
// sorting 64-bit (score key, complemented id) keys, and runs a token-id
// tie-break pass only when that score threshold ties.  The review comment on
// the same page describes a race to avoid: a threshold broadcast through shared
// memory that is cleared for the next phase without a barrier in between, so
// that late waves read a cleared threshold and drop every tied candidate.  This
// kernel has no broadcast slot at all: every wave scans the histogram itself
// and reaches the same digit, and histogram buffers rotate through three, so a
// buffer is cleared only one full barrier after its last read and refilled one
// barrier after that.
//
// One workgroup (256, 512 or 1024 threads: 4, 8 or 16 wave64s) owns one row.  Every
// thread keeps N candidates in VGPRs for the whole kernel: wave w holds the
// positions [w*64*N, (w+1)*64*N), its lane l the positions w*64*N +
// v*64*VEC + VEC*l + j (chunk v < N/VEC, j < VEC), so the row is read from
// memory once, each load instruction of a wave covering 64*VEC consecutive
// candidates (16-byte loads of candidate pairs, or of 4 scores or indices).
//
// Where the candidates come from and where the result goes are template
// policies, so one selection core serves three entry points: a gathered
// candidate buffer (the select), every DCP rank's local top-K arrays packed on
// the fly (the fused merge), and a dense score row with the column as id (the
// local top-K step, writing separate score and index arrays).
//
// Per row:
//   1. key = bits ^ (negative ? 0xFFFFFFFF : 0x80000000), an order-preserving
//      uint32 of the fp32 score (IEEE totalOrder).
//   2. Pass 0: LDS-atomic histogram of the top 11 key bits over the whole row.
//      Each atomic returns the item's rank inside its bin.  Every wave then
//      finds the bin d0 holding the K-th best key (two-level suffix scan: DPP
//      wave scans and ballots).
//   3. The items of bin d0 (a few percent of the row for smooth scores) write
//      themselves (score bits, id) into an LDS list at their rank; the list
//      passes turn the bits back into keys.  The remaining 21 key bits
//      are radix-selected over the list only (digits of 8, 8, 5 bits, small
//      histograms), stopping as soon as the chosen bin holds exactly the items
//      still needed.  Each list pass also keeps the first 8 items of every
//      digit in a per-digit bucket, so once the chosen digit holds at most 8
//      items (usually right after the first list pass) the threshold is
//      finished by comparing those items directly.  A bin too large for the
//      list falls back to the same passes over the register-resident row
//      (digits of 11 and 10 bits).
//   4. Only if more items share the threshold key than are still needed: the
//      same radix selection on u = ~id over the tied items (largest u = lowest
//      id), with the same finish by comparison.  If identical (key, id) pairs
//      still straddle the boundary, the lowest positions win.
//   5. Stable compaction: per-chunk selected counts packed into 8- or 16-bit
//      fields, scanned across the wave with DPP, in (wave, chunk, lane) order =
//      candidate-position order.  A wave's selected items fill one contiguous
//      output range, so each wave stages them in its own LDS area at their rank
//      inside the wave while the waves' counts are exchanged (one barrier),
//      then writes its range with consecutive stores, 64 items per store and
//      none past its count.  (A wave with more
//      selected items than its staging area stores every item at its rank
//      straight from registers; unselected items store to an offset past the
//      buffer's range, which the hardware drops, so no loop has a per-item
//      branch.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace dcptopk {
namespace {

constexpr int kWave = 64;
constexpr int kBins = 2048;      // widest digit: 11 bits
constexpr int kSmallBins = 256;  // list passes: digits of at most 8 bits
constexpr int kListCap = 2048;   // largest threshold bucket handled as a list
constexpr int kBucket = 8;       // items a list pass keeps per digit; smaller sub-bins finish by comparison
constexpr int kMaxSplit = kSplitMaxParts;  // most workgroups one row is split over (split-row select)
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr uint32_t kDropOffset = 0x80000000u;   // beyond any num_records used here
// Cache policy of the candidate loads and of the 8-byte result stores:
// non-temporal.  Every candidate is read exactly once and every result written
// once, so neither needs to stay in the caches; streaming the stores out as
// they are produced also leaves no dirty lines for the end-of-kernel release
// to write back.  (Measured on 256 rows x 8192 candidates: 8.82 -> 8.36 us per
// launch for the stores, 8.34 -> 7.92 us for the loads.)  The 4-byte stores of
// the split score/index output keep the default policy, which measured faster
// for them (5.53 -> 5.07 us for the local top-K of 64 rows x 4096 columns).
constexpr int kLoadPolicy = 2;   // nt
constexpr int kStorePolicy = 2;  // nt

typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));

// The padding candidate: what an empty output slot and an invalid local slot
// hold.
constexpr uint32_t kPadBits = 0xFF800000u;  // -inf
constexpr uint32_t kPadId = 0x7FFFFFFFu;    // INT32_MAX
constexpr uint32_t kPadKey = 0x007FFFFFu;   // the score key of -inf
constexpr uint32_t kPadBin = kPadKey >> 21; // its pass-0 bin
constexpr int kPadWords = 8;                // pass-0 counters of padding keys

// Race-stress build (a separate test library compiled with
// DCPTOPK_RACE_STRESS=1): every odd wave sleeps for tens of microseconds after
// each workgroup barrier, so it reads shared LDS long after the even waves have
// gone on to the next phase's writes, clears and reuse of buffers.  If any
// buffer were reused without a barrier after its last read (the race of the
// pages' review comment), the delayed waves would read the new contents and the
// result would differ from the oracle.
#ifndef DCPTOPK_RACE_STRESS
#define DCPTOPK_RACE_STRESS 0
#endif

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its
// outstanding global loads, so the row's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if constexpr (DCPTOPK_RACE_STRESS != 0) {
    if ((__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x)) >> 6) & 1) {
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_s_sleep(127);  // about 32k cycles
    }
  }
}

// Phase stamps, a diagnostic build (DCPTOPK_PHASE_STAMPS=1, a library of its
// own): lane 0 of the first and of the last wave of each of the first
// kStampRows workgroups records the shader clock (s_memtime) at each phase
// boundary of the select kernel, with a vector store into phase_stamps, which
// dcptopk_phase_stamps copies out.  A stamped wave finds its slots once, while
// its first loads are in flight (stamp_slots); a stamp is then the clock read,
// its wait and one store (about 64 cycles; looking the slots up at every stamp
// took about 220).  The first two boundaries (the wave's start and the moment
// its first row loads issue) are only read into registers with phase_clock()
// and stored after the first barrier with stamp_value(), so that nothing holds
// back the kernel argument and row loads.  In every other build stamp_slots()
// and phase_clock() return 0 and the stamps compile to nothing.
#ifndef DCPTOPK_PHASE_STAMPS
#define DCPTOPK_PHASE_STAMPS 0
#endif
#if DCPTOPK_PHASE_STAMPS
constexpr int kStampRows = 1024;  // workgroups stamped
constexpr int kStampSlots = 16;   // phase boundaries per wave
__device__ unsigned long long phase_stamps[kStampRows * 2 * kStampSlots];
#endif

// This wave's stamp slots if it is stamped (wave-uniform), else null.
template <int BLOCK>
__device__ __forceinline__ unsigned long long* stamp_slots(int w) {
#if DCPTOPK_PHASE_STAMPS
  return (w == 0 || w == BLOCK / kWave - 1) && blockIdx.x < kStampRows
             ? phase_stamps + (blockIdx.x * 2 + (w != 0)) * kStampSlots
             : nullptr;
#else
  (void)w;
  return nullptr;
#endif
}

__device__ __forceinline__ unsigned long long phase_clock() {
#if DCPTOPK_PHASE_STAMPS
  __builtin_amdgcn_sched_barrier(0);  // the read stays where it is written
  const unsigned long long now = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return now;
#else
  return 0;
#endif
}

__device__ __forceinline__ void stamp_value(unsigned long long* slots, int phase, int lane, unsigned long long value) {
#if DCPTOPK_PHASE_STAMPS
  if (slots != nullptr && lane == 0) slots[phase] = value;
#else
  (void)slots;
  (void)phase;
  (void)lane;
  (void)value;
#endif
}

__device__ __forceinline__ void stamp(unsigned long long* slots, int phase, int lane) {
#if DCPTOPK_PHASE_STAMPS
  const unsigned long long now = phase_clock();
  stamp_value(slots, phase, lane, now);
  __builtin_amdgcn_sched_barrier(0);
#else
  (void)slots;
  (void)phase;
  (void)lane;
#endif
}

__device__ __forceinline__ uint32_t lane_of(uint32_t x, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), lane));
}

__device__ __forceinline__ int first_lane(uint64_t ballot) { return __builtin_ctzll(ballot); }

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

__device__ __forceinline__ uint32_t lds_add(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele inside
// each row of 16 lanes with DPP row shifts, then the row totals carried across
// the rows with the DPP row broadcasts (lane 15 into rows 1 and 3, then lane
// 31 into rows 2 and 3), with no lane read through a scalar register in the
// chain (measured against reading lanes 15, 31 and 47 and adding them in:
// large 7.55 -> 7.43 us, decode 16 rows 5.78 -> 5.69, tie-heavy 7.73 -> 7.59).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
  (void)lane;
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ uint32_t score_key(uint32_t bits) {
  return bits ^ (static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u);
}

struct Digit {
  uint32_t digit;  // bin holding the need-th largest value among those counted
  uint32_t above;  // counted values in higher bins
  uint32_t count;  // counted values in that bin
};

// Finds the bin d of an NB-bin histogram (NB >= 256) with above(d) < need <=
// above(d) + hist[d], where above(d) sums the bins above d.  Every wave runs
// this on its own and gets the same (wave-uniform) answer.  Requires
// 1 <= need <= total.
//
// Level 1: lane l sums the PER bins [NB - PER*(l+1), NB - PER*l), so lane
// order is descending bin order; a wave scan and a ballot give the first lane
// whose running count reaches `need`.  Level 2: that lane's PER bins, one per
// lane, highest first; a second scan and ballot give the bin.
template <int NB>
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, uint32_t need, int lane) {
  constexpr int PER = NB / kWave;
  constexpr int VECS = PER / 4;
  static_assert(VECS >= 1, "at least 256 bins");
  const uint4* p = reinterpret_cast<const uint4*>(hist + NB - PER * (lane + 1));
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < VECS; ++i) {
    // rotate the start by lane so that the 64 lanes' 16-byte reads spread over
    // all banks instead of all starting on the same one
    const uint4 x = p[(i + lane) & (VECS - 1)];
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t incl = wave_inclusive_scan(sum, lane);
  // the forced top bits keep L and i inside the histogram even if `need`
  // exceeded the total (the callers never let it)
  const int L = first_lane(__ballot(incl >= need) | (1ull << 63));
  const uint32_t above_l = lane_of(incl, L) - lane_of(sum, L);
  const int top = NB - PER * L - 1;  // highest bin of lane L
  const uint32_t h = lane < PER ? hist[top - lane] : 0u;
  const uint32_t incl2 = wave_inclusive_scan(h, lane);
  const int i = first_lane(__ballot(lane < PER && above_l + incl2 >= need) | (1ull << (PER - 1)));
  Digit d;
  d.digit = static_cast<uint32_t>(top - i);
  d.count = lane_of(h, i);
  d.above = above_l + lane_of(incl2, i) - d.count;
  return d;
}

// find_digit over the pass-0 histogram with `extra` items added to bin
// `extra_bin` (the padding keys, which pass 0 counts apart).
__device__ __forceinline__ Digit find_digit_pass0(const uint32_t* hist, uint32_t need, int lane, uint32_t extra_bin,
                                                  uint32_t extra) {
  constexpr int PER = kBins / kWave;
  constexpr int VECS = PER / 4;
  const uint4* p = reinterpret_cast<const uint4*>(hist + kBins - PER * (lane + 1));
  uint32_t sum = lane == static_cast<int>((kBins - 1 - extra_bin) / PER) ? extra : 0u;
#pragma unroll
  for (int i = 0; i < VECS; ++i) {
    const uint4 x = p[(i + lane) & (VECS - 1)];
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t incl = wave_inclusive_scan(sum, lane);
  const int L = first_lane(__ballot(incl >= need) | (1ull << 63));
  const uint32_t above_l = lane_of(incl, L) - lane_of(sum, L);
  const int top = kBins - PER * L - 1;
  uint32_t h = lane < PER ? hist[top - lane] : 0u;
  h += (lane < PER && static_cast<uint32_t>(top - lane) == extra_bin) ? extra : 0u;
  const uint32_t incl2 = wave_inclusive_scan(h, lane);
  const int i = first_lane(__ballot(lane < PER && above_l + incl2 >= need) | (1ull << (PER - 1)));
  Digit d;
  d.digit = static_cast<uint32_t>(top - i);
  d.count = lane_of(h, i);
  d.above = above_l + lane_of(incl2, i) - d.count;
  return d;
}

// The same search for the small histograms of the list passes (NB <= 256):
// lane l holds PER = max(1, NB/64) bins; the bin inside lane L is resolved in
// scalar registers.
template <int NB>
__device__ __forceinline__ Digit find_digit_small(const uint32_t* hist, uint32_t need, int lane) {
  constexpr int PER = NB >= kWave ? NB / kWave : 1;
  constexpr int LANES = NB / PER;
  static_assert(PER == 1 || PER == 2 || PER == 4, "1, 2 or 4 bins per lane");
  uint32_t h[PER];  // h[0] = this lane's highest bin
  const int lo = NB - PER * (lane + 1);
  if constexpr (PER == 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(hist + lo);
    h[0] = x.w;
    h[1] = x.z;
    h[2] = x.y;
    h[3] = x.x;
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) h[j] = lane < LANES ? hist[lo + PER - 1 - j] : 0u;
  }
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += h[j];
  const uint32_t incl = wave_inclusive_scan(sum, lane);
  const int L = first_lane(__ballot(lane < LANES && incl >= need) | (1ull << (LANES - 1)));
  uint32_t above = lane_of(incl, L) - lane_of(sum, L);
  Digit d{0u, 0u, 0u};
  bool found = false;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t c = lane_of(h[j], L);
    if (!found && above + c >= need) {
      d.digit = static_cast<uint32_t>(NB - PER * L - 1 - j);
      d.above = above;
      d.count = c;
      found = true;
    }
    above += c;
  }
  return d;
}

// Radix-select state of one value stream (score keys, or complemented ids).
struct Radix {
  uint32_t prefix;  // digits fixed so far
  uint32_t mask;    // bits covered by prefix
  uint32_t need;    // values still to take among those matching prefix
  uint32_t count;   // values matching prefix after the last pass
};

__device__ __forceinline__ void advance(Radix& st, const Digit& d, int shift, uint32_t digit_mask) {
  st.prefix |= d.digit << shift;
  st.mask |= digit_mask << shift;
  st.need -= d.above;
  st.count = d.count;
}

template <int BLOCK>
struct alignas(16) SelectLds {
  static constexpr int kWaves = BLOCK / kWave;
  uint32_t hist[3][kBins];         // pass 0 (hist[0]) and the register passes, rotating
  uint32_t small[3][kSmallBins];   // list passes, rotating
  uint32_t padcnt[kPadWords];      // pass 0: counts of padding keys, by lane % kPadWords
  uint2 list[kListCap + 1];        // (score bits, id) of the items in the pass-0 threshold bin, then
                                   // one write-only dump slot for all other items
  uint32_t segment[2][kWaves];     // per-wave flagged counts (dup scan, select scan)
  uint32_t slices[3][kMaxSplit];   // split rows: per slice, keys above the threshold bin, selected
                                   // keys of the bin other than full duplicates, full duplicates
  uint32_t sink[kWave];            // per-lane target of atomics whose item does not count
  uint32_t common[4];              // OR / AND of the list's keys and of its complemented ids
};

// Clear `words` (a multiple of 4) words of LDS.
template <int BLOCK>
__device__ __forceinline__ void clear_words(uint32_t* p, int words, int t) {
  for (int i = 4 * t; i < words; i += 4 * BLOCK) *reinterpret_cast<uint4*>(p + i) = make_uint4(0u, 0u, 0u, 0u);
}

// Register pass p >= 1 over the digit at SHIFT (BITS wide) of the eligible
// values that match the prefix (the values are ~val[i] when COMPL, so ids are
// ranked with no complemented copy held in registers).  Uses hist[p % 3];
// after its barrier clears hist[(p + 2) % 3], which pass p - 1 used and pass
// p + 2 will use.
template <int BLOCK, int SHIFT, int BITS, bool COMPL, int N>
__device__ __forceinline__ void radix_pass(SelectLds<BLOCK>& lds, int pass, const uint32_t (&val)[N],
                                           uint32_t eligible, Radix& st, int t, int lane) {
  constexpr int NB = 1 << BITS;
  constexpr uint32_t kDigitMask = NB - 1;
  uint32_t* hist = lds.hist[pass % 3];
  uint32_t* sink = lds.sink + lane;
  // every item issues its atomic, to its bin if it counts, else to this lane's
  // sink word: no per-item branch
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t v = COMPL ? ~val[i] : val[i];
    const bool counts = ((eligible >> i) & 1u) && (v & st.mask) == st.prefix;
    lds_add(counts ? hist + ((v >> SHIFT) & kDigitMask) : sink);
  }
  lds_barrier();
  clear_words<BLOCK>(lds.hist[(pass + 2) % 3], kBins, t);
  advance(st, find_digit<NB>(hist, st.need, lane), SHIFT, kDigitMask);
}

// List pass q over the digit at SHIFT (BITS wide): score keys of the list
// (BY_ID false) or complemented ids of the list items whose key is `thr`.
// ALL: every list item matches (the first key pass, whose list holds exactly
// the items of the pass-0 threshold bin), so no item is tested and each reads
// its (score bits, id) pair in one LDS load; an item past its digit's bucket writes
// to a dump slot (the first word after the buckets, in hist[2], which no list
// path uses) instead of branching.
// Counts into small[q % 3] and, after its barrier, clears small[(q + 2) % 3]
// (used by pass q - 1, next used by pass q + 2).  The pass also sorts the list
// coarsely: each counted item's atomic returns its rank inside its digit, and
// the first kBucket items of every digit copy their (key, ~id) into
// bucket[digit * kBucket + rank].  Returns the chosen digit's bucket, which
// holds all of that digit's items when it has at most kBucket of them, so the
// threshold can then be finished by comparison with no further pass or
// barrier.  The buckets overlay the pass-0 histograms, which every wave has
// finished reading before the list build's barrier; each pass overwrites the
// previous pass's buckets, which are read only when no further pass follows.
template <int BLOCK, int SHIFT, int BITS, bool BY_ID, bool ALL = false>
__device__ __forceinline__ const uint2* list_pass(SelectLds<BLOCK>& lds, int q, int m, uint32_t thr, Radix& st,
                                                  int t, int lane) {
  constexpr int NB = 1 << BITS;
  constexpr uint32_t kDigitMask = NB - 1;
  static_assert(sizeof(lds.hist) >= (NB * kBucket + 1) * sizeof(uint2), "buckets and the dump slot fit");
  static_assert(!ALL || !BY_ID, "only the first key pass takes every item");
  uint32_t* hist = lds.small[q % 3];
  uint2* bucket = reinterpret_cast<uint2*>(&lds.hist[0][0]);
  for (int e = t; e < m; e += BLOCK) {
    const uint2 x = lds.list[e];
    const uint32_t kx = score_key(x.x);
    const uint32_t v = BY_ID ? ~x.y : kx;
    if constexpr (ALL) {
      const uint32_t d = (v >> SHIFT) & kDigitMask;
      const uint32_t r = lds_add(hist + d);
      bucket[r < static_cast<uint32_t>(kBucket) ? d * kBucket + r : NB * kBucket] = make_uint2(kx, ~x.y);
    } else if ((!BY_ID || kx == thr) && (v & st.mask) == st.prefix) {
      const uint32_t d = (v >> SHIFT) & kDigitMask;
      const uint32_t r = lds_add(hist + d);
      if (r < static_cast<uint32_t>(kBucket)) bucket[d * kBucket + r] = make_uint2(kx, ~x.y);
    }
  }
  lds_barrier();
  if (t < kSmallBins / 4) *reinterpret_cast<uint4*>(lds.small[(q + 2) % 3] + 4 * t) = make_uint4(0u, 0u, 0u, 0u);
  advance(st, find_digit_small<NB>(hist, st.need, lane), SHIFT, kDigitMask);
  return bucket + ((st.prefix >> SHIFT) & kDigitMask) * kBucket;
}

// The id tie-break's list pass: like list_pass with BY_ID, but over the
// digit of `bits` (<= 8) bits at a run-time `shift`, so that the digits can
// start at the highest bit where the tied items' ids differ.
template <int BLOCK>
__device__ __forceinline__ const uint2* list_pass_ids(SelectLds<BLOCK>& lds, int q, int m, uint32_t thr, Radix& st,
                                                      int shift, int bits, int t, int lane) {
  const uint32_t dmask = (1u << bits) - 1u;
  uint32_t* hist = lds.small[q % 3];
  uint2* bucket = reinterpret_cast<uint2*>(&lds.hist[0][0]);
  for (int e = t; e < m; e += BLOCK) {
    const uint2 x = lds.list[e];
    const uint32_t v = ~x.y;
    if (score_key(x.x) == thr && (v & st.mask) == st.prefix) {
      const uint32_t d = (v >> shift) & dmask;
      const uint32_t r = lds_add(hist + d);
      if (r < static_cast<uint32_t>(kBucket)) bucket[d * kBucket + r] = make_uint2(thr, v);
    }
  }
  lds_barrier();
  if (t < kSmallBins / 4) *reinterpret_cast<uint4*>(lds.small[(q + 2) % 3] + 4 * t) = make_uint4(0u, 0u, 0u, 0u);
  advance(st, find_digit_small<kSmallBins>(hist, st.need, lane), shift, dmask);
  return bucket + ((st.prefix >> shift) & dmask) * kBucket;
}

// Finishes the key threshold by comparison.  items[0..sk.count) hold the
// (key, ~id) pairs of the items that match sk's prefix (sk.count <= kBucket,
// written before a barrier this wave has passed).  The need-th largest key
// among them becomes sk's full threshold key (sk.need: how many items with
// that key are still needed; sk.count: how many there are).  If they tie
// (count > need), the same ranking on ~id among the tied ones fills ik the way
// the id passes would, and the function returns true.
__device__ __forceinline__ bool few_rank(const uint2* items, Radix& sk, Radix& ik, int lane) {
  const int c = static_cast<int>(sk.count);  // <= kBucket
  const uint2 x = lane < c ? items[lane] : make_uint2(0u, 0u);
  uint32_t kg = 0u, ke = 0u;
  for (int j = 0; j < c; ++j) {
    const uint32_t kj = lane_of(x.x, j);
    kg += kj > x.x ? 1u : 0u;
    ke += kj == x.x ? 1u : 0u;
  }
  // the lane holding the need-th largest key (the clamp keeps L in range)
  const int L = first_lane(__ballot(lane < c && kg < sk.need && sk.need <= kg + ke) | (1ull << (kBucket - 1)));
  sk.prefix = lane_of(x.x, L);
  sk.mask = ~0u;
  sk.need -= lane_of(kg, L);
  sk.count = lane_of(ke, L);
  if (sk.count <= sk.need) return false;  // every item with the threshold key is taken
  const bool tied = lane < c && x.x == sk.prefix;
  uint32_t ug = 0u, ue = 0u;
  for (int j = 0; j < c; ++j) {
    const bool tj = lane_of(x.x, j) == sk.prefix;
    const uint32_t uj = lane_of(x.y, j);
    ug += (tj && uj > x.y) ? 1u : 0u;
    ue += (tj && uj == x.y) ? 1u : 0u;
  }
  const int L2 = first_lane(__ballot(tied && ug < sk.need && sk.need <= ug + ue) | (1ull << (kBucket - 1)));
  ik.prefix = lane_of(x.y, L2);
  ik.mask = ~0u;
  ik.need = sk.need - lane_of(ug, L2);
  ik.count = lane_of(ue, L2);
  return true;
}

// The same finish for the id tie-break: items[0..ik.count) hold the tied items
// that match ik's prefix (ik.count <= kBucket); the need-th largest ~id among
// them becomes ik's full threshold.
__device__ __forceinline__ void few_rank_ids(const uint2* items, Radix& ik, int lane) {
  const int c = static_cast<int>(ik.count);
  const uint32_t u = lane < c ? items[lane].y : 0u;
  uint32_t g = 0u, e = 0u;
  for (int j = 0; j < c; ++j) {
    const uint32_t uj = lane_of(u, j);
    g += uj > u ? 1u : 0u;
    e += uj == u ? 1u : 0u;
  }
  const int L = first_lane(__ballot(lane < c && g < ik.need && ik.need <= g + e) | (1ull << (kBucket - 1)));
  ik.prefix = lane_of(u, L);
  ik.mask = ~0u;
  ik.need -= lane_of(g, L);
  ik.count = lane_of(e, L);
}

// OR / AND of v over the wave (wave-uniform): DPP row shifts inside each row
// of 16 lanes (lanes shifted in from outside the row keep the identity), then
// the four row results from lanes 15, 31, 47 and 63.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  return lane_of(v, 15) | lane_of(v, 31) | lane_of(v, 47) | lane_of(v, 63);
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  v &= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v &= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v &= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v &= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  return lane_of(v, 15) & lane_of(v, 31) & lane_of(v, 47) & lane_of(v, 63);
}

// OR and AND over the whole workgroup of this thread's partial key OR / AND
// (a, b) and complemented-id OR / AND (c, d): bits where every counted item
// agrees are ~(or ^ and).  DPP reductions inside each wave, then LDS atomics
// into lds.common[0..3], which the kernel initialised before its first
// barrier.  One barrier; a kernel calls it at most once.
template <int BLOCK>
__device__ __forceinline__ void block_common_bits(SelectLds<BLOCK>& lds, int lane, uint32_t a, uint32_t b, uint32_t c,
                                                  uint32_t d, uint32_t& kor, uint32_t& kand, uint32_t& uor,
                                                  uint32_t& uand) {
  a = wave_or(a);
  b = wave_and(b);
  c = wave_or(c);
  d = wave_and(d);
  if (lane == 0) {
    __hip_atomic_fetch_or(lds.common + 0, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_and(lds.common + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_or(lds.common + 2, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_and(lds.common + 3, d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  lds_barrier();
  kor = uniform(lds.common[0]);
  kand = uniform(lds.common[1]);
  uor = uniform(lds.common[2]);
  uand = uniform(lds.common[3]);
}

// The common bits of the threshold list's keys and complemented ids.
template <int BLOCK>
__device__ __forceinline__ void list_common_bits(SelectLds<BLOCK>& lds, int m, int t, int lane, uint32_t& kor,
                                                 uint32_t& kand, uint32_t& uor, uint32_t& uand) {
  uint32_t a = 0u, b = ~0u, c = 0u, d = ~0u;
  for (int e = t; e < m; e += BLOCK) {
    const uint2 x = lds.list[e];
    const uint32_t kx = score_key(x.x);
    a |= kx;
    b &= kx;
    c |= ~x.y;
    d &= ~x.y;
  }
  block_common_bits(lds, lane, a, b, c, d, kor, kand, uor, uand);
}

// Exclusive rank of every flagged item (flag[i] is 0 or 1) among the flagged
// items of its own wave, in candidate-position order; returns the wave's
// flagged count (wave-uniform).  Wave w owns the contiguous positions
// [w*64*N, (w+1)*64*N); inside it, chunk v holds 64*VEC consecutive
// positions, lane-major.  So a rank is: flagged items of earlier chunks of
// this wave (scalar) + of earlier lanes in this chunk (packed DPP scan) + of
// earlier slots of this thread.
template <int VEC, int N>
__device__ __forceinline__ uint32_t wave_rank(const uint32_t (&flag)[N], uint32_t (&rank)[N], int lane) {
  constexpr int NV = N / VEC;  // chunks per thread
  // per-thread count of flagged items in each chunk (<= VEC), packed into
  // fields wide enough for a wave's running count of one chunk (<= 64*VEC):
  // 8 bits up to VEC 2, 16 bits for VEC 4, so fields never carry
  constexpr int kFieldBits = kWave * VEC < 256 ? 8 : 16;
  constexpr int kPerWord = 32 / kFieldBits;
  constexpr uint32_t kFieldMask = (1u << kFieldBits) - 1u;
  constexpr int NW = (NV + kPerWord - 1) / kPerWord;
  uint32_t packed[NW];
#pragma unroll
  for (int q = 0; q < NW; ++q) packed[q] = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < VEC; ++j) c += flag[v * VEC + j];
    packed[v / kPerWord] += c << (kFieldBits * (v % kPerWord));
  }
  uint32_t excl[NW], total[NW];
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    const uint32_t incl = wave_inclusive_scan(packed[q], lane);
    excl[q] = incl - packed[q];
    total[q] = lane_of(incl, kWave - 1);  // this wave's count of each chunk, packed
  }
  uint32_t wave_total = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    uint32_t own = wave_total + ((excl[v / kPerWord] >> (kFieldBits * (v % kPerWord))) & kFieldMask);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      rank[v * VEC + j] = own;
      own += flag[v * VEC + j];
    }
    wave_total += (total[v / kPerWord] >> (kFieldBits * (v % kPerWord))) & kFieldMask;
  }
  return wave_total;
}

// Flagged items of the waves before wave w, once every wave has published its
// count in segment[w] and passed a barrier (wave-uniform).
template <int BLOCK>
__device__ __forceinline__ uint32_t waves_before(const uint32_t* segment, int w) {
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < BLOCK / kWave; ++i) before += i < w ? segment[i] : 0u;
  return uniform(before);
}

// Exclusive rank of every flagged item among all flagged items of the row in
// candidate-position order (one barrier).  `segment` must belong to this call
// alone.
template <int BLOCK, int VEC, int N>
__device__ __forceinline__ void position_rank(const uint32_t (&flag)[N], uint32_t* segment, uint32_t (&rank)[N],
                                              int lane, int w) {
  const uint32_t total = wave_rank<VEC, N>(flag, rank, lane);
  if (lane == 0) segment[w] = total;
  lds_barrier();
  const uint32_t before = waves_before<BLOCK>(segment, w);
#pragma unroll
  for (int i = 0; i < N; ++i) rank[i] += before;
}

// ---------------------------------------------------------------------------
// Candidate sources.  A source yields the (score bits, id) of this thread's
// items: chunk v of wave w holds positions first + v*64*VEC + j (j < VEC), with
// first = w*64*N + VEC*lane.  count(row) is the row's candidate count C (at
// most the launch's num_cand); the values at positions at or past C are
// ignored.  load() only issues the reads (into bits/idv and, for per-chunk
// values the same across the wave, two words per chunk of aux);
// finish<VEC>(v, ...) turns what arrived for chunk
// v into (score bits, id).  The kernel finishes each chunk just before it
// first uses it, after its first barrier, so the loads stay in flight while
// it clears LDS and the work on early chunks overlaps later chunks' arrival.
// ---------------------------------------------------------------------------

// A row-major gathered candidate buffer: raw buffer loads over the row, the
// chunk offset in a scalar register.
struct GatheredSource {
  const dcp_topk_cand* cand;
  int32_t num_cand;
  // chunks can be loaded one at a time (load_chunk), so the kernel may issue
  // part of a row's loads after its first barrier
  static constexpr bool kChunkLoads = true;

  __device__ __forceinline__ int count(int64_t) const { return num_cand; }

  template <int VEC>
  __device__ __forceinline__ void finish(int, const uint32_t*, uint32_t*, uint32_t*) const {}

  // issues the load of chunk v (v is a constant once the caller's loop is
  // unrolled)
  template <int VEC>
  __device__ __forceinline__ void load_chunk(int64_t row, int first, int C, int v, uint32_t* bits,
                                             uint32_t* idv) const {
    constexpr int kChunk = VEC * kWave;
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<dcp_topk_cand*>(cand + row * num_cand), 0, C * static_cast<int>(sizeof(dcp_topk_cand)),
        static_cast<int>(kBufferWord3));
    const int voff = first * static_cast<int>(sizeof(dcp_topk_cand));
    const int soff = v * kChunk * static_cast<int>(sizeof(dcp_topk_cand));
    if constexpr (VEC == 2) {
      const int4 x = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(src, voff, soff, kLoadPolicy));
      bits[2 * v] = x.x;
      idv[2 * v] = x.y;
      bits[2 * v + 1] = x.z;
      idv[2 * v + 1] = x.w;
    } else {
      const int2v x = __builtin_amdgcn_raw_buffer_load_b64(src, voff, soff, kLoadPolicy);
      bits[v] = x.x;
      idv[v] = x.y;
    }
  }

  template <int VEC, int NV>
  __device__ __forceinline__ void load(int64_t row, int first, int C, uint32_t* bits, uint32_t* idv,
                                       uint32_t*) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) load_chunk<VEC>(row, first, C, v, bits, idv);
  }
};

// Every DCP rank's local top-K arrays, read in place and packed on the fly
// (the fused merge): position r*local_k + j of a row is rank r's slot j, its
// id is local index + row start + rank offset with two's-complement wrap, and
// a negative local index is the padding candidate (vLLM PR #59367, Purpose).
// local_k is a multiple of 64*VEC, so a chunk never straddles two ranks and a
// chunk's rank is wave-uniform.  A wave reads every chunk's rank-table entry
// in one round of scalar loads, then the chunks' row starts as vector loads
// and then the data, all without a wait in between: a chunk's id base
// (row start in aux[2v], rank offset in aux[2v+1]) is back when its data is.
// (Against one round of scalar loads per chunk, each waiting for its row start
// before the next: 256 rows 8.13 -> 8.09 us, 8192 rows in one launch 125.5 ->
// 122.8 us, in one process on one box.)
struct RankSource {
  static constexpr bool kChunkLoads = false;  // a wave's loads go out together (see load)
  FusedRanks ranks;
  int32_t local_k;
  int32_t num_cand;  // dcp * local_k
  int32_t last_rank;  // dcp - 1

  __device__ __forceinline__ int count(int64_t) const { return num_cand; }

  template <int VEC, int NV>
  __device__ __forceinline__ void load(int64_t row, int first, int, uint32_t* bits, uint32_t* idv,
                                       uint32_t* aux) const {
    constexpr int kChunk = VEC * kWave;
    const int lane_off = first & (kChunk - 1);
    // the wave's first position, and the rank and local slot it falls in
    const int chunk0 = __builtin_amdgcn_readfirstlane(first - lane_off);
    int rk[NV], j0[NV];
    {
      int r = chunk0 / local_k;
      int j = chunk0 - r * local_k;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        // a chunk past the row (r > last_rank; its values are ignored) reads
        // the last rank's slots instead, which are in bounds
        rk[v] = r <= last_rank ? r : last_rank;
        j0[v] = r <= last_rank ? j : 0;
        j += kChunk;
        if (j == local_k) {
          j = 0;
          ++r;
        }
      }
    }
    const float* sp[NV];
    const int32_t* ip[NV];
    const int32_t* rp[NV];
    uint32_t off[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const PackRank& pr = ranks.rank[rk[v]];
      sp[v] = pr.scores;
      ip[v] = pr.idx;
      rp[v] = pr.row_starts;
      off[v] = static_cast<uint32_t>(pr.rank_offset);
    }
    __builtin_amdgcn_sched_barrier(0);  // every chunk's rank entry in one round of scalar loads
    // the chunks' row starts as vector loads, ahead of the data loads: the
    // data loads issue without waiting for them, the first barrier (which
    // waits for scalar loads) does not either, and waiting for a chunk's data
    // covers its row start (loads return in order)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(rp[v]), 0, static_cast<int>(row + 1) * static_cast<int>(sizeof(int32_t)),
          static_cast<int>(kBufferWord3));
      aux[2 * v] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(row) * 4, 0, 0));
      aux[2 * v + 1] = off[v];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (VEC == 4) {
        // raw buffer loads over the chunk's 256 slots of this row (32-bit
        // offsets from a scalar base, like the gathered source; against
        // 64-bit global addresses: 256 rows 8.09 -> 8.03 us, 8192 rows in one
        // launch 123.1 -> 120.3 us)
        const int64_t at = row * local_k + j0[v];
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(sp[v] + at), 0, kChunk * 4, static_cast<int>(kBufferWord3));
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(ip[v] + at), 0, kChunk * 4, static_cast<int>(kBufferWord3));
        const int4v s4 = __builtin_bit_cast(int4v, __builtin_amdgcn_raw_buffer_load_b128(sr, lane_off * 4, 0, kLoadPolicy));
        const int4v i4 = __builtin_bit_cast(int4v, __builtin_amdgcn_raw_buffer_load_b128(ir, lane_off * 4, 0, kLoadPolicy));
        bits[4 * v] = s4.x;
        bits[4 * v + 1] = s4.y;
        bits[4 * v + 2] = s4.z;
        bits[4 * v + 3] = s4.w;
        idv[4 * v] = i4.x;
        idv[4 * v + 1] = i4.y;
        idv[4 * v + 2] = i4.z;
        idv[4 * v + 3] = i4.w;
      } else if constexpr (VEC == 2) {
        // (narrower loads keep 64-bit global addresses: buffer loads here take
        // the partial-row kernel past 128 VGPRs)
        const int64_t at = row * local_k + j0[v] + lane_off;
        const int2v s2 = __builtin_nontemporal_load(reinterpret_cast<const int2v*>(sp[v] + at));
        const int2v i2 = __builtin_nontemporal_load(reinterpret_cast<const int2v*>(ip[v] + at));
        bits[2 * v] = s2.x;
        bits[2 * v + 1] = s2.y;
        idv[2 * v] = i2.x;
        idv[2 * v + 1] = i2.y;
      } else {
        const int64_t at = row * local_k + j0[v] + lane_off;
        bits[v] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp[v] + at));
        idv[v] = static_cast<uint32_t>(__builtin_nontemporal_load(ip[v] + at));
      }
      // issue the loads chunk by chunk (scores and indices together), so that
      // pass 0 can start on chunk 0 as soon as its two loads are back
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // bits/idv hold score bits and local indices, aux the chunks' id bases
  template <int VEC>
  __device__ __forceinline__ void finish(int v, const uint32_t* aux, uint32_t* bits, uint32_t* idv) const {
    const uint32_t base = aux[2 * v] + aux[2 * v + 1];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const bool invalid = static_cast<int32_t>(idv[v * VEC + j]) < 0;
      bits[v * VEC + j] = invalid ? kPadBits : bits[v * VEC + j];
      idv[v * VEC + j] = invalid ? kPadId : idv[v * VEC + j] + base;
    }
  }
};

// A dense fp32 score row (the local top-K step): the candidate at column c has
// id c; with per-row lengths only the first lengths[row] columns take part.
struct DenseSource {
  static constexpr bool kChunkLoads = false;
  const float* scores;
  int64_t row_stride;
  const int32_t* lengths;  // may be null
  int32_t num_cols;

  __device__ __forceinline__ int count(int64_t row) const {
    if (lengths == nullptr) return num_cols;
    const int len = lengths[row];
    return len < 0 ? 0 : (len < num_cols ? len : num_cols);
  }

  template <int VEC>
  __device__ __forceinline__ void finish(int, const uint32_t*, uint32_t*, uint32_t*) const {}

  template <int VEC, int NV>
  __device__ __forceinline__ void load(int64_t row, int first, int C, uint32_t* bits, uint32_t* idv,
                                       uint32_t*) const {
    constexpr int kChunk = VEC * kWave;
    // the range covers whole VEC-wide loads (C rounded up stays inside the
    // row, whose width is a multiple of VEC); values past C are ignored
    const int span = (C + VEC - 1) / VEC * VEC;
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(scores + row * row_stride), 0, span * static_cast<int>(sizeof(float)),
        static_cast<int>(kBufferWord3));
    const int voff = first * static_cast<int>(sizeof(float));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int soff = v * kChunk * static_cast<int>(sizeof(float));
      if constexpr (VEC == 4) {
        const int4 x = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(src, voff, soff, kLoadPolicy));
        bits[4 * v] = x.x;
        bits[4 * v + 1] = x.y;
        bits[4 * v + 2] = x.z;
        bits[4 * v + 3] = x.w;
      } else if constexpr (VEC == 2) {
        const int2v x = __builtin_amdgcn_raw_buffer_load_b64(src, voff, soff, kLoadPolicy);
        bits[2 * v] = x.x;
        bits[2 * v + 1] = x.y;
      } else {
        bits[v] = __builtin_amdgcn_raw_buffer_load_b32(src, voff, soff, kLoadPolicy);
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) idv[v * VEC + j] = static_cast<uint32_t>(first + v * kChunk + j);
    }
  }
};

// ---------------------------------------------------------------------------
// Output sinks.  bind(row, k) gives the row's writer; store(keep, slot, bits,
// id) writes one output slot (a store with keep == false is dropped by the
// buffer range check), pad(slot) writes the padding candidate.
// ---------------------------------------------------------------------------

// (score bits, id) pairs, the candidate layout; padding is (-inf, INT32_MAX).
struct PairSink {
  dcp_topk_cand* out;
  int64_t row_stride;

  struct Row {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ void store(bool keep, uint32_t slot, uint32_t bits, uint32_t id) const {
      const int2v data = {static_cast<int>(bits), static_cast<int>(id)};
      __builtin_amdgcn_raw_buffer_store_b64(data, r, static_cast<int>(keep ? slot * 8u : kDropOffset), 0, kStorePolicy);
    }
    __device__ __forceinline__ void pad(uint32_t slot) const { store(true, slot, kPadBits, kPadId); }
  };

  __device__ __forceinline__ Row bind(int64_t row, int k) const {
    return Row{__builtin_amdgcn_make_buffer_rsrc(out + row * row_stride, 0, k * static_cast<int>(sizeof(dcp_topk_cand)),
                                                 static_cast<int>(kBufferWord3))};
  }
};

// Separate score and local-index arrays, the layout the pack step reads;
// padding is (-inf, -1), which the pack turns into its padding candidate.
struct SplitSink {
  float* scores;
  int32_t* idx;
  int64_t row_stride;

  struct Row {
    __amdgpu_buffer_rsrc_t s, i;
    __device__ __forceinline__ void store(bool keep, uint32_t slot, uint32_t bits, uint32_t id) const {
      const int off = static_cast<int>(keep ? slot * 4u : kDropOffset);
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(bits), s, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(id), i, off, 0, 0);
    }
    __device__ __forceinline__ void pad(uint32_t slot) const { store(true, slot, kPadBits, 0xFFFFFFFFu); }
  };

  __device__ __forceinline__ Row bind(int64_t row, int k) const {
    return Row{__builtin_amdgcn_make_buffer_rsrc(scores + row * row_stride, 0, k * static_cast<int>(sizeof(float)),
                                                 static_cast<int>(kBufferWord3)),
               __builtin_amdgcn_make_buffer_rsrc(idx + row * row_stride, 0, k * static_cast<int>(sizeof(int32_t)),
                                                 static_cast<int>(kBufferWord3))};
  }
};

template <int BLOCK, int VEC, int N, bool FULL, class Source, class Sink>
__global__ __launch_bounds__(BLOCK) void stable_topk_kernel(Source src, Sink sink, int32_t k) {
  static_assert(N <= 32 && N % VEC == 0, "flags are 32-bit masks");
  constexpr int NV = N / VEC;
  constexpr int kChunk = VEC * kWave;  // consecutive positions per chunk and wave
  __shared__ SelectLds<BLOCK> lds;
  // per-wave output staging: half of a wave's slots, at most 448, then one
  // write-only spare slot (the area has kWave slots past kStageCap so that the
  // wave's whole-row copy-out reads stay inside it when kStageCap < 64)
  constexpr int kStageCap = kWave * N / 2 < 448 ? kWave * N / 2 : 448;
  __shared__ uint2 stage[BLOCK / kWave][kStageCap + kWave];
  const unsigned long long t_start = phase_clock();  // stamp 0: the wave starts

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = blockIdx.x;
  const int C = src.count(row);
  const typename Sink::Row dst = sink.bind(row, k);

  // Wave w reads positions [w*64*N, (w+1)*64*N), 64*VEC consecutive ones per
  // load.
  const int first = w * kWave * N + VEC * lane;  // this thread's position in chunk 0
  uint32_t bits[N], idv[N], aux[2 * NV];

  // k >= C: every candidate is selected, in place, then padding (a branch
  // of its own from the start, so that none of its code is shared with, and
  // hoisted into, the selection path)
  if (k >= C) {
    src.template load<VEC, NV>(row, first, C, bits, idv, aux);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      src.template finish<VEC>(v, aux, bits, idv);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int p = first + v * kChunk + j;
        dst.store(p < C, static_cast<uint32_t>(p), bits[v * VEC + j], idv[v * VEC + j]);
      }
    }
    for (int slot = C + t; slot < k; slot += BLOCK) dst.pad(static_cast<uint32_t>(slot));
    return;
  }

  // 1. issue the row's loads before touching LDS: all of them, or, for a
  // source that loads chunk by chunk and rows of 8 or more chunks per wave,
  // the first half.  The other chunks' loads then go out in pass 0, each just
  // before an earlier chunk is counted: the waves pass the first barrier once
  // half of their loads are issued, and count while the rest are held back
  // by the memory system instead of waiting for the last load to issue
  // (measured: tie-heavy 16 rows 8.56 -> 8.11 us, decode 16 rows 6.00 ->
  // 5.89, short-context 7.49 -> 7.30, the 256-row batch unchanged; a quarter
  // or three quarters up front measured slower)
  constexpr int kEarly = Source::kChunkLoads && NV >= 8 ? NV / 2 : NV;  // chunks loaded up front
  const unsigned long long t_loads = phase_clock();  // stamp 1: arguments read, row loads about to issue
  if constexpr (kEarly < NV) {
#pragma unroll
    for (int v = 0; v < kEarly; ++v) src.template load_chunk<VEC>(row, first, C, v, bits, idv);
  } else {
    src.template load<VEC, NV>(row, first, C, bits, idv, aux);
  }

  // (the stamp slots' address is looked up while the loads are in flight)
  unsigned long long* const stamps = stamp_slots<BLOCK>(w);
  // clear the histograms while the loads are in flight; the key transform
  // stays after the barrier so that pass 0 starts on the first chunk while
  // later chunks are still arriving
  clear_words<BLOCK>(&lds.hist[0][0], 3 * kBins + 3 * kSmallBins + kPadWords, t);
  if (t < 4) lds.common[t] = (t & 1) ? ~0u : 0u;  // OR slots 0, AND slots ~0 (list_common_bits)
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  stamp(stamps, 2, lane);  // loads issued, LDS cleared, first barrier
  stamp_value(stamps, 0, lane, t_start);
  stamp_value(stamps, 1, lane, t_loads);

  // FULL: the row fills every slot (C == BLOCK*N); else the last are masked
  // out: item i is valid if its position, first + (i / VEC) * kChunk + i % VEC,
  // is below C, i.e. if i's offset is below C - first (a compare per use
  // instead of a mask held in a register)
  const int room = C - first;  // items of this thread are valid below this offset
  auto ok = [&](int i) -> bool {
    return FULL || (i / VEC) * kChunk + i % VEC < room;
  };
  auto valid_mask = [&]() -> uint32_t {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) m |= ok(i) ? 1u << i : 0u;
    return m;
  };

  // 2. pass 0: histogram of the top 11 bits; each item keeps its rank in its
  // bin.  Padding keys (-inf: empty shard slots, which can fill whole ranks)
  // would all hit one bin, and LDS atomics to one address serialise, so they
  // count into kPadWords words instead (by lane) and join their bin in the
  // digit search (and, if that bin is the threshold's, in the list).  Each
  // chunk is finished, transformed and counted right after the wait for its
  // own loads, so pass 0 runs while later chunks are still arriving (this
  // needs the k >= C path to be a branch of its own: code shared with it was
  // hoisted above its branch, with every load wait).
  uint32_t key[N];
  uint32_t rank_in_bin[N];
  uint32_t* pad_word = lds.padcnt + (lane % kPadWords);
  uint32_t* spare = lds.sink + lane;  // target of masked-out items
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (kEarly < NV) {
      if (i % VEC == 0 && i / VEC + kEarly < NV) {
        // the scheduling barriers keep the load at its place in the stream
        __builtin_amdgcn_sched_barrier(0);
        src.template load_chunk<VEC>(row, first, C, i / VEC + kEarly, bits, idv);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (i % VEC == 0) src.template finish<VEC>(i / VEC, aux, bits, idv);
    key[i] = score_key(bits[i]);
    uint32_t* target = key[i] == kPadKey ? pad_word : lds.hist[0] + (key[i] >> 21);
    if constexpr (!FULL) target = ok(i) ? target : spare;
    rank_in_bin[i] = lds_add(target);
  }
  stamp(stamps, 3, lane);  // pass-0 atomics issued
  lds_barrier();
  // padding keys counted in pass 0, in total and in the words before this lane's
  stamp(stamps, 4, lane);  // pass-0 barrier
  const uint4 pw0 = *reinterpret_cast<const uint4*>(lds.padcnt);
  const uint4 pw1 = *reinterpret_cast<const uint4*>(lds.padcnt + 4);
  const uint32_t pad_total = pw0.x + pw0.y + pw0.z + pw0.w + pw1.x + pw1.y + pw1.z + pw1.w;
  static_assert(kPadWords == 8, "two uint4 reads");
  Radix sk{0u, 0u, static_cast<uint32_t>(k), 0u};
  advance(sk, find_digit_pass0(lds.hist[0], sk.need, lane, kPadBin, pad_total), 21, 0x7FFu);
  stamp(stamps, 5, lane);  // digit search

  const uint32_t m = sk.count;  // items in the threshold bin
  bool tie = false, dup = false;
  Radix ik{0u, 0u, 0u, 0u};
  // 3. the threshold bin as a list: each of its items writes its (score bits,
  // id) pair, which sit in adjacent registers as loaded, at its pass-0 rank
  // (every other item writes to one shared dump slot, so the loop has no
  // per-item branch); the list passes recompute the keys of the few list items
  // (writing keys instead takes a register copy per item: large 7.60 vs 7.58
  // us, decode 16 rows 5.81 vs 5.78).  The list is built in a block of its own, ahead
  // of the choice between the list passes and the register passes, so that
  // the pass-0 ranks die before that branch (the scheduling barrier keeps the
  // compiler from merging the two blocks): each path then fits in 128 VGPRs,
  // and two 512-thread workgroups share a CU.
  if (m != sk.need && m <= static_cast<uint32_t>(kListCap)) {
    const uint32_t d0 = sk.prefix >> 21;
    if (d0 != kPadBin) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool in_bin = ok(i) && (key[i] >> 21) == d0;
        lds.list[in_bin ? rank_in_bin[i] : static_cast<uint32_t>(kListCap)] = make_uint2(bits[i], idv[i]);
      }
    } else {
      // padding keys were ranked per lane word: they follow the bin's other
      // items, word by word
      uint32_t pad_base = lds.hist[0][kPadBin];
#pragma unroll
      for (int j = 0; j < kPadWords; ++j) pad_base += j < lane % kPadWords ? lds.padcnt[j] : 0u;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool in_bin = ok(i) && (key[i] >> 21) == d0;
        const uint32_t slot = rank_in_bin[i] + (key[i] == kPadKey ? pad_base : 0u);
        lds.list[in_bin ? slot : static_cast<uint32_t>(kListCap)] = make_uint2(bits[i], idv[i]);
      }
    }
    lds_barrier();
  }
  __builtin_amdgcn_sched_barrier(0);
  stamp(stamps, 6, lane);  // list built
  if (m != sk.need && m <= kListCap) {
    // then list pass 0 counts the next 8 key bits
    const uint2* items = list_pass<BLOCK, 13, 8, false, true>(lds, 0, m, 0u, sk, t, lane);
    stamp(stamps, 7, lane);  // first list pass
    int q = 1;
    bool same_ids_known = false, resolved = false;
    uint32_t uor = 0u, uand = 0u;
    if (sk.count == m && m > sk.need) {
      // everything fell into one bin again: look for bits shared by the whole
      // list (identical scores, as on tie-heavy rows) and skip their passes
      uint32_t kor, kand;
      list_common_bits(lds, m, t, lane, kor, kand, uor, uand);
      same_ids_known = true;
      if (kor == kand) {  // every list item has the same key
        sk.prefix = kor;
        sk.mask = ~0u;
      }
    }
    // 4. the rest of the key threshold: once the chosen digit holds at most
    // kBucket items (the usual case for smooth scores, right after list pass
    // 0) it is finished by comparison, together with its id threshold if it
    // ties
    do {
      if (sk.count == sk.need || sk.mask == ~0u) break;
      if (sk.count <= static_cast<uint32_t>(kBucket)) {
        tie = few_rank(items, sk, ik, lane);
        resolved = true;
        break;
      }
      items = list_pass<BLOCK, 5, 8, false>(lds, q++, m, 0u, sk, t, lane);
      if (sk.count == sk.need) break;
      if (sk.count <= static_cast<uint32_t>(kBucket)) {
        tie = few_rank(items, sk, ik, lane);
        resolved = true;
        break;
      }
      list_pass<BLOCK, 0, 5, false>(lds, q++, m, 0u, sk, t, lane);
    } while (false);
    if (!resolved) {
      // 5. id tie-break over the list items with the threshold key (all score
      // bits are fixed now and sk.prefix is the full threshold key)
      tie = sk.count > sk.need;
      if (tie) {
        ik.need = sk.need;
        ik.count = sk.count;
        // 8-bit digits of ~id from the highest bit where the list items' ids
        // can differ: the bits above it are shared by every list item (so by
        // every tied item) and are fixed without a pass
        const uint32_t differ = same_ids_known ? (uor ^ uand) : ~0u;
        if (differ == 0u) {
          // every list item has the same id: the tied items are full
          // duplicates, and positions decide among them
          ik.prefix = uand;
          ik.mask = ~0u;
        } else {
          int hb = 31 - __builtin_clz(differ);
          if (hb < 31) {
            ik.mask = ~0u << (hb + 1);
            ik.prefix = uand & ik.mask;
          }
          for (;;) {  // at most 4 passes
            const int shift = hb >= 7 ? hb - 7 : 0;
            items = list_pass_ids(lds, q++, m, sk.prefix, ik, shift, hb - shift + 1, t, lane);
            if (ik.count == ik.need) break;
            if (ik.count <= static_cast<uint32_t>(kBucket)) {
              few_rank_ids(items, ik, lane);
              break;
            }
            if (shift == 0) break;
            hb = shift - 1;
          }
        }
      }
    }
    dup = tie && ik.count > ik.need;  // identical (key, id) pairs straddle the boundary
  } else if (m != sk.need) {
    // 3'. a bin too large for the list (at the threshold of a short row, the
    // padding keys of its empty slots): the bits shared by all of the bin's
    // items first, so a bin of identical keys needs no key pass and one of
    // identical (key, id) pairs no id pass either; then the remaining passes
    // over the registers, from the highest bit where the values differ
    const uint32_t d0 = sk.prefix >> 21;
    uint32_t a = 0u, b = ~0u, c = 0u, e = ~0u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool in_bin = ok(i) && (key[i] >> 21) == d0;
      a |= in_bin ? key[i] : 0u;
      b &= in_bin ? key[i] : ~0u;
      c |= in_bin ? ~idv[i] : 0u;
      e &= in_bin ? ~idv[i] : ~0u;
    }
    uint32_t kor, kand, uor, uand;
    block_common_bits(lds, lane, a, b, c, e, kor, kand, uor, uand);
    // register passes run on hist[p % 3] for p = 1, 2, ... in turn (the
    // rotation that clears each histogram two passes before its next use)
    int p = 1;
    if (kor == kand) {  // every item of the bin has the same key
      sk.prefix = kor;
      sk.mask = ~0u;
    } else {
      do {
        radix_pass<BLOCK, 10, 11, false>(lds, p++, key, valid_mask(), sk, t, lane);
        if (sk.count == sk.need) break;
        radix_pass<BLOCK, 0, 10, false>(lds, p++, key, valid_mask(), sk, t, lane);
      } while (false);
    }
    tie = sk.count > sk.need;
    if (tie) {
      // the tied items are some of the bin's, so the bits where all of the
      // bin's ids agree are fixed for them too
      ik.need = sk.need;
      ik.count = sk.count;
      const uint32_t differ = uor ^ uand;
      if (differ == 0u) {  // full duplicates: positions decide among them
        ik.prefix = uand;
        ik.mask = ~0u;
      } else {
        uint32_t tied = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) tied |= (ok(i) && key[i] == sk.prefix) ? (1u << i) : 0u;
        const int hb = 31 - __builtin_clz(differ);
        if (hb < 31) {
          ik.mask = ~0u << (hb + 1);
          ik.prefix = uand & ik.mask;
        }
        do {
          if (hb >= 21) {
            radix_pass<BLOCK, 21, 11, true>(lds, p++, idv, tied, ik, t, lane);
            if (ik.count == ik.need) break;
          }
          if (hb >= 10) {
            radix_pass<BLOCK, 10, 11, true>(lds, p++, idv, tied, ik, t, lane);
            if (ik.count == ik.need) break;
          }
          radix_pass<BLOCK, 0, 10, true>(lds, p++, idv, tied, ik, t, lane);
        } while (false);
      }
      dup = ik.count > ik.need;
    }
  }

  stamp(stamps, 8, lane);  // threshold resolved
  uint32_t duprank[N];
  if (dup) {
    uint32_t same[N];
#pragma unroll
    for (int i = 0; i < N; ++i) same[i] = (ok(i) && key[i] == sk.prefix && ~idv[i] == ik.prefix) ? 1u : 0u;
    position_rank<BLOCK, VEC, N>(same, lds.segment[0], duprank, lane, w);
  }
  uint32_t sel[N];
  if (!tie) {
    // common case: sk.mask covers the top bits and sk.prefix is zero below
    // them, so (key & mask) >= prefix is simply key >= prefix
#pragma unroll
    for (int i = 0; i < N; ++i) sel[i] = (ok(i) && key[i] >= sk.prefix) ? 1u : 0u;
  } else if (!dup) {
    // the tied items (key == threshold) are taken by complemented id; the id
    // passes leave ik.prefix zero below ik.mask, so the test is (key, ~id) >=
    // (threshold key, ik.prefix), one 64-bit compare instead of three
    // (tie-heavy 16 rows 8.08 -> 7.83 us, short-context 7.27 -> 7.12)
    const uint64_t th = (static_cast<uint64_t>(sk.prefix) << 32) | ik.prefix;
#pragma unroll
    for (int i = 0; i < N; ++i)
      sel[i] = (ok(i) && ((static_cast<uint64_t>(key[i]) << 32) | ~idv[i]) >= th) ? 1u : 0u;
  } else {
    // full duplicates of the threshold pair: the first ik.need by position
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t u = ~idv[i];
      const bool wins = u > ik.prefix || (u == ik.prefix && duprank[i] < ik.need);
      sel[i] = (ok(i) && (key[i] > sk.prefix || (key[i] == sk.prefix && wins))) ? 1u : 0u;
    }
  }

  // 5. stable compaction and store.  Wave w's selected items fill the output
  // slots [out_first, out_first + out_count) (its positions precede all later
  // waves'), so each wave stages its own items in its own LDS area at their
  // rank inside the wave (unselected items write to the area's spare slot, so
  // the loop has no per-item branch) while the waves' counts are exchanged,
  // then writes its range with consecutive stores.  A wave with more selected
  // items than its area stores every item at its rank from the registers.
  stamp(stamps, 9, lane);  // selection flags
  uint32_t rank[N];
  const uint32_t out_count = wave_rank<VEC, N>(sel, rank, lane);
  stamp(stamps, 10, lane);  // ranks
  if (lane == 0) lds.segment[1][w] = out_count;
  const bool staged = out_count <= static_cast<uint32_t>(kStageCap);  // wave-uniform
  if (staged) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t slot = sel[i] ? rank[i] : static_cast<uint32_t>(kStageCap);
      stage[w][slot] = make_uint2(bits[i], idv[i]);
    }
  }
  stamp(stamps, 11, lane);  // staging writes
  lds_barrier();
  const uint32_t out_first = waves_before<BLOCK>(lds.segment[1], w);
  stamp(stamps, 12, lane);  // count exchange
  if (staged) {
    // all reads first, then the stores of the copies that hold any of the
    // wave's items: a store whose lanes all fall past out_count would write
    // nothing but still cost its issue, so the copies past the count are
    // skipped by a wave-uniform branch (measured: large 7.65 -> 7.60 us,
    // short-context 7.13 -> 6.97); inside the last copy, lanes past out_count
    // hold stale values and their stores are dropped (the reads stay inside
    // the wave's kStageCap + 64 slots)
    constexpr int kCopies = (kStageCap + kWave - 1) / kWave;
    uint2 x[kCopies];
#pragma unroll
    for (int u = 0; u < kCopies; ++u) x[u] = stage[w][u * kWave + lane];
#pragma unroll
    for (int u = 0; u < kCopies; ++u) {
      if (static_cast<uint32_t>(u * kWave) >= out_count) break;  // wave-uniform
      const uint32_t e = static_cast<uint32_t>(u * kWave + lane);
      dst.store(e < out_count, out_first + e, x[u].x, x[u].y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst.store(sel[i] != 0u, out_first + rank[i], bits[i], idv[i]);
  }
  stamp(stamps, 13, lane);  // stores issued
}

// ---------------------------------------------------------------------------
// Split-row select, for batches of few rows: one workgroup per row leaves most
// CUs idle, so here `parts` workgroups share a row.  Workgroup s of a row takes
// its slice, the candidates [s*L, (s+1)*L), and the row's workgroups exchange
// what they need through the caller's workspace at two row barriers:
//   1. every slice's pass-0 histogram: after the barrier every workgroup sums
//      them and finds the threshold bin (the same one everywhere);
//   2. every slice's items of that bin, with their positions, appended to the
//      row's list: after the barrier every workgroup resolves the exact
//      threshold from the list (radix passes), and counts from the slices'
//      histograms and the list how many items the earlier slices select, so
//      that it knows its output offset without a third exchange.
// Then each workgroup writes its slice's selected items, in position order, at
// that offset.  The launch is cooperative (the runtime guarantees that every
// workgroup of the grid is resident), so the row barriers always complete;
// they still give up after a bounded number of polls.  The workspace's
// per-row counters start at zero and the last workgroup of a row to finish
// sets them back to zero.
// ---------------------------------------------------------------------------
constexpr int kSplitHist = kSplitHistWords;  // words per slice histogram: kBins counts, then the padding count
static_assert(kSplitHistWords == kBins + 8, "slice histogram layout");
constexpr int kSplitSpin = 1 << 20;    // polls of a row barrier before it gives up

struct SplitWorkspace {
  uint32_t* ctrl;   // per row: arrivals at barrier 1, at barrier 2, list length, finished workgroups
  uint32_t* hist;   // per row and slice: kSplitHist words
  uint2* list;      // per row: num_cand (key, id) entries
  uint32_t* pos;    // per row: num_cand positions
};

// Every thread of the workgroup: its global writes so far are visible to the
// row's other workgroups, and theirs, written before they arrived, to it.
// One thread arrives with a release add and polls with relaxed loads (an
// acquire load per poll would invalidate the caches on every poll), then
// takes one acquire fence; the workgroup barriers on either side order the
// other threads' writes before the arrival and their reads after the fence.
__device__ __forceinline__ void row_barrier(uint32_t* counter, uint32_t parts, int t) {
  __syncthreads();
  if (t == 0) {
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int spin = 0;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < parts && ++spin < kSplitSpin)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// A radix pass over the row's list in the workspace (the threshold bin's m
// items): the digit at SHIFT (BITS wide) of the keys (BY_ID false) or of the
// complemented ids of the items whose key is thr, among those that match st;
// hist[p % 3] rotation as in radix_pass.
template <int BLOCK, int SHIFT, int BITS, bool BY_ID>
__device__ __forceinline__ void split_list_pass(SelectLds<BLOCK>& lds, int p, const uint2* list, uint32_t m,
                                                uint32_t thr, Radix& st, int t, int lane) {
  constexpr int NB = 1 << BITS;
  constexpr uint32_t kDigitMask = NB - 1;
  uint32_t* hist = lds.hist[p % 3];
  for (uint32_t e = static_cast<uint32_t>(t); e < m; e += BLOCK) {
    const uint2 x = list[e];
    const uint32_t v = BY_ID ? ~x.y : x.x;
    if ((!BY_ID || x.x == thr) && (v & st.mask) == st.prefix) lds_add(hist + ((v >> SHIFT) & kDigitMask));
  }
  lds_barrier();
  clear_words<BLOCK>(lds.hist[(p + 2) % 3], kBins, t);
  advance(st, find_digit<NB>(hist, st.need, lane), SHIFT, kDigitMask);
}

template <int BLOCK, int VEC, int N>
__global__ __launch_bounds__(BLOCK) void split_select_kernel(const dcp_topk_cand* __restrict__ cand, int32_t num_cand,
                                                             int32_t k, int32_t parts, int32_t slice_len,
                                                             SplitWorkspace ws, dcp_topk_cand* __restrict__ out) {
  constexpr int NV = N / VEC;
  constexpr int kChunk = VEC * kWave;
  __shared__ SelectLds<BLOCK> lds;
  constexpr int kStageCap = kWave * N / 2 < 448 ? kWave * N / 2 : 448;
  __shared__ uint2 stage[BLOCK / kWave][kStageCap + kWave];

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = blockIdx.x / parts;
  const int s = static_cast<int>(blockIdx.x % parts);
  const int start = s * slice_len;  // the slice's first position in the row
  // its candidates: none when the slice starts at or past the row's end
  const int len = num_cand <= start ? 0 : (num_cand - start < slice_len ? num_cand - start : slice_len);
  uint32_t* ctrl = ws.ctrl + row * 4;
  uint32_t* hist_g = ws.hist + row * parts * kSplitHist;
  uint2* list = ws.list + row * num_cand;
  uint32_t* lpos = ws.pos + row * num_cand;
  const PairSink::Row dst = PairSink{out, k}.bind(row, k);

  // the slice's candidates: wave w holds [w*64*N, (w+1)*64*N) of the slice,
  // 64*VEC consecutive ones per load, like the one-workgroup kernel
  const int first = w * kWave * N + VEC * lane;
  const int room = len - first;  // this thread's items are valid below this offset
  auto ok = [&](int i) -> bool { return (i / VEC) * kChunk + i % VEC < room; };
  uint32_t bits[N], idv[N];
  {
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<dcp_topk_cand*>(cand + row * num_cand + start), 0,
        len * static_cast<int>(sizeof(dcp_topk_cand)), static_cast<int>(kBufferWord3));
    const int voff = first * static_cast<int>(sizeof(dcp_topk_cand));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int soff = v * kChunk * static_cast<int>(sizeof(dcp_topk_cand));
      if constexpr (VEC == 2) {
        const int4 x = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(src, voff, soff, kLoadPolicy));
        bits[2 * v] = x.x;
        idv[2 * v] = x.y;
        bits[2 * v + 1] = x.z;
        idv[2 * v + 1] = x.w;
      } else {
        const int2v x = __builtin_amdgcn_raw_buffer_load_b64(src, voff, soff, kLoadPolicy);
        bits[v] = x.x;
        idv[v] = x.y;
      }
    }
  }
  clear_words<BLOCK>(&lds.hist[0][0], 3 * kBins + 3 * kSmallBins + kPadWords, t);
  if (t < 4) lds.common[t] = (t & 1) ? ~0u : 0u;
  if (t < 3 * kMaxSplit) (&lds.slices[0][0])[t] = 0u;
  lds_barrier();

  // pass 0 over the slice (padding keys in per-lane words, as in the
  // one-workgroup kernel), then the slice's histogram to the workspace
  uint32_t key[N];
  uint32_t* pad_word = lds.padcnt + (lane % kPadWords);
  uint32_t* spare = lds.sink + lane;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    key[i] = score_key(bits[i]);
    uint32_t* target = key[i] == kPadKey ? pad_word : lds.hist[0] + (key[i] >> 21);
    lds_add(ok(i) ? target : spare);
  }
  lds_barrier();
  uint32_t* my_hist = hist_g + s * kSplitHist;
  for (int b = 4 * t; b < kBins; b += 4 * BLOCK)
    *reinterpret_cast<uint4*>(my_hist + b) = *reinterpret_cast<const uint4*>(lds.hist[0] + b);
  if (t == 0) {
    uint32_t pads = 0u;
#pragma unroll
    for (int j = 0; j < kPadWords; ++j) pads += lds.padcnt[j];
    my_hist[kBins] = pads;
  }
  row_barrier(ctrl + 0, static_cast<uint32_t>(parts), t);

  // the row's histogram: the sum of the slices'
  for (int b = 4 * t; b < kBins; b += 4 * BLOCK) {
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int q = 0; q < parts; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(hist_g + q * kSplitHist + b);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    *reinterpret_cast<uint4*>(lds.hist[0] + b) = acc;
  }
  uint32_t pad_total = 0u;
  for (int q = 0; q < parts; ++q) pad_total += hist_g[q * kSplitHist + kBins];
  pad_total = uniform(pad_total);
  lds_barrier();
  Radix sk{0u, 0u, static_cast<uint32_t>(k), 0u};
  advance(sk, find_digit_pass0(lds.hist[0], sk.need, lane, kPadBin, pad_total), 21, 0x7FFu);
  const uint32_t d0 = sk.prefix >> 21;
  const bool listed = sk.count != sk.need;  // the threshold is inside bin d0: its items go to the list

  // this slice's items of bin d0 to the row's list (one global atomic per
  // wave for the wave's range)
  if (listed) {
    uint32_t mine = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) mine += static_cast<uint32_t>(__popcll(__ballot(ok(i) && (key[i] >> 21) == d0)));
    uint32_t base = 0u;
    if (lane == 0) base = __hip_atomic_fetch_add(ctrl + 2, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    base = lane_of(base, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool in = ok(i) && (key[i] >> 21) == d0;
      const uint64_t m = __ballot(in);
      const uint32_t e = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (in && e < static_cast<uint32_t>(num_cand)) {  // (always, unless the workspace was not zeroed)
        list[e] = make_uint2(key[i], idv[i]);
        lpos[e] = static_cast<uint32_t>(start + first + (i / VEC) * kChunk + i % VEC);
      }
      base += static_cast<uint32_t>(__popcll(m));
    }
  }
  row_barrier(ctrl + 1, static_cast<uint32_t>(parts), t);

  // the exact threshold from the list: the bits its items share first (a
  // list of identical keys needs no key pass, one of identical (key, id)
  // pairs, such as padding, no id pass), then radix passes from the highest
  // bit where they differ
  bool tie = false, dup = false;
  Radix ik{0u, 0u, 0u, 0u};
  // (a workspace that was not zeroed gives wrong results, never an access
  // outside it: the list length and the slice indexes are clamped)
  const uint32_t m = listed ? min(uniform(__hip_atomic_load(ctrl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)),
                                  static_cast<uint32_t>(num_cand))
                            : 0u;
  if (listed) {
    uint32_t a = 0u, b = ~0u, c = 0u, e = ~0u;
    for (uint32_t q = static_cast<uint32_t>(t); q < m; q += BLOCK) {
      const uint2 x = list[q];
      a |= x.x;
      b &= x.x;
      c |= ~x.y;
      e &= ~x.y;
    }
    uint32_t kor, kand, uor, uand;
    block_common_bits(lds, lane, a, b, c, e, kor, kand, uor, uand);
    int p = 1;
    if (kor == kand) {
      sk.prefix = kor;
      sk.mask = ~0u;
    } else {
      do {
        split_list_pass<BLOCK, 10, 11, false>(lds, p++, list, m, 0u, sk, t, lane);
        if (sk.count == sk.need) break;
        split_list_pass<BLOCK, 0, 10, false>(lds, p++, list, m, 0u, sk, t, lane);
      } while (false);
    }
    tie = sk.count > sk.need;
    if (tie) {
      ik.need = sk.need;
      ik.count = sk.count;
      const uint32_t differ = uor ^ uand;
      if (differ == 0u) {
        ik.prefix = uand;
        ik.mask = ~0u;
      } else {
        const int hb = 31 - __builtin_clz(differ);
        if (hb < 31) {
          ik.mask = ~0u << (hb + 1);
          ik.prefix = uand & ik.mask;
        }
        do {
          if (hb >= 21) {
            split_list_pass<BLOCK, 21, 11, true>(lds, p++, list, m, sk.prefix, ik, t, lane);
            if (ik.count == ik.need) break;
          }
          if (hb >= 10) {
            split_list_pass<BLOCK, 10, 11, true>(lds, p++, list, m, sk.prefix, ik, t, lane);
            if (ik.count == ik.need) break;
          }
          split_list_pass<BLOCK, 0, 10, true>(lds, p++, list, m, sk.prefix, ik, t, lane);
        } while (false);
      }
      dup = ik.count > ik.need;
    }
  }

  // per slice: keys above bin d0 (from the slices' histograms), selected keys
  // of bin d0 other than full duplicates, and full duplicates (from the list)
  const uint32_t thr = sk.prefix;
  auto selected = [&](uint32_t kk, uint32_t u) -> bool {  // not counting full duplicates
    if (!tie) return kk >= thr;
    return kk > thr || (kk == thr && (dup ? u > ik.prefix : u >= ik.prefix));
  };
  // wave q counts slice q's keys above bin d0 (and, when the whole bin is
  // taken, the bin itself); padding keys count here unless they are listed
  if (w < parts) {
    const uint32_t* h = hist_g + w * kSplitHist;
    uint32_t above = 0u;
    for (int b = lane; b < kBins; b += kWave) above += static_cast<uint32_t>(b) > d0 || (!listed && b == d0) ? h[b] : 0u;
    above = lane_of(wave_inclusive_scan(above, lane), kWave - 1);
    if (kPadBin > d0 || (kPadBin == d0 && !listed)) above += h[kBins];
    if (lane == 0) lds.slices[0][w] = above;
  }
  for (uint32_t q = static_cast<uint32_t>(t); q < m; q += BLOCK) {
    const uint2 x = list[q];
    const uint32_t sq = min(lpos[q] / static_cast<uint32_t>(slice_len), static_cast<uint32_t>(kMaxSplit - 1));
    const uint32_t u = ~x.y;
    if (selected(x.x, u)) lds_add(&lds.slices[1][sq]);
    if (dup && x.x == thr && u == ik.prefix) lds_add(&lds.slices[2][sq]);
  }
  lds_barrier();
  uint32_t out_base = 0u, dup_before = 0u;
  for (int q = 0; q < s; ++q) {
    const uint32_t dq = lds.slices[2][q];
    const uint32_t left = ik.need > dup_before ? ik.need - dup_before : 0u;  // duplicates still to take
    out_base += lds.slices[0][q] + lds.slices[1][q] + (dup ? (dq < left ? dq : left) : 0u);
    dup_before += dq;
  }
  out_base = uniform(out_base);
  dup_before = uniform(dup_before);

  // this slice's selection and its compaction, as in the one-workgroup kernel
  uint32_t sel[N];
  if (dup) {
    uint32_t same[N], duprank[N];
#pragma unroll
    for (int i = 0; i < N; ++i) same[i] = (ok(i) && key[i] == thr && ~idv[i] == ik.prefix) ? 1u : 0u;
    position_rank<BLOCK, VEC, N>(same, lds.segment[0], duprank, lane, w);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t u = ~idv[i];
      const bool wins = u > ik.prefix || (u == ik.prefix && dup_before + duprank[i] < ik.need);
      sel[i] = (ok(i) && (key[i] > thr || (key[i] == thr && wins))) ? 1u : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) sel[i] = (ok(i) && selected(key[i], ~idv[i])) ? 1u : 0u;
  }
  uint32_t rank[N];
  const uint32_t out_count = wave_rank<VEC, N>(sel, rank, lane);
  if (lane == 0) lds.segment[1][w] = out_count;
  const bool staged = out_count <= static_cast<uint32_t>(kStageCap);
  if (staged) {
#pragma unroll
    for (int i = 0; i < N; ++i) stage[w][sel[i] ? rank[i] : static_cast<uint32_t>(kStageCap)] = make_uint2(bits[i], idv[i]);
  }
  lds_barrier();
  const uint32_t out_first = out_base + waves_before<BLOCK>(lds.segment[1], w);
  if (staged) {
    constexpr int kCopies = (kStageCap + kWave - 1) / kWave;
    uint2 x[kCopies];
#pragma unroll
    for (int u = 0; u < kCopies; ++u) x[u] = stage[w][u * kWave + lane];
#pragma unroll
    for (int u = 0; u < kCopies; ++u) {
      if (static_cast<uint32_t>(u * kWave) >= out_count) break;  // wave-uniform
      const uint32_t e = static_cast<uint32_t>(u * kWave + lane);
      dst.store(e < out_count, out_first + e, x[u].x, x[u].y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst.store(sel[i] != 0u, out_first + rank[i], bits[i], idv[i]);
  }

  // the last workgroup of the row to finish resets the row's counters
  __syncthreads();
  if (t == 0 && __hip_atomic_fetch_add(ctrl + 3, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                    static_cast<uint32_t>(parts) - 1u) {
    ctrl[0] = 0u;
    ctrl[1] = 0u;
    ctrl[2] = 0u;
    __hip_atomic_store(ctrl + 3, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// full: every row has exactly BLOCK*N candidates, so no item is masked out
template <int BLOCK, int VEC, int N, class Source, class Sink>
hipError_t launch(const Source& src, const Sink& sink, bool uniform_rows, int32_t rows, int32_t num_cand, int32_t k,
                  hipStream_t stream) {
  Source a = src;
  Sink b = sink;
  void* args[] = {&a, &b, &k};
  const void* fn = uniform_rows && num_cand == BLOCK * N
                       ? reinterpret_cast<const void*>(&stable_topk_kernel<BLOCK, VEC, N, true, Source, Sink>)
                       : reinterpret_cast<const void*>(&stable_topk_kernel<BLOCK, VEC, N, false, Source, Sink>);
  return hipLaunchKernel(fn, dim3(rows), dim3(BLOCK), args, 0, stream);
}

// 256 threads up to 2048 candidates, 512 above (1024 for the rows past 8192
// noted below); the smallest item count per thread that covers the row.
// VEC 1 and 2:
template <int VEC, class Source, class Sink>
hipError_t launch_sized_narrow(const Source& src, const Sink& sink, bool u, int32_t rows, int32_t num_cand,
                               int32_t k, hipStream_t stream) {
  constexpr int kSmall = 256 * VEC;  // positions covered by 256 threads with one chunk
  if (num_cand <= kSmall) return launch<256, VEC, VEC>(src, sink, u, rows, num_cand, k, stream);
  if (num_cand <= 2 * kSmall) return launch<256, VEC, 2 * VEC>(src, sink, u, rows, num_cand, k, stream);
  if (num_cand <= 4 * kSmall) return launch<256, VEC, 4 * VEC>(src, sink, u, rows, num_cand, k, stream);
  if (num_cand <= 2048) return launch<256, VEC, 8>(src, sink, u, rows, num_cand, k, stream);
  if (num_cand <= 4096) return launch<512, VEC, 8>(src, sink, u, rows, num_cand, k, stream);
  if (num_cand <= 8192) return launch<512, VEC, 16>(src, sink, u, rows, num_cand, k, stream);
  if constexpr (std::is_same<Source, GatheredSource>::value) {
    // rows of 8192 to 16384: a full 16384-candidate row keeps 512 threads x
    // 32 items; a partial row takes 1024 threads x 16 items, at 4 waves per
    // SIMD where the partial-row 32-item kernel has 2 (2048 rows x 12000,
    // k 3000: 83.5 -> 77.4 us; 16 rows x 16384 at 1024 x 16: 8.20 -> 8.88 us)
    if (!(u && num_cand == 512 * 32)) return launch<1024, VEC, 16>(src, sink, u, rows, num_cand, k, stream);
  }
  return launch<512, VEC, 32>(src, sink, u, rows, num_cand, k, stream);
}

// Any VEC (VEC 4: 256 consecutive positions per wave load).
template <int VEC, class Source, class Sink>
hipError_t launch_sized(const Source& src, const Sink& sink, bool uniform_rows, int32_t rows, int32_t num_cand,
                        int32_t k, hipStream_t stream) {
  const bool u = uniform_rows;
  if constexpr (VEC == 4) {
    if (num_cand <= 1024) return launch<256, 4, 4>(src, sink, u, rows, num_cand, k, stream);
    if (num_cand <= 2048) return launch<256, 4, 8>(src, sink, u, rows, num_cand, k, stream);
    if (num_cand <= 4096) return launch<512, 4, 8>(src, sink, u, rows, num_cand, k, stream);
    if (num_cand <= 8192) return launch<512, 4, 16>(src, sink, u, rows, num_cand, k, stream);
    // more than 8192: 1024 threads x 16 items (4 waves per SIMD; 512 x 32
    // has 2: fused merge 256 rows of DCP 8 x 2048 14.6 -> 12.6 us, 2048 rows
    // of DCP 6 x 2048 101.3 -> 88.5 us; local top-K with per-row lengths,
    // 64 x 16384 9.91 -> 8.85 us, 2048 x 12000 72.9 -> 61.0 us)
    return launch<1024, 4, 16>(src, sink, u, rows, num_cand, k, stream);
  } else {
    return launch_sized_narrow<VEC>(src, sink, u, rows, num_cand, k, stream);
  }
}

}  // namespace

hipError_t launch_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, dcp_topk_cand* out,
                         hipStream_t stream) {
  const GatheredSource src{cand, num_cand};
  const PairSink sink{out, k};
  if ((num_cand % 2 == 0) && (reinterpret_cast<uintptr_t>(cand) % 16 == 0))
    return launch_sized<2>(src, sink, true, rows, num_cand, k, stream);
  return launch_sized<1>(src, sink, true, rows, num_cand, k, stream);
}

hipError_t launch_fused(const FusedRanks& ranks, int32_t dcp, int32_t rows, int32_t local_k, int32_t k,
                        dcp_topk_cand* out, hipStream_t stream) {
  const PairSink sink{out, k};
  if (dcp * local_k == 0)  // no candidates: every slot is padding, nothing is read
    return launch_sized<1>(GatheredSource{nullptr, 0}, sink, true, rows, 0, k, stream);
  const RankSource src{ranks, local_k, dcp * local_k, dcp - 1};
  // the widest load every rank's arrays allow: VEC consecutive slots per lane
  // need local_k to be a multiple of 64*VEC and 4*VEC-byte aligned arrays
  auto fits = [&](int vec) {
    bool ok = local_k % (vec * kWave) == 0;
    for (int r = 0; r < dcp; ++r)
      ok = ok && reinterpret_cast<uintptr_t>(ranks.rank[r].scores) % (4 * vec) == 0 &&
           reinterpret_cast<uintptr_t>(ranks.rank[r].idx) % (4 * vec) == 0;
    return ok;
  };
  if (fits(4)) return launch_sized<4>(src, sink, true, rows, dcp * local_k, k, stream);
  if (fits(2)) return launch_sized<2>(src, sink, true, rows, dcp * local_k, k, stream);
  return launch_sized<1>(src, sink, true, rows, dcp * local_k, k, stream);
}

hipError_t launch_local(const float* scores, int64_t score_row_stride, const int32_t* lengths, int32_t rows,
                        int32_t num_cols, int32_t k, float* out_scores, int32_t* out_idx, int64_t out_row_stride,
                        hipStream_t stream) {
  const DenseSource src{scores, score_row_stride, lengths, num_cols};
  const SplitSink sink{out_scores, out_idx, out_row_stride};
  const bool uniform_rows = lengths == nullptr;
  auto fits = [&](int vec) {
    return num_cols % vec == 0 && score_row_stride % vec == 0 && reinterpret_cast<uintptr_t>(scores) % (4 * vec) == 0;
  };
  if (fits(4)) return launch_sized<4>(src, sink, uniform_rows, rows, num_cols, k, stream);
  if (fits(2)) return launch_sized<2>(src, sink, uniform_rows, rows, num_cols, k, stream);
  return launch_sized<1>(src, sink, uniform_rows, rows, num_cols, k, stream);
}

namespace {

template <int VEC, int N>
hipError_t launch_split_sized(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, int32_t parts,
                              int32_t slice_len, const SplitWorkspace& ws, dcp_topk_cand* out, hipStream_t stream) {
  auto kernel = split_select_kernel<512, VEC, N>;
  // every workgroup of the grid must be resident at once (the row barriers
  // wait for all of a row's workgroups); checked here rather than left to the
  // runtime
  int device = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 512, 0);
  if (e != hipSuccess) return e;
  if (static_cast<int64_t>(rows) * parts > static_cast<int64_t>(cus) * per_cu) return hipErrorCooperativeLaunchTooLarge;
  void* args[] = {const_cast<dcp_topk_cand**>(&cand), &num_cand, &k, &parts, &slice_len,
                  const_cast<SplitWorkspace*>(&ws), &out};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<uint32_t>(rows * parts)),
                                    dim3(512), args, 0, stream);
}

template <int VEC>
hipError_t launch_split_vec(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, int32_t parts,
                            int32_t slice_len, const SplitWorkspace& ws, dcp_topk_cand* out, hipStream_t stream) {
  if (slice_len <= 512 * 4) return launch_split_sized<VEC, 4>(cand, rows, num_cand, k, parts, slice_len, ws, out, stream);
  static_assert(kSplitMaxSlice == 512 * 16, "the widest split kernel holds 16 items per thread");
  if (slice_len <= 512 * 8) return launch_split_sized<VEC, 8>(cand, rows, num_cand, k, parts, slice_len, ws, out, stream);
  return launch_split_sized<VEC, 16>(cand, rows, num_cand, k, parts, slice_len, ws, out, stream);
}

}  // namespace

hipError_t launch_select_split(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, int32_t parts,
                               void* workspace, dcp_topk_cand* out, hipStream_t stream) {
  const SplitLayout l = split_layout(rows, num_cand, parts);
  char* base = static_cast<char*>(workspace);
  const SplitWorkspace ws{reinterpret_cast<uint32_t*>(base + l.ctrl), reinterpret_cast<uint32_t*>(base + l.hist),
                          reinterpret_cast<uint2*>(base + l.list), reinterpret_cast<uint32_t*>(base + l.pos)};
  const int32_t slice_len = static_cast<int32_t>(split_slice_len(num_cand, parts));
  if ((num_cand % 2 == 0) && (reinterpret_cast<uintptr_t>(cand) % 16 == 0))
    return launch_split_vec<2>(cand, rows, num_cand, k, parts, slice_len, ws, out, stream);
  return launch_split_vec<1>(cand, rows, num_cand, k, parts, slice_len, ws, out, stream);
}

}  // namespace dcptopk

#if DCPTOPK_PHASE_STAMPS
// Copies the phase stamps of the launches since the last call out, then
// clears them (diagnostic build only; synchronous).  bytes <=
// sizeof(phase_stamps); the stamps of workgroup b, wave slot s (0: first wave,
// 1: last wave) are the 16 words from (b * 2 + s) * 16; a phase the kernel did
// not pass reads 0.
extern "C" __attribute__((visibility("default"))) int dcptopk_phase_stamps(void* host, size_t bytes) {
  if (bytes > sizeof(dcptopk::phase_stamps)) return -1;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(host, HIP_SYMBOL(dcptopk::phase_stamps), bytes, 0, hipMemcpyDeviceToHost);
  void* addr = nullptr;
  if (e == hipSuccess) e = hipGetSymbolAddress(&addr, HIP_SYMBOL(dcptopk::phase_stamps));
  if (e == hipSuccess) e = hipMemset(addr, 0, sizeof(dcptopk::phase_stamps));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return static_cast<int>(e);
}
#endif
