// Internal launchers of libdcptopk (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libdcptopk.h"

namespace dcptopk {

// Enqueue the stable top-K select over `rows` rows of `num_cand` candidates.
// Arguments are already validated: rows >= 1, 1 <= k, 0 <= num_cand <=
// DCP_TOPK_MAX_CANDIDATES, 8-byte aligned non-overlapping buffers.
hipError_t launch_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k,
                         dcp_topk_cand* out, hipStream_t stream);

// Split-row select: the caller's workspace, per row, holds four counters, one
// pass-0 histogram per slice (kSplitHistWords words: the 2048 bin counts, then
// the slice's padding count and 7 spare words), and the row's threshold-bin
// list (num_cand (key, id) pairs and num_cand positions).  Regions start on
// 256-byte boundaries.
constexpr int kSplitMaxParts = 8;
constexpr int kSplitHistWords = 2048 + 8;
constexpr int kSplitMaxSlice = 8192;  // most candidates one workgroup of a split row holds

struct SplitLayout {
  size_t ctrl, hist, list, pos, bytes;  // byte offsets of the regions, total bytes
};

inline size_t split_round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline SplitLayout split_layout(int64_t rows, int64_t num_cand, int64_t parts) {
  SplitLayout l;
  l.ctrl = 0;
  l.hist = split_round_up(static_cast<size_t>(rows) * 4 * sizeof(uint32_t));
  l.list = l.hist + split_round_up(static_cast<size_t>(rows * parts) * kSplitHistWords * sizeof(uint32_t));
  l.pos = l.list + split_round_up(static_cast<size_t>(rows * num_cand) * 2 * sizeof(uint32_t));
  l.bytes = l.pos + split_round_up(static_cast<size_t>(rows * num_cand) * sizeof(uint32_t));
  return l;
}

// Candidates per slice when a row of num_cand is split `parts` ways: the
// even share rounded up to a multiple of 64.
inline int64_t split_slice_len(int64_t num_cand, int64_t parts) {
  return ((num_cand + parts - 1) / parts + 63) / 64 * 64;
}

// Enqueue the split-row select (one cooperative launch of rows * parts
// workgroups).  Arguments are already validated: 1 <= parts <=
// kSplitMaxParts, 1 <= k < num_cand, split_slice_len(num_cand, parts) <=
// kSplitMaxSlice, a workspace of split_layout(...).bytes bytes, 256-byte
// aligned, whose counters are zero.  Returns hipErrorCooperativeLaunchTooLarge
// when the grid cannot be resident at once.
hipError_t launch_select_split(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, int32_t parts,
                               void* workspace, dcp_topk_cand* out, hipStream_t stream);

// One rank's inputs to the pack kernel.
struct PackRank {
  const float* scores;
  const int32_t* idx;
  const int32_t* row_starts;
  int32_t rank_offset;
};

// Most ranks one pack launch handles; larger DCP groups take several launches.
constexpr int kMaxPackRanks = 8;

// Most ranks the fused merge reads in one launch (the ranks travel in the
// kernel's arguments).
constexpr int kMaxFusedRanks = DCP_TOPK_FUSED_MAX_RANKS;

struct FusedRanks {
  PackRank rank[kMaxFusedRanks];
};

// Enqueue the fused merge: select straight from the ranks' local arrays
// (contiguous rows of local_k), as if they had been packed into a (rows,
// dcp*local_k) buffer.  Arguments are already validated: 1 <= dcp <=
// kMaxFusedRanks, local_k a multiple of 64, dcp*local_k <=
// DCP_TOPK_MAX_CANDIDATES.
hipError_t launch_fused(const FusedRanks& ranks, int32_t dcp, int32_t rows, int32_t local_k, int32_t k,
                        dcp_topk_cand* out, hipStream_t stream);

// Enqueue the local top-K: per row, the k best of the first lengths[row] (all
// num_cols if lengths is null) columns, ids = columns, into separate score and
// index arrays.  Arguments are already validated.
hipError_t launch_local(const float* scores, int64_t score_row_stride, const int32_t* lengths, int32_t rows,
                        int32_t num_cols, int32_t k, float* out_scores, int32_t* out_idx, int64_t out_row_stride,
                        hipStream_t stream);

// Enqueue the pack of `nranks` (<= kMaxPackRanks) ranks: rank r's row t goes to
// dst + t*dst_row_stride + r*local_k.  Arguments are already validated.
hipError_t launch_pack(const PackRank* ranks, int nranks, int64_t src_row_stride, int32_t rows,
                       int32_t local_k, dcp_topk_cand* dst, int64_t dst_row_stride, hipStream_t stream);

// Checks of a chunked merge's shape and host arrays (every check of
// dcp_topk_merge_chunked that does not involve the workspace or the output).
// *nothing_to_do is set when rows == 0.
int check_merge_shape(const float* const* local_scores, const int32_t* const* local_idx,
                      const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp, int32_t rows,
                      int32_t local_k, int32_t k, bool* nothing_to_do);

// The rest of the chunked merge once its shape and workspace are valid: the
// output and rank-array checks (nothing may overlap the workspace's
// dcp_topk_merge_workspace_bytes(rows, dcp, local_k) bytes or the output),
// then, per DCP_TOPK_MERGE_ROWS-row chunk, the pack of every rank into the
// workspace and the select of the chunk into `out`.  Returns a status code.
int merge_chunks(const float* const* local_scores, const int32_t* const* local_idx, const int32_t* const* row_starts,
                 const int32_t* rank_offsets, int32_t dcp, int32_t rows, int32_t local_k, int32_t k, void* workspace,
                 dcp_topk_cand* out, hipStream_t stream);

}  // namespace dcptopk
