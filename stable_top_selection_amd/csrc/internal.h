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

// One rank's inputs to the pack kernel.
struct PackRank {
  const float* scores;
  const int32_t* idx;
  const int32_t* row_starts;
  int32_t rank_offset;
};

// Most ranks one pack launch handles; larger DCP groups take several launches.
constexpr int kMaxPackRanks = 8;

// Enqueue the pack of `nranks` (<= kMaxPackRanks) ranks: rank r's row t goes to
// dst + t*dst_row_stride + r*local_k.  Arguments are already validated.
hipError_t launch_pack(const PackRank* ranks, int nranks, int64_t src_row_stride, int32_t rows,
                       int32_t local_k, dcp_topk_cand* dst, int64_t dst_row_stride, hipStream_t stream);

}  // namespace dcptopk
