// C ABI of libdcptopk: argument checks, launch dispatch and the chunked merge.
//
// Every check runs before anything is enqueued; no entry point allocates,
// synchronises or keeps state.
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "internal.h"
#include "libdcptopk.h"

namespace {

constexpr size_t kCandBytes = sizeof(dcp_topk_cand);
static_assert(sizeof(dcp_topk_cand) == 8, "packed candidate is 8 bytes");

struct Span {
  uintptr_t begin;
  uintptr_t bytes;
};

bool overlap(Span a, Span b) {
  return a.bytes > 0 && b.bytes > 0 && a.begin < b.begin + b.bytes && b.begin < a.begin + a.bytes;
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Bytes covered by `rows` rows of `width` elements of `elem` bytes at `stride`
// elements per row; false on overflow.
bool strided_span(const void* p, int64_t rows, int64_t width, int64_t stride, size_t elem, Span* out) {
  if (rows <= 0 || width <= 0) {
    *out = {reinterpret_cast<uintptr_t>(p), 0};
    return true;
  }
  const unsigned __int128 n = static_cast<unsigned __int128>(rows - 1) * static_cast<uint64_t>(stride) +
                              static_cast<uint64_t>(width);
  const unsigned __int128 b = n * elem;
  if (b > (static_cast<unsigned __int128>(1) << 62)) return false;
  *out = {reinterpret_cast<uintptr_t>(p), static_cast<uintptr_t>(b)};
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DCP_TOPK_OK : DCP_TOPK_EHIP; }

int check_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, const dcp_topk_cand* out) {
  if (rows < 0 || num_cand < 0 || k < 1) return DCP_TOPK_EINVAL;
  if (rows == 0) return DCP_TOPK_OK;
  if (out == nullptr || (num_cand > 0 && cand == nullptr)) return DCP_TOPK_EINVAL;
  if (!aligned(out, kCandBytes) || (cand != nullptr && !aligned(cand, kCandBytes))) return DCP_TOPK_EINVAL;
  if (num_cand > DCP_TOPK_MAX_CANDIDATES || k > DCP_TOPK_MAX_CANDIDATES || rows > DCP_TOPK_MAX_ROWS)
    return DCP_TOPK_EUNSUPPORTED;
  Span in_span, out_span;
  if (!strided_span(cand, rows, num_cand, num_cand, kCandBytes, &in_span)) return DCP_TOPK_EINVAL;
  if (!strided_span(out, rows, k, k, kCandBytes, &out_span)) return DCP_TOPK_EINVAL;
  if (overlap(in_span, out_span)) return DCP_TOPK_EINVAL;
  return DCP_TOPK_OK;
}

int check_pack(const float* scores, const int32_t* idx, int64_t src_row_stride, const int32_t* row_starts,
               int32_t rows, int32_t local_k, const dcp_topk_cand* dst, int64_t dst_row_stride) {
  if (rows < 0 || local_k < 0) return DCP_TOPK_EINVAL;
  if (rows == 0 || local_k == 0) return DCP_TOPK_OK;
  if (scores == nullptr || idx == nullptr || row_starts == nullptr || dst == nullptr) return DCP_TOPK_EINVAL;
  if (src_row_stride < local_k || dst_row_stride < local_k) return DCP_TOPK_EINVAL;
  if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(row_starts, 4) || !aligned(dst, kCandBytes))
    return DCP_TOPK_EINVAL;
  if (rows > DCP_TOPK_MAX_ROWS) return DCP_TOPK_EUNSUPPORTED;
  Span s, i, r, d;
  if (!strided_span(scores, rows, local_k, src_row_stride, 4, &s) ||
      !strided_span(idx, rows, local_k, src_row_stride, 4, &i) || !strided_span(row_starts, rows, 1, 1, 4, &r) ||
      !strided_span(dst, rows, local_k, dst_row_stride, kCandBytes, &d))
    return DCP_TOPK_EINVAL;
  if (overlap(d, s) || overlap(d, i) || overlap(d, r)) return DCP_TOPK_EINVAL;
  return DCP_TOPK_OK;
}

// Rank r's local arrays (rows x local_k, contiguous rows) and row starts:
// non-null, 4-byte aligned, disjoint from every span in `outputs`.
int check_ranks(const float* const* local_scores, const int32_t* const* local_idx, const int32_t* const* row_starts,
                int32_t dcp, int32_t rows, int32_t local_k, const Span* outputs, int n_outputs) {
  for (int r = 0; r < dcp; ++r) {
    const float* sc = local_scores[r];
    const int32_t* ix = local_idx[r];
    const int32_t* rs = row_starts[r];
    if (sc == nullptr || ix == nullptr || rs == nullptr) return DCP_TOPK_EINVAL;
    if (!aligned(sc, 4) || !aligned(ix, 4) || !aligned(rs, 4)) return DCP_TOPK_EINVAL;
    Span s, i, rsp;
    if (!strided_span(sc, rows, local_k, local_k, 4, &s) || !strided_span(ix, rows, local_k, local_k, 4, &i) ||
        !strided_span(rs, rows, 1, 1, 4, &rsp))
      return DCP_TOPK_EINVAL;
    for (int o = 0; o < n_outputs; ++o)
      if (overlap(outputs[o], s) || overlap(outputs[o], i) || overlap(outputs[o], rsp)) return DCP_TOPK_EINVAL;
  }
  return DCP_TOPK_OK;
}

}  // namespace

namespace dcptopk {

int check_merge_shape(const float* const* local_scores, const int32_t* const* local_idx,
                      const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp, int32_t rows,
                      int32_t local_k, int32_t k, bool* nothing_to_do) {
  *nothing_to_do = false;
  if (dcp < 1 || rows < 0 || local_k < 0 || k < 1) return DCP_TOPK_EINVAL;
  if (local_scores == nullptr || local_idx == nullptr || row_starts == nullptr || rank_offsets == nullptr)
    return DCP_TOPK_EINVAL;
  if (static_cast<int64_t>(dcp) * local_k > DCP_TOPK_MAX_CANDIDATES || k > DCP_TOPK_MAX_CANDIDATES)
    return DCP_TOPK_EUNSUPPORTED;
  *nothing_to_do = rows == 0;
  return DCP_TOPK_OK;
}

int merge_chunks(const float* const* local_scores, const int32_t* const* local_idx, const int32_t* const* row_starts,
                 const int32_t* rank_offsets, int32_t dcp, int32_t rows, int32_t local_k, int32_t k, void* workspace,
                 dcp_topk_cand* out, hipStream_t stream) {
  const int32_t num_cand = dcp * local_k;
  const size_t need = dcp_topk_merge_workspace_bytes(rows, dcp, local_k);
  if (out == nullptr || !aligned(out, kCandBytes)) return DCP_TOPK_EINVAL;
  Span ws{reinterpret_cast<uintptr_t>(workspace), need};
  Span o;
  if (!strided_span(out, rows, k, k, kCandBytes, &o)) return DCP_TOPK_EINVAL;
  if (overlap(ws, o)) return DCP_TOPK_EINVAL;
  // The workspace holds one chunk (at most DCP_TOPK_MERGE_ROWS rows); the
  // inputs span all rows.
  if (local_k > 0) {
    const Span outputs[2] = {o, ws};
    const int st = check_ranks(local_scores, local_idx, row_starts, dcp, rows, local_k, outputs, 2);
    if (st != DCP_TOPK_OK) return st;
  }

  dcp_topk_cand* buf = static_cast<dcp_topk_cand*>(workspace);
  for (int64_t c0 = 0; c0 < rows; c0 += DCP_TOPK_MERGE_ROWS) {
    const int32_t n = static_cast<int32_t>(rows - c0 < DCP_TOPK_MERGE_ROWS ? rows - c0 : DCP_TOPK_MERGE_ROWS);
    if (local_k > 0) {
      for (int g = 0; g < dcp; g += kMaxPackRanks) {
        const int nr = dcp - g < kMaxPackRanks ? dcp - g : kMaxPackRanks;
        PackRank pr[kMaxPackRanks];
        for (int r = 0; r < nr; ++r) {
          pr[r] = {local_scores[g + r] + c0 * local_k, local_idx[g + r] + c0 * local_k, row_starts[g + r] + c0,
                   rank_offsets[g + r]};
        }
        const hipError_t e = launch_pack(pr, nr, local_k, n, local_k, buf + static_cast<int64_t>(g) * local_k,
                                         num_cand, stream);
        if (e != hipSuccess) return DCP_TOPK_EHIP;
      }
    }
    const hipError_t e = launch_select(buf, n, num_cand, k, out + c0 * k, stream);
    if (e != hipSuccess) return DCP_TOPK_EHIP;
  }
  return DCP_TOPK_OK;
}

}  // namespace dcptopk

extern "C" {

const char* dcp_topk_status_string(int status) {
  switch (status) {
    case DCP_TOPK_OK:
      return "ok";
    case DCP_TOPK_EINVAL:
      return "invalid argument";
    case DCP_TOPK_EUNSUPPORTED:
      return "unsupported shape";
    case DCP_TOPK_EWORKSPACE:
      return "workspace too small or misaligned";
    case DCP_TOPK_EHIP:
      return "HIP launch failed";
    case DCP_TOPK_ESCRATCH:
      return "shape needs more than the static scratch buffer";
    default:
      return "unknown status";
  }
}

size_t dcp_topk_merge_workspace_bytes(int32_t rows, int32_t dcp, int32_t local_k) {
  if (rows < 0 || dcp < 0 || local_k < 0) return 0;
  const int64_t chunk = rows < DCP_TOPK_MERGE_ROWS ? rows : DCP_TOPK_MERGE_ROWS;
  // 1024 rows of up to 2^62 candidates can exceed size_t: such a shape has no
  // valid size (and the merge rejects it as unsupported)
  const unsigned __int128 b = static_cast<unsigned __int128>(chunk) * static_cast<uint64_t>(dcp) *
                              static_cast<uint64_t>(local_k) * kCandBytes;
  return b > SIZE_MAX ? 0 : static_cast<size_t>(b);
}

int dcp_topk_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, dcp_topk_cand* out,
                    hipStream_t stream) {
  const int st = check_select(cand, rows, num_cand, k, out);
  if (st != DCP_TOPK_OK || rows == 0) return st;
  return hip_status(dcptopk::launch_select(cand, rows, num_cand, k, out, stream));
}

size_t dcp_topk_select_split_workspace_bytes(int32_t rows, int32_t num_cand, int32_t parts) {
  // (num_cand <= DCP_TOPK_MAX_CANDIDATES also keeps the byte count far below
  // the range of size_t)
  if (rows < 0 || num_cand < 0 || num_cand > DCP_TOPK_MAX_CANDIDATES || parts < 1 || parts > DCP_TOPK_SPLIT_MAX_PARTS)
    return 0;
  return dcptopk::split_layout(rows, num_cand, parts).bytes;
}

int dcp_topk_select_split(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k, int32_t parts,
                          void* workspace, size_t workspace_bytes, dcp_topk_cand* out, hipStream_t stream) {
  int st = check_select(cand, rows, num_cand, k, out);
  if (st != DCP_TOPK_OK || rows == 0) return st;
  if (parts < 1 || parts > DCP_TOPK_SPLIT_MAX_PARTS || dcptopk::split_slice_len(num_cand, parts) > dcptopk::kSplitMaxSlice)
    return DCP_TOPK_EUNSUPPORTED;
  if (k >= num_cand) return hip_status(dcptopk::launch_select(cand, rows, num_cand, k, out, stream));
  const size_t need = dcp_topk_select_split_workspace_bytes(rows, num_cand, parts);
  if (workspace == nullptr || !aligned(workspace, DCP_TOPK_WORKSPACE_ALIGN) || workspace_bytes < need)
    return DCP_TOPK_EWORKSPACE;
  const Span ws{reinterpret_cast<uintptr_t>(workspace), need};
  Span in_span, out_span;
  if (!strided_span(cand, rows, num_cand, num_cand, kCandBytes, &in_span) ||
      !strided_span(out, rows, k, k, kCandBytes, &out_span))
    return DCP_TOPK_EINVAL;
  if (overlap(ws, in_span) || overlap(ws, out_span)) return DCP_TOPK_EINVAL;
  const hipError_t e = dcptopk::launch_select_split(cand, rows, num_cand, k, parts, workspace, out, stream);
  if (e == hipErrorCooperativeLaunchTooLarge) {
    (void)hipGetLastError();  // clear the rejected launch's error (it enqueued nothing) for later callers
    return DCP_TOPK_EUNSUPPORTED;
  }
  return hip_status(e);
}

int dcp_topk_pack(const float* local_scores, const int32_t* local_idx, int64_t src_row_stride,
                  const int32_t* row_starts, int32_t rank_offset, int32_t rows, int32_t local_k, dcp_topk_cand* dst,
                  int64_t dst_row_stride, hipStream_t stream) {
  const int st = check_pack(local_scores, local_idx, src_row_stride, row_starts, rows, local_k, dst, dst_row_stride);
  if (st != DCP_TOPK_OK || rows == 0 || local_k == 0) return st;
  const dcptopk::PackRank r{local_scores, local_idx, row_starts, rank_offset};
  return hip_status(dcptopk::launch_pack(&r, 1, src_row_stride, rows, local_k, dst, dst_row_stride, stream));
}

int dcp_topk_merge_chunked(const float* const* local_scores, const int32_t* const* local_idx,
                           const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp, int32_t rows,
                           int32_t local_k, int32_t k, void* workspace, size_t workspace_bytes, dcp_topk_cand* out,
                           hipStream_t stream) {
  bool nothing = false;
  int st = dcptopk::check_merge_shape(local_scores, local_idx, row_starts, rank_offsets, dcp, rows, local_k, k,
                                      &nothing);
  if (st != DCP_TOPK_OK || nothing) return st;
  const size_t need = dcp_topk_merge_workspace_bytes(rows, dcp, local_k);
  if (need > 0 && (workspace == nullptr || !aligned(workspace, DCP_TOPK_WORKSPACE_ALIGN))) return DCP_TOPK_EWORKSPACE;
  if (workspace_bytes < need) return DCP_TOPK_EWORKSPACE;
  return dcptopk::merge_chunks(local_scores, local_idx, row_starts, rank_offsets, dcp, rows, local_k, k, workspace,
                               out, stream);
}

int dcp_topk_merge_fused(const float* const* local_scores, const int32_t* const* local_idx,
                         const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp, int32_t rows,
                         int32_t local_k, int32_t k, dcp_topk_cand* out, hipStream_t stream) {
  if (dcp < 1 || rows < 0 || local_k < 0 || k < 1) return DCP_TOPK_EINVAL;
  if (local_scores == nullptr || local_idx == nullptr || row_starts == nullptr || rank_offsets == nullptr)
    return DCP_TOPK_EINVAL;
  if (dcp > dcptopk::kMaxFusedRanks || local_k % 64 != 0 ||
      static_cast<int64_t>(dcp) * local_k > DCP_TOPK_MAX_CANDIDATES || k > DCP_TOPK_MAX_CANDIDATES ||
      rows > DCP_TOPK_MAX_ROWS)
    return DCP_TOPK_EUNSUPPORTED;
  if (rows == 0) return DCP_TOPK_OK;
  if (out == nullptr || !aligned(out, kCandBytes)) return DCP_TOPK_EINVAL;
  Span o;
  if (!strided_span(out, rows, k, k, kCandBytes, &o)) return DCP_TOPK_EINVAL;
  dcptopk::FusedRanks ranks{};
  if (local_k > 0) {
    const int st = check_ranks(local_scores, local_idx, row_starts, dcp, rows, local_k, &o, 1);
    if (st != DCP_TOPK_OK) return st;
    for (int r = 0; r < dcp; ++r) ranks.rank[r] = {local_scores[r], local_idx[r], row_starts[r], rank_offsets[r]};
  }
  return hip_status(dcptopk::launch_fused(ranks, local_k > 0 ? dcp : 0, rows, local_k, k, out, stream));
}

int dcp_topk_local(const float* scores, int64_t score_row_stride, const int32_t* lengths, int32_t rows,
                   int32_t num_cols, int32_t k, float* out_scores, int32_t* out_idx, int64_t out_row_stride,
                   hipStream_t stream) {
  if (rows < 0 || num_cols < 0 || k < 1) return DCP_TOPK_EINVAL;
  if (num_cols > DCP_TOPK_MAX_CANDIDATES || k > DCP_TOPK_MAX_CANDIDATES || rows > DCP_TOPK_MAX_ROWS)
    return DCP_TOPK_EUNSUPPORTED;
  if (rows == 0) return DCP_TOPK_OK;
  if (out_scores == nullptr || out_idx == nullptr || (num_cols > 0 && scores == nullptr)) return DCP_TOPK_EINVAL;
  if (score_row_stride < num_cols || out_row_stride < k) return DCP_TOPK_EINVAL;
  if (!aligned(out_scores, 4) || !aligned(out_idx, 4) || (scores != nullptr && !aligned(scores, 4)) ||
      (lengths != nullptr && !aligned(lengths, 4)))
    return DCP_TOPK_EINVAL;
  Span s, l, os, oi;
  if (!strided_span(scores, rows, num_cols, score_row_stride, 4, &s) ||
      !strided_span(lengths, lengths != nullptr ? rows : 0, 1, 1, 4, &l) ||
      !strided_span(out_scores, rows, k, out_row_stride, 4, &os) ||
      !strided_span(out_idx, rows, k, out_row_stride, 4, &oi))
    return DCP_TOPK_EINVAL;
  if (overlap(os, oi) || overlap(os, s) || overlap(os, l) || overlap(oi, s) || overlap(oi, l)) return DCP_TOPK_EINVAL;
  return hip_status(dcptopk::launch_local(scores, score_row_stride, lengths, rows, num_cols, k, out_scores, out_idx,
                                          out_row_stride, stream));
}

}  // extern "C"
