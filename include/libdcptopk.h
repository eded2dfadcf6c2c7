/*
 * libdcptopk — stable global top-K selection for the decode-context-parallel
 * (DCP) sparse-indexer merge, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (vLLM PR #47348, "[Kernel] Optimize CuTeDSL DCP top-k
 * merge", Summary): every DCP rank holds the local top-K of its 1/DCP shard of
 * the KV cache; the merge picks, for every query row, the global top-K of the
 * gathered candidates, ordered by score descending and, among equal scores, by
 * the lowest global token id, deterministically.  The pack step and the row
 * chunking follow vLLM PR #59367 ("[Bugfix][Attention] Reserve the sparse
 * indexer's DCP top-k merge scratch through the workspace manager", Purpose).
 *
 * Conventions shared by every entry point:
 *
 *  - A candidate is 8 bytes: an fp32 score then an int32 global token id
 *    (dcp_topk_cand).  Scores are never converted or rounded: every result
 *    copies the score's bits.
 *  - Order: scores compare through the order-preserving 32-bit key of their
 *    bits (IEEE 754 totalOrder: -NaN < -inf < ... < -0 < +0 < ... < +inf <
 *    +NaN); equal scores compare by id as an unsigned 32-bit value, lowest
 *    first (for the ids the merge produces, which are >= 0, this is the lowest
 *    global token id); candidates that agree on score bits and id are ordered
 *    by their position in the row, lowest first.
 *  - Outputs list the selected candidates in candidate-position order.  When a
 *    row has fewer than K candidates, slots [C, K) hold the padding candidate
 *    (-inf, INT32_MAX), the same value that marks an empty shard slot.
 *  - Every pointer to candidates, scores, ids or row starts is a DEVICE pointer
 *    owned by the caller; host arrays of device pointers are read during the
 *    call only.  The library allocates nothing, keeps no pointer and no global
 *    state, and synchronises nothing: every call only enqueues work on
 *    `stream`, so calls are safe from several host threads on several streams
 *    and can be captured into a HIP graph.  The one exception is
 *    dcp_topk_merge_chunked_static, whose workspace is a static buffer of the
 *    library on each GPU (see there).
 *  - Errors are returned as negative status codes and never abort.  Arguments
 *    are checked before anything is enqueued; a failed check enqueues nothing.
 *    Faults inside a kernel surface at the caller's next synchronisation, as
 *    with any asynchronous launch.
 */
#ifndef LIBDCPTOPK_H
#define LIBDCPTOPK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI; everything else in the library is hidden. */
#define DCP_TOPK_API __attribute__((visibility("default")))

/* Rows per step of the chunked merge (vLLM PR #59367, Purpose: the merge walks
 * the rows 1024 at a time so its scratch stays bounded). */
#define DCP_TOPK_MERGE_ROWS 1024

/* Largest candidate count per row, and largest k, that the entry points
 * accept.  The pages benchmark rows of 4096, 8192 and 16384 candidates
 * (PR #47348, Benchmarks). */
#define DCP_TOPK_MAX_CANDIDATES 16384

/* Largest row count that one call of dcp_topk_select, dcp_topk_select_split,
 * dcp_topk_merge_fused, dcp_topk_local or dcp_topk_pack accepts (more rows
 * return DCP_TOPK_EUNSUPPORTED): one launch runs a workgroup of up to 1024
 * threads per row in one grid, whose size in threads is a 32-bit count.  The
 * chunked merges launch 1024 rows at a time and take any row count. */
#define DCP_TOPK_MAX_ROWS 4194303

/* Alignment the chunked merge requires of its workspace, in bytes. */
#define DCP_TOPK_WORKSPACE_ALIGN 256

/* One packed candidate: fp32 score then int32 global token id, 8 bytes
 * (PR #59367, Purpose: the packed candidates are a (T, K, 2) 32-bit array). */
typedef struct dcp_topk_cand {
  float score;
  int32_t id;
} dcp_topk_cand;

/* Status codes. */
enum {
  DCP_TOPK_OK = 0,
  DCP_TOPK_EINVAL = -1,       /* bad argument: null pointer, negative size,
                                 k < 1, misaligned or overlapping buffers */
  DCP_TOPK_EUNSUPPORTED = -2, /* valid but unsupported shape (num_cand or k
                                 above DCP_TOPK_MAX_CANDIDATES, rows above
                                 DCP_TOPK_MAX_ROWS, or a limit of one entry
                                 point); the caller can fall back to another
                                 selector or split the rows */
  DCP_TOPK_EWORKSPACE = -3,   /* workspace too small or not 256-byte aligned */
  DCP_TOPK_EHIP = -4,         /* the HIP runtime rejected a launch */
  DCP_TOPK_ESCRATCH = -5      /* the shape needs more scratch than
                                 dcp_topk_merge_chunked_static's static
                                 buffer (DCP_TOPK_STATIC_SCRATCH_BYTES) */
};

/*
 * dcp_topk_pack — one rank's local top-K into packed global candidates.
 *
 * PR #59367, Purpose: the pack step takes a row start per query row.  For row
 * t in [0, rows) and slot j in [0, local_k):
 *
 *   dst[t * dst_row_stride + j] =
 *       local_idx[t*src_row_stride + j] < 0
 *         ? (-inf, INT32_MAX)                                   (invalid slot)
 *         : (local_scores[t*src_row_stride + j],
 *            local_idx[t*src_row_stride + j] + row_starts[t] + rank_offset)
 *
 * The id sum wraps in two's complement; the score is copied bit for bit.
 *
 *   local_scores    device, fp32, rows x local_k with row stride src_row_stride
 *   local_idx       device, int32, same layout as local_scores
 *   src_row_stride  elements between consecutive rows, >= local_k
 *   row_starts      device, int32[rows]; rows <= DCP_TOPK_MAX_ROWS
 *   rank_offset     added to every valid id of this rank
 *   dst             device, 8-byte aligned; the first slot of this rank in
 *                   row 0 of a row-major gathered buffer (for DCP rank r of a
 *                   (rows, dcp*local_k) buffer: buffer + r*local_k)
 *   dst_row_stride  candidates between consecutive rows of dst, >= local_k
 *
 * rows == 0 or local_k == 0 returns DCP_TOPK_OK and enqueues nothing.  The
 * output must not overlap the inputs (DCP_TOPK_EINVAL).
 */
DCP_TOPK_API int dcp_topk_pack(const float* local_scores, const int32_t* local_idx, int64_t src_row_stride,
                  const int32_t* row_starts, int32_t rank_offset, int32_t rows, int32_t local_k,
                  dcp_topk_cand* dst, int64_t dst_row_stride, hipStream_t stream);

/*
 * dcp_topk_select — stable top-K of every row of a gathered candidate buffer.
 *
 * PR #47348, Summary: the selector radix-selects the K-th score key over the
 * 32-bit score keys first and runs a token-id tie-break pass only when that
 * threshold ties; the result equals ordering every candidate by the 64-bit key
 * (score key in the high word, complemented id in the low word).
 *
 *   cand      device, 8-byte aligned, rows x num_cand candidates, row-major
 *             (rank r's candidates of a row at columns [r*local_k, (r+1)*local_k)
 *             when the buffer is a DCP gather; any order works)
 *   rows      query rows, 0 <= rows <= DCP_TOPK_MAX_ROWS
 *   num_cand  candidates per row, 0 <= num_cand <= DCP_TOPK_MAX_CANDIDATES
 *   k         candidates to select per row, >= 1 (k > num_cand pads)
 *   out       device, 8-byte aligned, rows x k candidates, row-major; must not
 *             overlap cand
 *
 * Row t of out holds the min(k, num_cand) best candidates of row t of cand in
 * candidate-position order, then padding.  rows == 0 returns DCP_TOPK_OK and
 * enqueues nothing; cand may be NULL when num_cand == 0.
 */
DCP_TOPK_API int dcp_topk_select(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k,
                    dcp_topk_cand* out, hipStream_t stream);

/* Most workgroups dcp_topk_select_split spreads one row over. */
#define DCP_TOPK_SPLIT_MAX_PARTS 8

/*
 * dcp_topk_select_split_workspace_bytes — workspace that dcp_topk_select_split
 * needs for (rows, num_cand, parts): four regions, each rounded up to a
 * multiple of 256 bytes: rows * 16 bytes of counters, rows * parts * 8224
 * bytes of slice histograms, rows * num_cand * 8 bytes of threshold-bin list
 * entries and rows * num_cand * 4 bytes of their positions.  Returns 0 for
 * arguments outside rows >= 0, 0 <= num_cand <= DCP_TOPK_MAX_CANDIDATES,
 * 1 <= parts <= DCP_TOPK_SPLIT_MAX_PARTS.
 */
DCP_TOPK_API size_t dcp_topk_select_split_workspace_bytes(int32_t rows, int32_t num_cand, int32_t parts);

/*
 * dcp_topk_select_split — dcp_topk_select with each row spread over `parts`
 * workgroups, for batches of few rows.
 *
 * PR #50009 (Top-K performance) measures the merge at 1 to 64 decode rows,
 * where one workgroup per row leaves most of the GPU's 256 compute units
 * idle.  Here workgroup s of a row takes the candidates [s*L, (s+1)*L) with L
 * = ceil(num_cand / parts) rounded up to a multiple of 64, and the row's
 * workgroups exchange their pass-0 histograms and their threshold-bin items
 * through `workspace` at two in-kernel barriers.  The result is the same as
 * dcp_topk_select's, bit for bit.
 *
 *   cand, rows, num_cand, k, out   as for dcp_topk_select
 *   parts            workgroups per row, 1 <= parts <= DCP_TOPK_SPLIT_MAX_PARTS,
 *                    with L <= 8192
 *   workspace        device, DCP_TOPK_WORKSPACE_ALIGN-aligned, at least
 *                    dcp_topk_select_split_workspace_bytes(rows, num_cand,
 *                    parts) bytes, overlapping neither cand nor out.  It must
 *                    be zero-filled before its first use; every call leaves
 *                    its counters at zero again, so it can be reused by later
 *                    calls on the same stream.  Two calls in flight at once
 *                    (on different streams) need different workspaces.
 *   workspace_bytes  its size
 *
 * One cooperative launch of rows * parts workgroups, which must all be
 * resident on the GPU at once: a larger grid returns DCP_TOPK_EUNSUPPORTED
 * before anything runs (use dcp_topk_select there).  Rows with k >= num_cand
 * need no selection and go through dcp_topk_select's kernel, which does not
 * touch the workspace.  DCP_TOPK_EUNSUPPORTED also for parts or L out of
 * range, DCP_TOPK_EWORKSPACE for a missing, short or misaligned workspace.
 */
DCP_TOPK_API int dcp_topk_select_split(const dcp_topk_cand* cand, int32_t rows, int32_t num_cand, int32_t k,
                          int32_t parts, void* workspace, size_t workspace_bytes, dcp_topk_cand* out,
                          hipStream_t stream);

/*
 * dcp_topk_merge_workspace_bytes — workspace that dcp_topk_merge_chunked needs:
 * one chunk's row-major gathered buffer, min(rows, DCP_TOPK_MERGE_ROWS) * dcp *
 * local_k * 8 bytes.  (PR #59367, Purpose, bounds the scratch of its
 * multi-GPU merge at (1 + 2 dcp) * 8 * 1024 * K bytes; on one GPU nothing is
 * exchanged, so only the buffer the selector reads remains.)  Returns 0 for
 * negative arguments and when the size does not fit in a size_t (such shapes
 * exceed DCP_TOPK_MAX_CANDIDATES, which the merge rejects).
 */
DCP_TOPK_API size_t dcp_topk_merge_workspace_bytes(int32_t rows, int32_t dcp, int32_t local_k);

/*
 * dcp_topk_merge_chunked — the whole merge for one GPU: pack every rank's
 * local top-K into the workspace and select, DCP_TOPK_MERGE_ROWS rows at a
 * time (PR #59367, Purpose: the selector is row-independent, so walking the
 * rows in chunks does not change the result).
 *
 *   local_scores  HOST array of dcp DEVICE pointers; rank r's fp32 scores,
 *                 rows x local_k, contiguous rows
 *   local_idx     HOST array of dcp DEVICE pointers; int32, same layout
 *   row_starts    HOST array of dcp DEVICE pointers; int32[rows] each
 *   rank_offsets  HOST array of dcp int32 values
 *   dcp           ranks, >= 1; dcp * local_k <= DCP_TOPK_MAX_CANDIDATES
 *   rows, local_k, k   as in dcp_topk_pack / dcp_topk_select
 *   workspace     device, DCP_TOPK_WORKSPACE_ALIGN-aligned, at least
 *                 dcp_topk_merge_workspace_bytes(rows, dcp, local_k) bytes;
 *                 its contents on return are unspecified; it must not overlap
 *                 any input or out
 *   out           device, rows x k candidates; must not overlap any input
 *
 * Equivalent to dcp_topk_pack of every rank into a (rows, dcp*local_k) buffer
 * followed by dcp_topk_select(buffer, rows, dcp*local_k, k, out).
 */
DCP_TOPK_API int dcp_topk_merge_chunked(const float* const* local_scores, const int32_t* const* local_idx,
                           const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp,
                           int32_t rows, int32_t local_k, int32_t k, void* workspace,
                           size_t workspace_bytes, dcp_topk_cand* out, hipStream_t stream);

/* Most DCP ranks dcp_topk_merge_fused reads in one call. */
#define DCP_TOPK_FUSED_MAX_RANKS 16

/*
 * dcp_topk_merge_fused — the merge without a gathered buffer: the selector
 * reads every rank's local top-K arrays in place and packs each candidate as
 * it loads it.  This is the one-GPU form of the consumer in vLLM PR #50009
 * ("[DCP][Performance] Add Shared-DCP peer-addressable decode data paths",
 * Top-K performance), where the stable top-K loads each owner's candidate
 * shard through local and peer views instead of from an all-gathered copy; it
 * removes the write and re-read of the packed buffer that
 * dcp_topk_merge_chunked makes.
 *
 *   local_scores, local_idx, row_starts, rank_offsets, dcp, rows, k, out
 *                 as in dcp_topk_merge_chunked
 *   local_k       a multiple of 64 (so that no wave's load straddles two
 *                 ranks); other values return DCP_TOPK_EUNSUPPORTED
 *
 * Limits (DCP_TOPK_EUNSUPPORTED): dcp <= DCP_TOPK_FUSED_MAX_RANKS, dcp *
 * local_k <= DCP_TOPK_MAX_CANDIDATES, rows <= DCP_TOPK_MAX_ROWS.  No
 * workspace and no chunking: all rows go in one launch.  The result is
 * bit-identical to dcp_topk_merge_chunked with the same arguments (so to
 * dcp_topk_pack of every rank followed by dcp_topk_select); out must not
 * overlap any input (DCP_TOPK_EINVAL).
 */
DCP_TOPK_API int dcp_topk_merge_fused(const float* const* local_scores, const int32_t* const* local_idx,
                         const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp,
                         int32_t rows, int32_t local_k, int32_t k, dcp_topk_cand* out, hipStream_t stream);

/*
 * dcp_topk_local — the step before the merge: every rank's local top-K of
 * its indexer scores.  PR #47348 (Summary) has each DCP rank hold the local
 * top-K of its shard of the KV cache; PR #50009 (Top-K performance) measures
 * 2048 candidates per rank taken from 4096 local score columns.  The pages do
 * not state this step's tie rule; this library uses the merge's: for each row
 * t the candidates are the columns c < len(t), with score scores[t, c] and id
 * c, ordered by score key descending then by lowest column, and the min(k,
 * len(t)) best are written in column order, followed by (-inf, -1) slots,
 * which dcp_topk_pack turns into its padding candidate.  The output is
 * exactly the (local_scores, local_idx) pair that dcp_topk_pack,
 * dcp_topk_merge_chunked and dcp_topk_merge_fused take.
 *
 *   scores            device, fp32, rows x num_cols, row stride
 *                     score_row_stride (>= num_cols) elements
 *   lengths           device int32[rows], or NULL; len(t) = lengths[t]
 *                     clamped to [0, num_cols] (NULL: every column)
 *   num_cols          0 <= num_cols <= DCP_TOPK_MAX_CANDIDATES (rows: at most
 *                     DCP_TOPK_MAX_ROWS)
 *   k                 1 <= k <= DCP_TOPK_MAX_CANDIDATES
 *   out_scores        device, fp32, rows x k, row stride out_row_stride (>= k)
 *   out_idx           device, int32, same layout as out_scores
 *
 * The two outputs must not overlap each other or an input (DCP_TOPK_EINVAL);
 * rows == 0 returns DCP_TOPK_OK and enqueues nothing.
 */
DCP_TOPK_API int dcp_topk_local(const float* scores, int64_t score_row_stride, const int32_t* lengths,
                   int32_t rows, int32_t num_cols, int32_t k, float* out_scores, int32_t* out_idx,
                   int64_t out_row_stride, hipStream_t stream);

/* Bytes of the static device buffer dcp_topk_merge_chunked_static uses on
 * each GPU: one DCP_TOPK_MERGE_ROWS-row chunk of 8192 candidates (DCP 4 x
 * local K 2048), 64 MiB. */
#define DCP_TOPK_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * dcp_topk_merge_chunked_static — dcp_topk_merge_chunked for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same merge, bit for bit, with
 * its chunk workspace in a static device buffer of the library instead of a
 * caller workspace.  It calls no hipMalloc, hipFree or other allocating
 * routine.
 *
 *   arguments     as in dcp_topk_merge_chunked, without workspace and
 *                 workspace_bytes; `stream` must belong to the current device
 *
 * The buffer holds DCP_TOPK_STATIC_SCRATCH_BYTES bytes on every GPU the
 * library runs on, from the first call on that GPU until the process ends.
 * Shapes whose dcp_topk_merge_workspace_bytes(rows, dcp, local_k) exceeds it
 * return DCP_TOPK_ESCRATCH and enqueue nothing (with 1024 or more rows: dcp *
 * local_k > 8192).  Every call on one GPU uses that GPU's one buffer:
 * calls that overlap in time on one GPU (on different streams, or from
 * several host threads without ordering) race and give undefined results;
 * calls on one stream are ordered and safe.  The buffer needs no clearing
 * (every chunk's pack writes all of it before the select reads it).
 */
DCP_TOPK_API int dcp_topk_merge_chunked_static(const float* const* local_scores, const int32_t* const* local_idx,
                           const int32_t* const* row_starts, const int32_t* rank_offsets, int32_t dcp,
                           int32_t rows, int32_t local_k, int32_t k, dcp_topk_cand* out, hipStream_t stream);

/* Static, human-readable name of a status code. */
DCP_TOPK_API const char* dcp_topk_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBDCPTOPK_H */
