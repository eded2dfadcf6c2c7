// Pack DCP ranks' local top-K into the row-major gathered candidate buffer.
//
// vLLM PR #59367 ("[Bugfix][Attention] Reserve the sparse indexer's DCP top-k
// merge scratch through the workspace manager", Purpose): the pack step turns a
// rank's local top-K (score, local index) into packed (score, global id)
// candidates using one row start per query row, and the selector reads a
// row-major buffer with the rank dimension inside the row.  On one GPU nothing
// is exchanged, so the pack writes each rank's slice straight to its columns
// [r*local_k, (r+1)*local_k) of that buffer (no separate rank-major buffer and
// no strided copy).
//
// HBM-bound: 8 bytes read and 8 bytes written per candidate.  A thread packs 4
// consecutive candidates: one 16-byte load of scores, one of indices, two
// 16-byte stores.  Grid: x = rows, y = column blocks of 1024, z = ranks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dcptopk {
namespace {

constexpr int kPackBlock = 256;
constexpr int kPerThread = 4;
constexpr uint32_t kPadBits = 0xFF800000u;  // -inf
constexpr uint32_t kPadId = 0x7FFFFFFFu;    // INT32_MAX

typedef int int4v __attribute__((ext_vector_type(4)));

struct PackArgs {
  PackRank rank[kMaxPackRanks];
};

__device__ __forceinline__ uint2 pack_one(uint32_t score_bits, int32_t idx, uint32_t base) {
  if (idx < 0) return make_uint2(kPadBits, kPadId);
  return make_uint2(score_bits, static_cast<uint32_t>(idx) + base);
}

template <bool VEC>
__global__ __launch_bounds__(kPackBlock) void pack_kernel(PackArgs args, int64_t src_row_stride, int32_t local_k,
                                                          dcp_topk_cand* __restrict__ dst, int64_t dst_row_stride) {
  const int64_t row = blockIdx.x;
  const int r = blockIdx.z;
  const int j0 = (blockIdx.y * kPackBlock + threadIdx.x) * kPerThread;
  if (j0 >= local_k) return;
  const PackRank& pr = args.rank[r];
  // two's-complement wrap, like the id sum
  const uint32_t base = static_cast<uint32_t>(pr.row_starts[row]) + static_cast<uint32_t>(pr.rank_offset);
  const int64_t src = row * src_row_stride + j0;
  uint2* out = reinterpret_cast<uint2*>(dst + row * dst_row_stride + static_cast<int64_t>(r) * local_k + j0);
  if (VEC && j0 + kPerThread <= local_k) {
    // the local arrays are read once: non-temporal loads; the packed buffer is
    // read again by the select right after, so its stores keep the default
    // policy
    const int4v s = __builtin_nontemporal_load(reinterpret_cast<const int4v*>(pr.scores + src));
    const int4v i = __builtin_nontemporal_load(reinterpret_cast<const int4v*>(pr.idx + src));
    const uint2 c0 = pack_one(static_cast<uint32_t>(s.x), i.x, base), c1 = pack_one(static_cast<uint32_t>(s.y), i.y, base);
    const uint2 c2 = pack_one(static_cast<uint32_t>(s.z), i.z, base), c3 = pack_one(static_cast<uint32_t>(s.w), i.w, base);
    reinterpret_cast<uint4*>(out)[0] = make_uint4(c0.x, c0.y, c1.x, c1.y);
    reinterpret_cast<uint4*>(out)[1] = make_uint4(c2.x, c2.y, c3.x, c3.y);
  } else {
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(pr.scores);
    for (int j = 0; j < kPerThread && j0 + j < local_k; ++j) out[j] = pack_one(sb[src + j], pr.idx[src + j], base);
  }
}

}  // namespace

hipError_t launch_pack(const PackRank* ranks, int nranks, int64_t src_row_stride, int32_t rows, int32_t local_k,
                       dcp_topk_cand* dst, int64_t dst_row_stride, hipStream_t stream) {
  PackArgs args{};
  bool vec = (src_row_stride % kPerThread == 0) && (dst_row_stride % 2 == 0) && (local_k % 2 == 0) &&
             (reinterpret_cast<uintptr_t>(dst) % 16 == 0);
  for (int r = 0; r < nranks; ++r) {
    args.rank[r] = ranks[r];
    vec = vec && (reinterpret_cast<uintptr_t>(ranks[r].scores) % 16 == 0) &&
          (reinterpret_cast<uintptr_t>(ranks[r].idx) % 16 == 0);
  }
  const int per_block = kPackBlock * kPerThread;
  const dim3 grid(static_cast<unsigned>(rows), static_cast<unsigned>((local_k + per_block - 1) / per_block),
                  static_cast<unsigned>(nranks));
  void* kargs[] = {&args, &src_row_stride, &local_k, &dst, &dst_row_stride};
  const void* fn = vec ? reinterpret_cast<const void*>(&pack_kernel<true>)
                       : reinterpret_cast<const void*>(&pack_kernel<false>);
  return hipLaunchKernel(fn, grid, dim3(kPackBlock), kargs, 0, stream);
}

}  // namespace dcptopk
