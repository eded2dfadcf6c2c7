// The chunked merge with its workspace in a static device buffer, for callers
// that cannot allocate device memory.
//
// The buffer is one file-scope device array.  Host code must not pass the
// array's name to a kernel or a copy: on the host that name is only a stand-in
// for the symbol.  Its device address on each GPU is looked up once, with that
// GPU current (hipGetSymbolAddress), and that address is what the chunk walk
// receives as its workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "libdcptopk.h"

namespace {

// One chunk's row-major gathered buffer: DCP_TOPK_MERGE_ROWS rows of up to
// 8192 candidates (the workspace dcp_topk_merge_chunked needs at DCP 4 x
// local K 2048).
static __device__ __align__(256) unsigned char scratch[DCP_TOPK_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_lookup;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of `scratch` on the current device (looked up on the first
// call on that device), or nullptr.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_lookup);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int dcp_topk_merge_chunked_static(const float* const* local_scores, const int32_t* const* local_idx,
                                             const int32_t* const* row_starts, const int32_t* rank_offsets,
                                             int32_t dcp, int32_t rows, int32_t local_k, int32_t k,
                                             dcp_topk_cand* out, hipStream_t stream) {
  bool nothing = false;
  const int st = dcptopk::check_merge_shape(local_scores, local_idx, row_starts, rank_offsets, dcp, rows, local_k,
                                            k, &nothing);
  if (st != DCP_TOPK_OK || nothing) return st;
  if (dcp_topk_merge_workspace_bytes(rows, dcp, local_k) > static_cast<size_t>(DCP_TOPK_STATIC_SCRATCH_BYTES))
    return DCP_TOPK_ESCRATCH;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return DCP_TOPK_EHIP;
  return dcptopk::merge_chunks(local_scores, local_idx, row_starts, rank_offsets, dcp, rows, local_k, k, ws, out,
                               stream);
}
