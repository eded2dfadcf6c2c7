// Reference kernels for the select's roofline, not part of libdcptopk: what a
// launch of the headline's shape costs with no work (the launch floor), and
// what it costs to move the headline's bytes with nothing else done (a bare
// read of 256 rows of 8192 eight-byte candidates, and that read with the
// 256 x 2048 eight-byte outputs written too).  Built into
// libdcptopk_floor.so and timed by stable_top_selection_amd/floor_probe.py.
//
// Every kernel runs one 512-thread workgroup per row, and each wave reads its
// row's candidates the way the select's gathered source does: wave w owns
// 8 KiB of the row, read as 8 loads of 16 bytes per lane, 1 KiB per wave and
// load, non-temporal.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 512;
constexpr int kWave = 64;
constexpr int kLoads = 8;                                  // 16-byte loads per lane and row
constexpr int kRowVecs = kBlock * kLoads;                  // uint4 per row: 8192 candidates
constexpr int kOutVecs = 1024;                             // uint4 written per row: 2048 candidates
constexpr uint32_t kNever = 0x9E3779B9u;                   // a sum the synthetic data never reaches

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void floor_empty_kernel() {}

// Offset (in uint4) of load j of this thread inside its row.
__device__ __forceinline__ int vec_offset(int j) {
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  return w * kWave * kLoads + j * kWave + lane;
}

template <bool WRITE>
__global__ __launch_bounds__(kBlock) void floor_stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                             uint32_t* __restrict__ sink) {
  const u32x4* row = src + static_cast<int64_t>(blockIdx.x) * kRowVecs;
  u32x4 v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) v[j] = __builtin_nontemporal_load(row + vec_offset(j));
  if constexpr (WRITE) {
    // 16 KiB per row: the first two loads of every thread, as the output of
    // 2048 selected candidates would be, in 2 stores of 16 bytes per lane
    u32x4* out = dst + static_cast<int64_t>(blockIdx.x) * kOutVecs;
    __builtin_nontemporal_store(v[0], out + threadIdx.x);
    __builtin_nontemporal_store(v[1], out + kBlock + threadIdx.x);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  // keeps every load live; the inputs are chosen so that it never stores
  if (acc == kNever) sink[blockIdx.x] = acc;
}

}  // namespace

// Entry points return 0, -1 for an invalid argument (nothing launched) or -4
// when the HIP runtime rejects the launch (the codes of libdcptopk).
extern "C" {

// One launch of `workgroups` empty workgroups of `threads` threads (1 to 1024).
__attribute__((visibility("default"))) int floor_empty(int32_t workgroups, int32_t threads, hipStream_t stream) {
  if (workgroups < 1 || threads < 1 || threads > 1024) return -1;
  return hipLaunchKernel(reinterpret_cast<const void*>(&floor_empty_kernel), dim3(workgroups), dim3(threads), nullptr,
                         0, stream) == hipSuccess ? 0 : -4;
}

// Reads rows x 64 KiB from src (16-byte aligned) and, if dst is not NULL,
// writes rows x 16 KiB to dst (16-byte aligned).  sink holds `rows` words; it
// is written only if a row's loads sum to kNever.
__attribute__((visibility("default"))) int floor_stream(const void* src, void* dst, uint32_t* sink, int32_t rows,
                                                        hipStream_t stream) {
  if (rows < 1 || src == nullptr || sink == nullptr) return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return -1;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  void* args[] = {&s, &d, &sink};
  const void* fn = dst != nullptr ? reinterpret_cast<const void*>(&floor_stream_kernel<true>)
                                  : reinterpret_cast<const void*>(&floor_stream_kernel<false>);
  return hipLaunchKernel(fn, dim3(rows), dim3(kBlock), args, 0, stream) == hipSuccess ? 0 : -4;
}

// Bytes floor_stream reads and writes per row.
__attribute__((visibility("default"))) int64_t floor_row_read_bytes() { return int64_t{kRowVecs} * 16; }
__attribute__((visibility("default"))) int64_t floor_row_write_bytes() { return int64_t{kOutVecs} * 16; }

}  // extern "C"
