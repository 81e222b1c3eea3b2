// Memory-read ceilings of this GPU, for context beside the decode roofline.
// Not part of the decode path: a separate library (libpagedkv_ceiling.so)
// that only the benchmark loads.
//
//   pc_stream_read: every 16-byte chunk of a buffer read once, in address
//     order, by a grid-stride loop (the plain streaming rate).
//   pc_tile_read: whole 4 KiB tiles at the given tile indices of a buffer,
//     4 tiles per wave, consecutive lanes on consecutive 16-byte chunks (the
//     decode's own access shape: 4 KiB (block, KV head) tiles at scattered
//     addresses).
// Loaded data is XOR-folded and written to `sink` (one 16-byte word per
// thread) so no load is dead.  Both return 0, or -1 for bad arguments.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* buf, int64_t n, uint4* sink) {
  // four independent 16-byte loads per thread and iteration
  uint4 acc = make_uint4(0, 0, 0, 0);
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  for (; i < n; i += stride) {
    const uint4 v = buf[i];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// One 64-lane wave per kTiles tiles of 4 KiB: all 16 loads of a wave are
// issued before any is used (16 KiB in flight per wave).
constexpr int kTiles = 4;
constexpr int kTileBytes = 4096;
__global__ __launch_bounds__(64) void tile_read_kernel(const char* buf, const int32_t* ids, int32_t n_tiles,
                                                       uint4* sink) {
  const int lane = threadIdx.x;
  const int64_t first = int64_t(blockIdx.x) * kTiles;
  uint4 v[kTiles][kTileBytes / 1024];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int64_t k = first + t < n_tiles ? first + t : n_tiles - 1;
    const char* tile = buf + int64_t(ids[k]) * kTileBytes + lane * 16;
#pragma unroll
    for (int j = 0; j < kTileBytes / 1024; ++j) v[t][j] = *reinterpret_cast<const uint4*>(tile + j * 1024);
  }
  uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int j = 0; j < kTileBytes / 1024; ++j) {
      acc.x ^= v[t][j].x;
      acc.y ^= v[t][j].y;
      acc.z ^= v[t][j].z;
      acc.w ^= v[t][j].w;
    }
  sink[int64_t(blockIdx.x) * 64 + lane] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) of buf with `blocks` workgroups of 256
// threads; sink holds blocks * 256 16-byte words.
extern "C" int pc_stream_read(const void* buf, int64_t bytes, int32_t blocks, void* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Reads n_tiles whole 4 KiB tiles at the indices in ids (device int32, each
// < the buffer's tile count, which the caller guarantees), 4 tiles per
// 64-lane wave; sink holds ceil(n_tiles / 4) * 64 16-byte words.
extern "C" int pc_tile_read(const void* buf, const int32_t* ids, int32_t n_tiles, void* sink, void* stream) {
  if (!buf || !ids || !sink || n_tiles <= 0) return -1;
  const int32_t waves = (n_tiles + kTiles - 1) / kTiles;
  hipLaunchKernelGGL(tile_read_kernel, dim3(waves), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(buf), ids, n_tiles, static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
