// Memory-read ceilings of this GPU, for context beside the decode roofline.
// Not part of the decode path: a separate library (libpagedkv_ceiling.so)
// that only the benchmark loads.
//
//   pc_stream_read: every 16-byte chunk of a buffer read once, in address
//     order, by a grid-stride loop (the plain streaming rate).
//   pc_tile_read: whole 4 KiB tiles at the given tile indices of a buffer,
//     16 tiles per wave, 4 in flight, consecutive lanes on consecutive 16-byte chunks (the
//     decode's own access shape: 4 KiB (block, KV head) tiles at scattered
//     addresses).
// Both take a flag: nonzero loads with the non-temporal cache policy (as the
// decode does for rows no other unit reads), zero with the default one.
// Loaded data is XOR-folded and written to `sink` (one 16-byte word per
// thread) so no load is dead.  Both return 0, or -1 for bad arguments.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* buf, int64_t n, uint4* sink) {
  uint4 acc = make_uint4(0, 0, 0, 0);
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
    const uint4 v = load16<NT>(buf + i);
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// One 64-lane wave walks kTilesPerWave tiles of 4 KiB with kRing tiles in
// flight: the loads of tile t + kRing are issued right after tile t is
// consumed.  Indices past the wave's last tile re-read that tile (cached), so
// every wave runs the same unconditional load sequence.
constexpr int kTileBytes = 4096;
constexpr int kTilesPerWave = 16;
constexpr int kRing = 4;
template <bool NT>
__global__ __launch_bounds__(64) void tile_read_kernel(const char* buf, const int32_t* ids, int32_t n_tiles,
                                                       uint4* sink) {
  const int lane = threadIdx.x;
  const int64_t first = int64_t(blockIdx.x) * kTilesPerWave;
  const int64_t last = first + kTilesPerWave - 1 < n_tiles ? first + kTilesPerWave - 1 : n_tiles - 1;
  auto addr = [&](int t) {
    const int64_t k = first + t < last ? first + t : last;
    return buf + int64_t(ids[k]) * kTileBytes + lane * 16;
  };
  uint4 ring[kRing][kTileBytes / 1024];
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    const char* a = addr(r);
#pragma unroll
    for (int j = 0; j < kTileBytes / 1024; ++j) ring[r][j] = load16<NT>(reinterpret_cast<const uint4*>(a + j * 1024));
  }
  uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int r = t % kRing;
#pragma unroll
    for (int j = 0; j < kTileBytes / 1024; ++j) {
      acc.x ^= ring[r][j].x;
      acc.y ^= ring[r][j].y;
      acc.z ^= ring[r][j].z;
      acc.w ^= ring[r][j].w;
    }
    if (t + kRing < kTilesPerWave) {
      __builtin_amdgcn_sched_barrier(0);
      const char* a = addr(t + kRing);
#pragma unroll
      for (int j = 0; j < kTileBytes / 1024; ++j) ring[r][j] = load16<NT>(reinterpret_cast<const uint4*>(a + j * 1024));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  sink[int64_t(blockIdx.x) * 64 + lane] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) of buf with `blocks` workgroups of 256
// threads; sink holds blocks * 256 16-byte words.
extern "C" int pc_stream_read(const void* buf, int64_t bytes, int32_t blocks, void* sink, int nontemporal,
                              void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(blocks), dim3(kThreads), 0, st,
                       static_cast<const uint4*>(buf), bytes / 16, static_cast<uint4*>(sink));
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(blocks), dim3(kThreads), 0, st,
                       static_cast<const uint4*>(buf), bytes / 16, static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Reads n_tiles whole 4 KiB tiles at the indices in ids (device int32, each
// < the buffer's tile count, which the caller guarantees), 16 tiles per
// 64-lane wave; sink holds ceil(n_tiles / 16) * 64 16-byte words.
extern "C" int pc_tile_read(const void* buf, const int32_t* ids, int32_t n_tiles, void* sink, int nontemporal,
                            void* stream) {
  if (!buf || !ids || !sink || n_tiles <= 0) return -1;
  const int32_t waves = (n_tiles + kTilesPerWave - 1) / kTilesPerWave;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(tile_read_kernel<true>, dim3(waves), dim3(64), 0, st, static_cast<const char*>(buf), ids,
                       n_tiles, static_cast<uint4*>(sink));
  else
    hipLaunchKernelGGL(tile_read_kernel<false>, dim3(waves), dim3(64), 0, st, static_cast<const char*>(buf), ids,
                       n_tiles, static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
