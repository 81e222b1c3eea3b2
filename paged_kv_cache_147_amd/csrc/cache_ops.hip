// KV-cache writes and copy-on-write block copies for gfx950.
//
// pa_write_kv puts each new token's K and V rows into the slot the pool gave
// it: a new token goes into its sequence's last block while that block has
// room ("vllm-pagedattention" (chenyuan1125.github.io), 页表真正解开的…).
// pa_copy_blocks duplicates whole blocks before a branch writes into a last
// block it still shares with others ("vllm-pagedattention", 一块内存，如何安全
// 地属于多条序列).  Both are pure 16-byte bit moves: one lane per 16 bytes,
// consecutive lanes on consecutive bytes of a row, so every wave reads and
// writes whole 128-byte lines.
#include "device_common.h"

#include <algorithm>
#include <cmath>

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One lane per 16-byte chunk of every (token, KV head) row, K and V.
__global__ __launch_bounds__(kThreads) void write_kv_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ kn,
    const char* __restrict__ vn, const int64_t* __restrict__ slots, int64_t chunks_per_token,
    int32_t chunks_per_row, int32_t row_bytes, int32_t block_size, int64_t num_slots,
    int64_t total_chunks) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t t = i / chunks_per_token;
  const int64_t in_tok = i - t * chunks_per_token;  // (kv head, chunk)
  const int64_t g = in_tok / chunks_per_row;
  const int64_t ch = in_tok - g * chunks_per_row;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;  // padding, or out of the pool
  const int64_t blk = slot / block_size;
  const int64_t row = slot - blk * block_size;
  const int64_t kv_heads = chunks_per_token / chunks_per_row;
  const int64_t dst = ((blk * kv_heads + g) * block_size + row) * row_bytes + ch * 16;
  const int64_t src = i * 16;  // new rows are [T][Hkv][d], densely packed
  *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(kn + src);
  *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(vn + src);
}

// blockIdx.x: pair, blockIdx.y: 0 = K, 1 = V.  A block of the cache is
// block_bytes contiguous bytes (all KV heads of one physical block).
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const int32_t* __restrict__ pairs,
    int64_t block_bytes, int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* cache = blockIdx.y == 0 ? kc : vc;
  const uint4* from = reinterpret_cast<const uint4*>(cache + int64_t(src) * block_bytes);
  uint4* to = reinterpret_cast<uint4*>(cache + int64_t(dst) * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) to[i] = from[i];
}

// Swap copies (preemption: a request's blocks go to host memory and come
// back later, "vllm-paged-attention-engine" (aiqz.cc), 连续批处理：随到随走的新秩序).
// Workgroup (i, half, part) moves part `part` of the K (half 0) or V (half 1)
// bytes of block blocks[i] between the caches and the host buffer, laid out
// [n][K, V][block bytes]; 16-byte loads and stores, consecutive lanes on
// consecutive bytes, so each wave moves 1 KB contiguous over the link.  Ids
// outside [0, num_blocks) are skipped.
__global__ __launch_bounds__(kThreads) void swap_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                        char* __restrict__ host, const int32_t* __restrict__ blocks,
                                                        int64_t block_bytes, int32_t num_blocks, int32_t to_host) {
  const int32_t b = blocks[blockIdx.x];
  if (b < 0 || b >= num_blocks) return;
  char* cache = (blockIdx.y == 0 ? kc : vc) + int64_t(b) * block_bytes;
  char* h = host + (int64_t(blockIdx.x) * 2 + blockIdx.y) * block_bytes;
  const int64_t n = block_bytes / 16;
  const int64_t per = (n + gridDim.z - 1) / gridDim.z;
  const int64_t lo = per * blockIdx.z, hi = min(n, lo + per);
  uint4* dst = reinterpret_cast<uint4*>(to_host ? h : cache);
  const uint4* srcp = reinterpret_cast<const uint4*>(to_host ? cache : h);
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) dst[i] = srcp[i];
}

// E4M3 code ("FN": no infinities, largest finite 448) of a float32: the
// nearest code, ties to the even code, magnitudes >= 448 saturate to +-448,
// NaN gives 0x7F.  Exact integer work on the float32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;              // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;      // |y| >= 448 = 1.75 * 2^8
  const int e = int(a >> 23) - 127;               // exponent of |y|
  if (e < -6) {                                   // below the smallest normal 2^-6:
    // steps of 2^-9; |y| * 512 < 8 is exact, rint rounds ties to even; 8 is
    // code 0x08, the smallest normal
    return sign | uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
  }
  uint32_t q = (a & 0x7fffffu) >> 20;             // 3 mantissa bits, then round the other 20
  const uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) q += 1;   // a carry moves into the exponent
  return sign | ((uint32_t(e + 7) << 3) + q);
}

// pa_write_kv_fp8: each thread quantises 16 consecutive elements of one new
// row (16 bytes of E4M3 out), x * inv_scale in float32 first.
template <class T>
__global__ __launch_bounds__(kThreads) void write_kv_fp8_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const char* __restrict__ kn, const char* __restrict__ vn,
    const int64_t* __restrict__ slots, int64_t groups_per_token, int32_t groups_per_row, int32_t head_dim,
    int32_t block_size, int64_t num_slots, int64_t total, float k_inv, float v_inv) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= 2 * total) return;
  const bool is_v = i >= total;
  const int64_t j = is_v ? i - total : i;
  const int64_t tok = j / groups_per_token;
  const int64_t rem = j % groups_per_token;              // (head, group) within the token
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t head = rem / groups_per_row, grp = rem % groups_per_row;
  const int64_t num_kv_heads = groups_per_token / groups_per_row;
  const char* src = (is_v ? vn : kn) + ((tok * num_kv_heads + head) * head_dim + grp * 16) * T::bytes;
  const float inv = is_v ? v_inv : k_inv;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float x;
      if constexpr (T::bytes == 4) x = reinterpret_cast<const float*>(src)[4 * q + b];
      else x = widen1(T{}, reinterpret_cast<const uint16_t*>(src)[4 * q + b]);
      word |= e4m3_code(x * inv) << (8 * b);
    }
    w[q] = word;
  }
  const int64_t blk = slot / block_size, row = slot % block_size;
  uint8_t* dst = (is_v ? vc : kc) + ((blk * num_kv_heads + head) * block_size + row) * head_dim + grp * 16;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

pa_status check_cache_shape(int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, pa_dtype dtype, bool codes_ok = true) {
  if (!(codes_ok ? valid_storage_dtype(dtype) : valid_dtype(dtype))) return fail(PA_E_UNSUPPORTED, "dtype");
  if (num_kv_heads <= 0 || num_blocks <= 0) return fail(PA_E_INVAL, "num_kv_heads and num_blocks must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(PA_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size must be 8, 16 or 32");
  return ok();
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pa_dtype dtype, pa_stream stream) {
  pa_status st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_E_INVAL, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return fail(PA_E_INVAL, "null device pointer");
  const int32_t row_bytes = head_dim * dtype_bytes(dtype);
  const int32_t chunks_per_row = row_bytes / 16;
  const int64_t chunks_per_token = int64_t(num_kv_heads) * chunks_per_row;
  const int64_t total = chunks_per_token * num_tokens;
  const int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > INT32_MAX) return fail(PA_E_INVAL, "too many tokens for one launch");
  hipLaunchKernelGGL(write_kv_kernel, dim3(unsigned(grid)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), slot_mapping, chunks_per_token, chunks_per_row,
                     row_bytes, block_size, int64_t(num_blocks) * block_size, total);
  return launch_status("write_kv kernel");
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, pa_dtype dtype, pa_stream stream) {
  pa_status st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (n_pairs < 0) return fail(PA_E_INVAL, "n_pairs must be >= 0");
  if (n_pairs == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_E_INVAL, "null device pointer");
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * dtype_bytes(dtype);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(n_pairs), 2), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), pairs, block_bytes, num_blocks);
  return launch_status("copy_blocks kernel");
}

namespace {

pa_status launch_swap(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n, const void* host,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      pa_dtype dtype, pa_stream stream, bool to_host) {
  pa_status st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (n < 0) return fail(PA_E_INVAL, "n must be >= 0");
  if (n == 0) return ok();
  if (!k_cache || !v_cache || !blocks || !host) return fail(PA_E_INVAL, "null pointer");
  // the kernel reaches the host buffer through its device-side address,
  // which exists for pinned (hipHostMalloc) memory only
  void* dev_host = nullptr;
  if (hipHostGetDevicePointer(&dev_host, const_cast<void*>(host), 0) != hipSuccess || !dev_host) {
    (void)hipGetLastError();
    return fail(PA_E_INVAL, "host buffer is not pinned host memory (hipHostMalloc)");
  }
  const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * dtype_bytes(dtype);
  const unsigned parts = unsigned(std::max<int64_t>(1, block_bytes / (kThreads * 16 * 4)));  // 4 rounds per workgroup
  hipLaunchKernelGGL(swap_kernel, dim3(unsigned(n), 2, parts), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), static_cast<char*>(dev_host), blocks,
                     block_bytes, num_blocks, to_host ? 1 : 0);
  return launch_status("swap kernel");
}

}  // namespace

extern "C" pa_status pa_swap_out(const void* k_cache, const void* v_cache, const int32_t* blocks, int32_t n,
                                 void* host, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype dtype, pa_stream stream) {
  return launch_swap(const_cast<void*>(k_cache), const_cast<void*>(v_cache), blocks, n, host, num_kv_heads,
                     head_dim, block_size, num_blocks, dtype, stream, true);
}

extern "C" pa_status pa_swap_in(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n, const void* host,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                pa_dtype dtype, pa_stream stream) {
  return launch_swap(k_cache, v_cache, blocks, n, host, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                     stream, false);
}

extern "C" pa_status pa_write_kv_fp8(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                     pa_dtype src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float k_scale, float v_scale, pa_stream stream) {
  pa_status st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, src_dtype, false);
  if (st != PA_OK) return st;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_E_INVAL, "k_scale and v_scale must be finite and positive");
  if (num_tokens < 0) return fail(PA_E_INVAL, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return fail(PA_E_INVAL, "null device pointer");
  const int32_t groups_per_row = head_dim / 16;
  const int64_t groups_per_token = int64_t(num_kv_heads) * groups_per_row;
  const int64_t total = groups_per_token * num_tokens;
  const int64_t grid = (2 * total + kThreads - 1) / kThreads;
  if (grid > INT32_MAX) return fail(PA_E_INVAL, "too many tokens for one launch");
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;   // rounded to float32 once, on the host
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  auto go = [&](auto tag) {
    hipLaunchKernelGGL(write_kv_fp8_kernel<decltype(tag)>, dim3(unsigned(grid)), dim3(kThreads), 0, hs,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const char*>(k_new), static_cast<const char*>(v_new), slot_mapping,
                       groups_per_token, groups_per_row, head_dim, block_size, int64_t(num_blocks) * block_size,
                       total, k_inv, v_inv);
  };
  if (src_dtype == PA_F32) go(F32{});
  else if (src_dtype == PA_F16) go(F16{});
  else go(BF16{});
  return launch_status("write_kv_fp8 kernel");
}
