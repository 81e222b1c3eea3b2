// Internal: the parameter block of the decode kernels and the fixed-partition
// unit mapping, shared by the 16-bit / float32 kernels and the E4M3 kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"

namespace pkv {

struct DecodeParams {
  void* out;
  const void* q;
  const char* k;
  const char* v;
  const int32_t* tables;
  const int32_t* ctx_lens;
  void* part_o;         // [S][Hq][num_parts][D] the partitions' weighted sums, scaled (float32 for
                        // float32 caches, f16 for the others; see record_scale_exp)
  float* part_ml;       // same rows, (max in the log2 domain, sum of weights, a, unused): the weighted
                        // sums are the stored values times a
  int64_t tile_bytes;   // paged: bytes of one (block, KV head) tile
  int64_t region_bytes; // contiguous: bytes of one (sequence, KV head) region
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t log2_block;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_ctx;
  int32_t part_tokens;  // partition length
  int32_t num_parts;    // partitions of the longest context (record slots per head)
  int32_t full_parts;   // partitions that can be full under the bound (max_ctx / part_tokens)
  int32_t out_f32;
  float scale_log2e;    // scale * log2(e) (times k_scale for E4M3 caches): scores live in the log2 domain
  float v_scale;        // E4M3 caches: V element = value(code) * v_scale
};

// The fixed-partition grid: workgroup id -> unit, in two phases.
// * Phase 1 (ids below phase1_units): every (KV head, sequence, partition)
//   whose partition could be full under the context bound, full_parts
//   partitions per sequence.  A unit runs only if its partition is full
//   (ends at or before the context's end); the rest exit at once.
//   - KV head varies fastest: consecutive workgroups go to the 8 XCDs in
//     turn, so with Hkv a multiple of 8 each XCD serves a fixed set of KV
//     heads for every sequence and all XCDs get the same work.
//   - Sequences are taken in chunks of kSeqChunk; inside a chunk, partition
//     varies slowest.  Sequences that share prefix blocks (forks, beams) sit
//     next to each other, so their reads of the same (block, head) tile happen
//     at about the same time on the same XCD and hit its L2, while the
//     working set of a chunk stays within that L2.
// * Phase 2 (Hkv x S ids, KV head fastest): each sequence's last partition
//   when it is partial, or the zero output row of an empty context.
// Dispatch follows the grid order, so the partial partitions (shorter, and
// never shared between sequences) come after all full ones: the shortest
// work ends the launch, which keeps its tail short.
constexpr int kSeqChunk = 32;
struct Unit { int g, s, part; };

__host__ __device__ inline int64_t padded_seqs(int64_t S) { return (S + kSeqChunk - 1) / kSeqChunk * kSeqChunk; }
__host__ __device__ inline int64_t phase1_units(const DecodeParams& p) {
  return int64_t(p.full_parts) * padded_seqs(p.num_seqs) * p.num_kv_heads;
}
__host__ __device__ inline int64_t grid_units(const DecodeParams& p) {
  return phase1_units(p) + int64_t(p.num_seqs) * p.num_kv_heads;
}

constexpr int kUnitNone = 0;     // nothing to do
constexpr int kUnitRange = 1;    // reduce partition u.part of (u.s, u.g)
constexpr int kUnitZeroRow = 2;  // empty context: write the group's zero output rows

// Resolves workgroup `id` against its sequence's context, which it reads
// (clamped to max_ctx) into *ctx.
__device__ __forceinline__ int unit_of(int id, const DecodeParams& p, Unit* u, int* ctx) {
  const int64_t n1 = phase1_units(p);
  if (id < n1) {
    u->g = id % p.num_kv_heads;
    const int rest = id / p.num_kv_heads;
    const int chunk = rest / (kSeqChunk * p.full_parts);
    const int within = rest % (kSeqChunk * p.full_parts);
    u->part = within / kSeqChunk;
    u->s = chunk * kSeqChunk + within % kSeqChunk;
    if (u->s >= p.num_seqs) return kUnitNone;   // padding of the last chunk
    *ctx = min(p.ctx_lens[u->s], p.max_ctx);
    return (u->part + 1) * p.part_tokens <= *ctx ? kUnitRange : kUnitNone;
  }
  const int k = int(id - n1);
  u->g = k % p.num_kv_heads;
  u->s = k / p.num_kv_heads;
  *ctx = min(p.ctx_lens[u->s], p.max_ctx);
  if (*ctx <= 0) {
    u->part = 0;
    return kUnitZeroRow;
  }
  u->part = *ctx / p.part_tokens;
  return *ctx % p.part_tokens ? kUnitRange : kUnitNone;
}

// Power-of-two exponent k under which a record row whose largest magnitude is
// amax is stored as f16: amax * 2^k lies in [2^14, 2^15), inside the f16
// range, and every value keeps f16's 11 significant bits (the relative
// rounding error is at most 2^-11; values below 2^-24 of the row maximum
// round to subnormals or zero).  A zero or non-finite maximum gets k = 0.
__device__ __forceinline__ int record_scale_exp(float amax) {
  if (!(amax > 0.f) || !__builtin_isfinite(amax)) return 0;
  // amax = m 2^e with m in [0.5, 1); k is kept within +-126 so that both 2^k
  // and 2^-k are normal float32 numbers
  const int k = 15 - __builtin_amdgcn_frexp_expf(amax);
  return k < -126 ? -126 : (k > 126 ? 126 : k);
}

// Launches decode_fp8_kernel over the fixed-partition grid (E4M3 caches,
// head_dim D of 64 or 128, q of type q_dtype, G query heads per KV head); the
// caller launches the combine kernel when contexts span several partitions.
pa_status launch_decode_fp8_partitions(const DecodeParams& p, pa_dtype q_dtype, int D, int G, hipStream_t st);

}  // namespace pkv
