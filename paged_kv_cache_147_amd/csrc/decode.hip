// Paged decode attention for gfx950 (CDNA4): one query token per sequence,
// K/V rows gathered through block tables.
//
// What is computed ("Paged Attention" (daiw.org), 直觉 and 定义;
// "vllm-pagedattention" (chenyuan1125.github.io), 页表真正解开的…): for
// sequence s and query head h with KV head g = h / G (G = Hq / Hkv),
//   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) V_t,   t < ctx[s],
// where K_t, V_t are row t % B of block block_tables[s][t / B].  The pages
// note that the attention itself is unchanged by paging; the kernel differs
// from a contiguous one only in how it forms row addresses.  Score, softmax
// and weighted sum are done partition by partition so no score ever goes to
// HBM (the tiling idea the pages credit to FlashAttention,
// "vllm-pagedattention", 它和 FlashAttention 优化的是两张不同的账).
//
// Work decomposition (decode is HBM-bound: ~1 flop per byte for MHA, ~4 for
// a GQA group of 4, far below the VALU ridge):
//   * one 64-lane wave per (partition, KV head, sequence); a partition is a
//     fixed number of tokens, so results never depend on which physical
//     blocks hold them;
//   * 8 lanes share one token row: lane (r = lane / 8, c = lane % 8) holds
//     16-byte chunks j * 128 + c * 16 of row r of each 8-token pass, so one
//     16-byte load instruction of the wave covers 8 full 128-byte lines;
//   * the G query heads of the KV head are processed together: each K row is
//     loaded once and dotted with G queries (v_dot2 on 16-bit pairs);
//   * pass 1 streams K and leaves scaled scores in LDS, a softmax step turns
//     them into weights, pass 2 streams V and accumulates in float32 (the
//     weights are never rounded to 16 bits);
//   * when a context spans several partitions, each writes its (max, sum,
//     weighted sum) to the workspace and decode_combine_kernel merges them
//     with the log-sum-exp identity, in partition order.  (Merging inside the
//     same launch would need device-scope release/acquire fences per wave;
//     on this GPU those write back and invalidate the XCD's L2 and cost far
//     more than one short extra launch.)
// Loads are double-buffered: while one buffer of rows is being consumed the
// next is in flight, and the first V rows are requested before the softmax.
// Block ids of a partition are fetched once, one per lane, and broadcast
// with readlane, so each pass's base address is a scalar.
#include "device_common.h"

#include <cmath>

namespace pkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// Word 3 of a raw (untyped) buffer resource on gfx9-family GPUs: 32-bit data
// format, no swizzle; loads through it are plain byte-addressed loads.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kRowsPerPass = 8;
constexpr int kMaxPartition = 512;
// Automatic partition size: the largest of 512 / 256 / 128 tokens that still
// yields at least this many (sequence, KV head, partition) units, i.e. about
// eight waves per compute unit of an MI355X (256 CUs).  Longer partitions
// amortise each wave's fixed costs; enough units keep every CU busy.
constexpr int64_t kAutoMinUnits = 2048;

// ---- element helpers ------------------------------------------------------

__device__ __forceinline__ float dot_chunk(F32, uint4 k, uint4 q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

__device__ __forceinline__ float dot_chunk(F16, uint4 k, uint4 q, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.x), __builtin_bit_cast(half2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.y), __builtin_bit_cast(half2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.z), __builtin_bit_cast(half2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w), __builtin_bit_cast(half2_t, q.w), acc, false);
  return acc;
}

__device__ __forceinline__ float dot_chunk(BF16, uint4 k, uint4 q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.x), __builtin_bit_cast(bf162_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.y), __builtin_bit_cast(bf162_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.z), __builtin_bit_cast(bf162_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.w), __builtin_bit_cast(bf162_t, q.w), acc, false);
  return acc;
}

// Exact widening of one 16-byte chunk to float32.
__device__ __forceinline__ void widen(F32, uint4 c, float* o) {
  o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
  o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
}

__device__ __forceinline__ void widen(F16, uint4 c, float* o) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    half2_t h = __builtin_bit_cast(half2_t, w[i]);
    o[2 * i] = float(h.x);
    o[2 * i + 1] = float(h.y);
  }
}

__device__ __forceinline__ void widen(BF16, uint4 c, float* o) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// float32 -> 16-bit output, round to nearest even.
__device__ __forceinline__ uint16_t narrow(F16, float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t narrow(BF16, float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Eight float32 values -> eight 16-bit outputs in one 16-byte store.
template <class T>
__device__ __forceinline__ void store_narrow(T, uint16_t* o, const float* a, float inv) {
  if constexpr (T::bytes == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(narrow(T{}, a[2 * i] * inv)) | (uint32_t(narrow(T{}, a[2 * i + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Lane-exchange steps within the 8 lanes of a row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int kRowRor8 = 0x128;      // lane i <- (i + 8) mod 16 within a row

// Sum over the 8 lanes of a token row; every lane of the row gets the total.
__device__ __forceinline__ float row8_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  return x;
}

// ---- kernels ----------------------------------------------------------------

struct DecodeParams {
  void* out;
  const void* q;
  const char* k;
  const char* v;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* part_o;        // [S][Hq][num_parts][D] unnormalised partition sums
  float* part_ml;       // [S][Hq][num_parts][2] (max, sum of weights), log2 domain
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
  int32_t part_tokens;
  int32_t num_parts;
  int32_t out_f32;
  float scale_log2e;    // scale * log2(e): scores live in the log2 domain
};

// q.K on the matrix cores: for a GQA group (G >= 2) of 16-bit heads, the
// scores of 16 tokens x G heads are a small dense contraction over head_dim,
// done as head_dim / 32 v_mfma_f32_16x16x32 steps (A = 16 K rows, B = the
// group's queries padded to 16 columns).  A 16-token tile must sit inside one
// block (block_size >= 16, or the contiguous layout).  MHA (G == 1), float32
// caches and 8-token blocks use packed dot products on the vector ALUs.
template <class T, int G>
constexpr bool mfma_capable() { return T::bytes == 2 && G >= 2; }

// Passes (of 8 token rows) held by one V load buffer; two buffers alternate,
// so up to 2 * passes_per_buffer * 8 rows are in flight per wave.  The
// vector-ALU score path uses the same buffers for K.
template <int G>
constexpr int passes_per_buffer() { return G <= 2 ? 4 : 2; }

// Rows of LDS scores a partition of `part_tokens` tokens needs: both passes
// run in pairs of buffers (at most 8 passes = 64 rows per pair), so the count
// is rounded up to 64 rows; 64 more floats serve as a sink for the MFMA
// lanes that carry padding heads.
__host__ __device__ constexpr int lds_rows(int part_tokens) { return (part_tokens + 63) / 64 * 64; }
template <int G>
__host__ __device__ constexpr int lds_floats(int part_tokens) { return lds_rows(part_tokens) * G + 64; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_qk(BF16, uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_qk(F16, uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_qk(F32, uint4, uint4, f32x4_t c) { return c; }

// Linear workgroup id -> (KV head, sequence, partition).
// * KV head varies fastest: consecutive workgroups go to the 8 XCDs in turn,
//   so with Hkv a multiple of 8 each XCD serves a fixed set of KV heads for
//   every sequence and all XCDs get the same work.
// * Sequences are taken in chunks of kSeqChunk; inside a chunk, partition
//   varies slowest.  Sequences that share prefix blocks (forks, beams) sit
//   next to each other, so their reads of the same (block, head) tile happen
//   at about the same time on the same XCD and hit its L2, while the working
//   set of a chunk stays within that L2.
// * Partitions past a sequence's end exit at once; they fall at the end of
//   each chunk rather than on particular XCDs.
constexpr int kSeqChunk = 32;
struct Unit { int g, s, part; };
__device__ __forceinline__ Unit unit_of(int id, const DecodeParams& p) {
  Unit u;
  u.g = id % p.num_kv_heads;
  const int rest = id / p.num_kv_heads;
  const int chunk = rest / (kSeqChunk * p.num_parts);
  const int within = rest % (kSeqChunk * p.num_parts);
  u.part = within / kSeqChunk;
  u.s = chunk * kSeqChunk + within % kSeqChunk;
  if (u.s >= p.num_seqs) {  // padding of the last chunk: an empty unit
    u.s = 0;
    u.part = p.num_parts;
  }
  return u;
}

template <class T, int D, int G, bool PAGED, bool MFMA>
__global__ __launch_bounds__(kWave) void decode_partition_kernel(DecodeParams p) {
  constexpr int EPC = 16 / T::bytes;          // elements per 16-byte chunk
  constexpr int ROW_BYTES = D * T::bytes;
  constexpr int NCH = ROW_BYTES / 128;        // chunks per lane per row
  constexpr int NV = NCH * EPC;               // values per lane per row (= D / 8)
  static_assert(!MFMA || mfma_capable<T, G>(), "MFMA scores need 16-bit data and G >= 2");
  constexpr int U = MFMA ? 2 : passes_per_buffer<G>();
  constexpr int KT = 1;  // 16-token score tiles per K buffer (MFMA path)
  constexpr int KK = D / 32;                  // MFMA steps over head_dim
  static_assert(NCH >= 1, "row must span the 8 lanes");

  extern __shared__ float lds[];  // [rows][G] scores, then weights; + 64-float sink

  const Unit unit = unit_of(blockIdx.x, p);
  const int g = unit.g, s = unit.s, part = unit.part;
  const int lane = threadIdx.x;
  const int r = lane >> 3;
  const int c = lane & 7;

  const int ctx = min(p.ctx_lens[s], p.max_ctx);
  const int64_t head0 = int64_t(s) * p.num_q_heads + int64_t(g) * G;  // first query row
  if (ctx <= 0) {
    // no context: defined as a zero output row
    if (part == 0) {
      for (int i = lane; i < G * D; i += kWave) {
        if (p.out_f32 || T::bytes == 4) reinterpret_cast<float*>(p.out)[head0 * D + i] = 0.f;
        else reinterpret_cast<uint16_t*>(p.out)[head0 * D + i] = 0;
      }
    }
    return;
  }
  const int tok0 = part * p.part_tokens;
  if (tok0 >= ctx) return;
  const int tok1 = min(tok0 + p.part_tokens, ctx);
  const int nparts_seq = (ctx + p.part_tokens - 1) / p.part_tokens;
  const int npass = (tok1 - tok0 + kRowsPerPass - 1) / kRowsPerPass;

  // Physical ids of this partition's blocks, one per lane (clamped into the
  // pool so a corrupt table cannot read outside the caches).
  int lane_block = 0;
  if constexpr (PAGED) {
    const int b0 = tok0 >> p.log2_block;
    const int nb = ((tok1 - 1) >> p.log2_block) - b0 + 1;
    if (lane < nb) {
      const int id = p.tables[int64_t(s) * p.max_blocks + b0 + lane];
      lane_block = min(max(id, 0), p.num_blocks - 1);
    }
  }

  // First row of pass `pass` (clamped to the last real pass, so padding
  // passes re-read cached rows) and how many of its 8 rows are in the context.
  auto pass_rows = [&](const char* base, int pass, int& live_rows) -> const char* {
    const int t = tok0 + min(pass, npass - 1) * kRowsPerPass;
    live_rows = min(tok1 - t, kRowsPerPass);
    if constexpr (PAGED) {
      const int lb = (t >> p.log2_block) - (tok0 >> p.log2_block);
      const int phys = __builtin_amdgcn_readlane(lane_block, lb);
      return base + (int64_t(phys) * p.num_kv_heads + g) * p.tile_bytes +
             int64_t(t & (p.block_size - 1)) * ROW_BYTES;
    } else {
      return base + (int64_t(s) * p.num_kv_heads + g) * p.region_bytes + int64_t(t) * ROW_BYTES;
    }
  };
  auto rsrc_of = [](const char* rows, int nrows) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rows), 0, nrows * ROW_BYTES, kRawBufferWord3);
  };
  auto load16 = [](__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  };

  // Row loads are buffer loads: a scalar resource for a pass's rows plus a
  // per-lane offset (row r, chunk c) and an immediate per chunk; the hardware
  // range-checks every load against the resource.  Rows past the context are
  // never read: their lanes re-read the pass's last real row, and since their
  // scores are masked to -inf they get weight 0, so the (finite) duplicate
  // contributes exactly nothing.
  auto load_buf = [&](const char* base, uint4 (&buf)[U][NCH], int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int live;
      const auto rs = rsrc_of(pass_rows(base, b * U + u, live), kRowsPerPass);
      const uint32_t off = uint32_t(min(r, live - 1)) * ROW_BYTES + uint32_t(c) * 16;
#pragma unroll
      for (int j = 0; j < NCH; ++j) buf[u][j] = load16(rs, off + j * 128);
    }
  };

  // ---- pass 1: scores, scaled to the log2 domain, into LDS ----------------
  float run_max = -INFINITY;
  uint4 bufA[U][NCH], bufB[U][NCH];
  if constexpr (MFMA) {
    // Lane (m = lane % 16, q4 = lane / 16) holds, of token m of a 16-token
    // tile, elements [32 kk + 8 q4, +8) for step kk -- the A layout of
    // v_mfma_f32_16x16x32 -- and of query head m the same elements as the B
    // operand (zero for m >= G).  The result D[4 q4 + i][m] is the score of
    // token 4 q4 + i for head m.
    const int m = lane & 15;
    const int q4 = lane >> 4;
    uint4 qb[KK];
    {
      const char* qrow = reinterpret_cast<const char*>(p.q) + (head0 + min(m, G - 1)) * ROW_BYTES + q4 * 16;
      const uint32_t keep = m < G ? ~0u : 0u;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint4 v = *reinterpret_cast<const uint4*>(qrow + kk * 64);
        qb[kk] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
      }
    }
    // The two 8-row passes of a tile are consecutive rows of one block (or of
    // the contiguous region), so one resource spans both.
    auto load_tile = [&](uint4 (&kt)[KK], int tile) {
      int live0, live1;
      const char* rows0 = pass_rows(p.k, 2 * tile, live0);
      pass_rows(p.k, 2 * tile + 1, live1);
      const int live = 2 * tile + 1 < npass ? kRowsPerPass + live1 : live0;
      const auto rs = rsrc_of(rows0, 2 * kRowsPerPass);
      const uint32_t off = uint32_t(min(m, live - 1)) * ROW_BYTES + uint32_t(q4) * 16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kt[kk] = load16(rs, off + kk * 64);
    };
    float* sink = lds + lds_rows(p.part_tokens) * G + lane;
    auto score_tile = [&](const uint4 (&kt)[KK], int tile) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = mfma_qk(T{}, kt[kk], qb[kk], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile * 16 + q4 * 4 + i;
        float sc = acc[i] * p.scale_log2e;
        if (tok0 + row >= tok1 || m >= G) sc = -INFINITY;  // past the context, or a padding head
        *(m < G ? lds + row * G + m : sink) = sc;
        run_max = fmaxf(run_max, sc);
      }
    };
    auto load_tiles = [&](uint4 (&kt)[KT][KK], int b) {
#pragma unroll
      for (int t = 0; t < KT; ++t) load_tile(kt[t], b * KT + t);
    };
    auto score_tiles = [&](const uint4 (&kt)[KT][KK], int b) {
#pragma unroll
      for (int t = 0; t < KT; ++t) score_tile(kt[t], b * KT + t);
    };
    const int npairs = (npass + 4 * KT - 1) / (4 * KT);  // pairs of K buffers
    uint4 ktA[KT][KK], ktB[KT][KK];
    load_tiles(ktA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_tiles(ktB, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 0; i < npairs; ++i) {
      score_tiles(ktA, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
      load_tiles(ktA, 2 * i + 2);
      __builtin_amdgcn_sched_barrier(0);
      score_tiles(ktB, 2 * i + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_tiles(ktB, 2 * i + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first V rows start streaming while the weights are formed
    load_buf(p.v, bufA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.v, bufB, 1);
    __builtin_amdgcn_sched_barrier(0);
    // head m's scores sit in lanes m, m+16, m+32, m+48; leave each lane i
    // with the max of head i % G, as the vector-ALU path does
    run_max = fmaxf(run_max, __shfl_xor(run_max, 16));
    run_max = fmaxf(run_max, __shfl_xor(run_max, 32));
    run_max = __shfl(run_max, lane % G);
  } else {
    // Lane (r, c) holds chunks j * 128 + c * 16 of row r of each 8-row pass;
    // the query chunks matching them stay in registers.
    uint4 qc[G][NCH];
    {
      const char* qrow = reinterpret_cast<const char*>(p.q) + head0 * ROW_BYTES + c * 16;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < NCH; ++j)
          qc[h][j] = *reinterpret_cast<const uint4*>(qrow + h * ROW_BYTES + j * 128);
    }
    auto score_buf = [&](const uint4 (&buf)[U][NCH], int b) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pass = b * U + u;
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < NCH; ++j) a = dot_chunk(T{}, buf[u][j], qc[h][j], a);
          sc[h] = row8_sum(a);
        }
        float mine = sc[0];
#pragma unroll
        for (int h = 1; h < G; ++h) mine = (c % G == h) ? sc[h] : mine;
        mine *= p.scale_log2e;
        if (tok0 + pass * kRowsPerPass + r >= tok1) mine = -INFINITY;  // past the context
        // lanes c and c + G hold the same head: both store the same value
        lds[(pass * kRowsPerPass + r) * G + c % G] = mine;
        run_max = fmaxf(run_max, mine);
      }
    };
    const int npairs = (npass + 2 * U - 1) / (2 * U);
    load_buf(p.k, bufA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.k, bufB, 1);
    __builtin_amdgcn_sched_barrier(0);
    // The scheduling barriers keep the order "consume one buffer, refill it,
    // consume the other, refill it", so one buffer is always in flight.
    for (int i = 0; i < npairs; ++i) {
      score_buf(bufA, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.k, bufA, 2 * i + 2);
      __builtin_amdgcn_sched_barrier(0);
      score_buf(bufB, 2 * i + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.k, bufB, 2 * i + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first V rows start streaming while the weights are formed
    load_buf(p.v, bufA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.v, bufB, 1);
    __builtin_amdgcn_sched_barrier(0);
    // lane i's run_max belongs to head i % G: reduce over that head's lanes
#pragma unroll
    for (int mm = G; mm < kWave; mm <<= 1) run_max = fmaxf(run_max, __shfl_xor(run_max, mm));
  }

  // ---- softmax weights -----------------------------------------------------
  // The V pass runs whole pairs of 2U passes; the score pass wrote whole
  // pairs of 16-token tiles (MFMA) or the same 2U-pass pairs.  Rows the V pass
  // reaches beyond the written scores are padding and get weight 0.
  const int npass_v = (npass + 2 * U - 1) / (2 * U) * (2 * U);
  const int rows_k = MFMA ? (npass + 4 * KT - 1) / (4 * KT) * (32 * KT) : npass_v * kRowsPerPass;
  __syncthreads();
  float wsum = 0.f;
  const int nent = npass_v * kRowsPerPass * G;
  const int nent_k = rows_k * G;
  for (int e = lane; e < nent; e += kWave) {  // entry e belongs to head e % G = lane % G
    const float w = e < nent_k ? __builtin_amdgcn_exp2f(lds[e] - run_max) : 0.f;
    lds[e] = w;
    wsum += w;
  }
#pragma unroll
  for (int mm = G; mm < kWave; mm <<= 1) wsum += __shfl_xor(wsum, mm);
  __syncthreads();

  // ---- pass 2: weighted sum of V --------------------------------------------
  float acc[G][NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[h][e] = 0.f;
  auto accumulate_buf = [&](const uint4 (&buf)[U][NCH], int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pass = b * U + u;
      const float* wrow = lds + (pass * kRowsPerPass + r) * G;
      float w[G];
#pragma unroll
      for (int h = 0; h < G; ++h) w[h] = wrow[h];
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        float vv[EPC];
        widen(T{}, buf[u][j], vv);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][j * EPC + e] = fmaf(w[h], vv[e], acc[h][j * EPC + e]);
      }
    }
  };
  const int npairs_v = npass_v / (2 * U);
  for (int i = 0; i < npairs_v; ++i) {
    accumulate_buf(bufA, 2 * i);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.v, bufA, 2 * i + 2);
    __builtin_amdgcn_sched_barrier(0);
    accumulate_buf(bufB, 2 * i + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.v, bufB, 2 * i + 3);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum the 8 row lanes sharing chunk position c (lanes c, c+8, ..., c+56).
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      float x = acc[h][e];
      x += dpp<kRowRor8>(x);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[h][e] = x;
    }

  // Lane h (h < G) holds head h's max and weight sum.
  float head_l[G], head_m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    head_l[h] = __shfl(wsum, h);
    head_m[h] = __shfl(run_max, h);
  }

  if (nparts_seq == 1) {
    // Lane (r, c) writes head r's values at its chunk positions.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (r != h) continue;
      const float inv = 1.f / head_l[h];
      const int64_t row = head0 + h;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int d0 = j * (128 / T::bytes) + c * EPC;
        const float* a = &acc[h][j * EPC];
        if (p.out_f32 || T::bytes == 4) {
          float* o = reinterpret_cast<float*>(p.out) + row * D + d0;
#pragma unroll
          for (int e = 0; e < EPC; e += 4)
            *reinterpret_cast<float4*>(o + e) =
                make_float4(a[e] * inv, a[e + 1] * inv, a[e + 2] * inv, a[e + 3] * inv);
        } else {
          store_narrow(T{}, reinterpret_cast<uint16_t*>(p.out) + row * D + d0, a, inv);
        }
      }
    }
    return;
  }

  // Several partitions: publish this one's (m, l, o) for decode_combine_kernel.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (r != h) continue;
    const int64_t prow = (head0 + h) * p.num_parts + part;
    float* o = p.part_o + prow * D;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int d0 = j * (128 / T::bytes) + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4)
        *reinterpret_cast<float4*>(o + d0 + e) =
            make_float4(acc[h][j * EPC + e], acc[h][j * EPC + e + 1], acc[h][j * EPC + e + 2],
                        acc[h][j * EPC + e + 3]);
    }
    if (c == 0) {
      p.part_ml[prow * 2 + 0] = head_m[h];
      p.part_ml[prow * 2 + 1] = head_l[h];
    }
  }
}

// Merges the partitions of each (sequence, query head):
//   M = max_i m_i,  L = sum_i l_i 2^(m_i - M),  out = sum_i 2^(m_i - M) o_i / L.
// One wave per (sequence, query head).  Lane i holds partition i's (m, l)
// (64 partitions per round), so the max and the sum are wave reductions; each
// lane then owns D / 64 output elements and adds the partitions in index
// order, so the result never depends on the order in which partitions
// finished.  Every load address is known up front, so the loads of a round are
// all in flight together.
template <class T, int D>
__global__ __launch_bounds__(kWave) void decode_combine_kernel(DecodeParams p) {
  const int64_t head = blockIdx.x;  // s * Hq + query head
  const int s = int(head / p.num_q_heads);
  const int lane = threadIdx.x;
  const int ctx = min(p.ctx_lens[s], p.max_ctx);
  if (ctx <= 0) return;
  const int np = (ctx + p.part_tokens - 1) / p.part_tokens;
  if (np <= 1) return;  // the partition kernel wrote this output itself
  constexpr int PER = D / kWave;  // output values per lane
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + head * p.num_parts;
  const float* po = p.part_o + head * p.num_parts * D + lane * PER;

  float M = -INFINITY;
  for (int i = lane; i < np; i += kWave) M = fmaxf(M, ml[i].x);
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));

  float L = 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int base = 0; base < np; base += kWave) {
    const int n = min(np - base, kWave);
    const float2 mine = lane < n ? ml[base + lane] : make_float2(-INFINITY, 0.f);
    const float f = __builtin_amdgcn_exp2f(mine.x - M);  // 0 for lanes past n
    L += mine.y * f;
    int i = 0;
    for (; i + 8 <= n; i += 8) {
      float x[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int k = 0; k < PER; ++k) x[u][k] = po[int64_t(base + i + u) * D + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float fu = __shfl(f, i + u);
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] = fmaf(fu, x[u][k], o[k]);
      }
    }
    for (; i < n; ++i) {
      const float fu = __shfl(f, i);
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = fmaf(fu, po[int64_t(base + i) * D + k], o[k]);
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) L += __shfl_xor(L, m);
  const float inv = 1.f / L;
  const int64_t obase = head * D + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float x = o[k] * inv;
    if constexpr (T::bytes == 4) {
      reinterpret_cast<float*>(p.out)[obase + k] = x;
    } else {
      if (p.out_f32) reinterpret_cast<float*>(p.out)[obase + k] = x;
      else reinterpret_cast<uint16_t*>(p.out)[obase + k] = narrow(T{}, x);
    }
  }
}

// ---- host side ---------------------------------------------------------------

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

struct Plan {
  int part_tokens = 0;
  int num_parts = 0;
  int max_ctx = 0;
  size_t workspace = 0;
  size_t part_o_bytes = 0;
  size_t part_ml_bytes = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared validation of the attention shape; fills the plan.
pa_status plan_decode(int S, int Hq, int Hkv, int D, pa_dtype kv, pa_dtype out, int block,
                      int ctx_bound, int partition, float scale, Plan* plan) {
  if (S < 0 || Hq <= 0 || Hkv <= 0) return fail(PA_E_INVAL, "num_seqs >= 0, heads > 0 required");
  if (!valid_dtype(kv)) return fail(PA_E_UNSUPPORTED, "kv dtype");
  if (out != PA_F32 && out != kv) return fail(PA_E_UNSUPPORTED, "out dtype must be f32 or kv dtype");
  if (Hq % Hkv) return fail(PA_E_INVAL, "num_q_heads must be a multiple of num_kv_heads");
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
  if (D != 64 && D != 128) return fail(PA_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!std::isfinite(scale)) return fail(PA_E_INVAL, "scale must be finite");
  if (ctx_bound <= 0) return fail(PA_E_INVAL, "context bound must be positive");
  const int unit = block > 8 ? block : 8;
  const int cap = block > 0 ? (64 * block < kMaxPartition ? 64 * block : kMaxPartition) : kMaxPartition;
  int pt = partition;
  if (pt == 0) {
    pt = 128;
    for (int cand : {512, 256}) {
      if (cand % unit == 0 && cand <= cap &&
          int64_t(S) * Hkv * ((ctx_bound + cand - 1) / cand) >= kAutoMinUnits) {
        pt = cand;
        break;
      }
    }
  }
  if (pt <= 0 || pt % unit || pt > cap)
    return fail(PA_E_INVAL, "partition_size must be a multiple of 8 and of block_size, at most " +
                                std::to_string(cap));
  plan->part_tokens = pt;
  plan->max_ctx = ctx_bound;
  plan->num_parts = (ctx_bound + pt - 1) / pt;
  if (int64_t(plan->num_parts) * (int64_t(S) + kSeqChunk) * Hkv > INT32_MAX || int64_t(S) * Hq > INT32_MAX)
    return fail(PA_E_UNSUPPORTED, "too many (partition, sequence, head) units for one launch");
  plan->workspace = 0;
  if (plan->num_parts > 1 && S > 0) {
    const size_t rows = size_t(S) * Hq * plan->num_parts;
    plan->part_o_bytes = align256(rows * D * sizeof(float));
    plan->part_ml_bytes = align256(rows * 2 * sizeof(float));
    plan->workspace = plan->part_o_bytes + plan->part_ml_bytes;
  }
  return ok();
}

template <class T, int D, int G, bool PAGED>
void launch_one(const DecodeParams& p, dim3 grid, hipStream_t st) {
  const size_t lds = size_t(lds_floats<G>(p.part_tokens)) * sizeof(float);
  if constexpr (mfma_capable<T, G>()) {
    if (!PAGED || p.block_size >= 16) {
      hipLaunchKernelGGL((decode_partition_kernel<T, D, G, PAGED, true>), grid, dim3(kWave), lds, st, p);
      return;
    }
  }
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G, PAGED, false>), grid, dim3(kWave), lds, st, p);
}

template <class T, int D, bool PAGED>
pa_status launch_g(const DecodeParams& p, int G, int S, int Hkv, hipStream_t st) {
  const int64_t seqs_padded = (int64_t(S) + kSeqChunk - 1) / kSeqChunk * kSeqChunk;
  const dim3 grid(unsigned(int64_t(p.num_parts) * seqs_padded * Hkv));
  switch (G) {
    case 1: launch_one<T, D, 1, PAGED>(p, grid, st); break;
    case 2: launch_one<T, D, 2, PAGED>(p, grid, st); break;
    case 4: launch_one<T, D, 4, PAGED>(p, grid, st); break;
    case 8: launch_one<T, D, 8, PAGED>(p, grid, st); break;
  }
  pa_status ps = launch_status("decode partition kernel");
  if (ps != PA_OK || p.num_parts <= 1) return ps;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(unsigned(int64_t(S) * p.num_q_heads)), dim3(kWave),
                     0, st, p);
  return launch_status("decode combine kernel");
}

template <bool PAGED>
pa_status launch(const DecodeParams& p, pa_dtype kv, int D, int G, int S, int Hkv, hipStream_t st) {
  if (kv == PA_F32) return D == 64 ? launch_g<F32, 64, PAGED>(p, G, S, Hkv, st) : launch_g<F32, 128, PAGED>(p, G, S, Hkv, st);
  if (kv == PA_F16) return D == 64 ? launch_g<F16, 64, PAGED>(p, G, S, Hkv, st) : launch_g<F16, 128, PAGED>(p, G, S, Hkv, st);
  return D == 64 ? launch_g<BF16, 64, PAGED>(p, G, S, Hkv, st) : launch_g<BF16, 128, PAGED>(p, G, S, Hkv, st);
}

pa_status check_paged(const pa_decode_args* a, Plan* plan) {
  if (!a) return fail(PA_E_INVAL, "args is null");
  if (a->block_size != 8 && a->block_size != 16 && a->block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size must be 8, 16 or 32");
  if (a->max_blocks <= 0 || a->num_blocks <= 0)
    return fail(PA_E_INVAL, "max_blocks and num_blocks must be positive");
  const int64_t table_ctx = int64_t(a->max_blocks) * a->block_size;
  if (table_ctx > INT32_MAX) return fail(PA_E_INVAL, "max_blocks * block_size must fit int32");
  if (a->max_ctx < 0 || a->max_ctx > table_ctx)
    return fail(PA_E_INVAL, "max_ctx must be in [0, max_blocks * block_size]");
  const int bound = a->max_ctx ? a->max_ctx : int(table_ctx);
  return plan_decode(a->num_seqs, a->num_q_heads, a->num_kv_heads, a->head_dim, a->kv_dtype,
                     a->out_dtype, a->block_size, bound, a->partition_size, a->scale, plan);
}

pa_status check_contig(const pa_contig_args* a, Plan* plan) {
  if (!a) return fail(PA_E_INVAL, "args is null");
  if (a->capacity <= 0 || a->capacity % 8)
    return fail(PA_E_INVAL, "capacity must be a positive multiple of 8");
  if (a->max_ctx < 0 || a->max_ctx > a->capacity)
    return fail(PA_E_INVAL, "max_ctx must be in [0, capacity]");
  const int bound = a->max_ctx ? a->max_ctx : a->capacity;
  return plan_decode(a->num_seqs, a->num_q_heads, a->num_kv_heads, a->head_dim, a->kv_dtype,
                     a->out_dtype, 0, bound, a->partition_size, a->scale, plan);
}

pa_status check_workspace(const Plan& plan, const void* ws, size_t bytes) {
  if (plan.workspace == 0) return ok();
  if (!ws || bytes < plan.workspace)
    return fail(PA_E_INVAL, "workspace too small: need " + std::to_string(plan.workspace) + " bytes");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(PA_E_INVAL, "workspace must be 256-byte aligned");
  return ok();
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pa_status pa_decode_workspace_bytes(const pa_decode_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PA_E_INVAL, "bytes_out is null");
  Plan plan;
  pa_status st = check_paged(a, &plan);
  if (st != PA_OK) return st;
  *bytes_out = plan.workspace;
  return ok();
}

extern "C" pa_status pa_decode(const pa_decode_args* a, pa_stream stream) {
  Plan plan;
  pa_status st = check_paged(a, &plan);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return ok();
  if (!a->out || !a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->ctx_lens)
    return fail(PA_E_INVAL, "null device pointer");
  st = check_workspace(plan, a->workspace, a->workspace_bytes);
  if (st != PA_OK) return st;
  const int eb = dtype_bytes(a->kv_dtype);
  DecodeParams p{};
  p.out = a->out;
  p.q = a->q;
  p.k = static_cast<const char*>(a->k_cache);
  p.v = static_cast<const char*>(a->v_cache);
  p.tables = a->block_tables;
  p.ctx_lens = a->ctx_lens;
  p.part_o = static_cast<float*>(a->workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + plan.part_o_bytes);
  p.num_seqs = a->num_seqs;
  p.tile_bytes = int64_t(a->block_size) * a->head_dim * eb;
  p.region_bytes = 0;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.block_size = a->block_size;
  p.log2_block = log2_exact(a->block_size);
  p.max_blocks = a->max_blocks;
  p.num_blocks = a->num_blocks;
  p.max_ctx = plan.max_ctx;
  p.part_tokens = plan.part_tokens;
  p.num_parts = plan.num_parts;
  p.out_f32 = a->out_dtype == PA_F32;
  p.scale_log2e = a->scale * 1.4426950408889634f;
  return launch<true>(p, a->kv_dtype, a->head_dim, a->num_q_heads / a->num_kv_heads, a->num_seqs,
                      a->num_kv_heads, static_cast<hipStream_t>(stream));
}

extern "C" pa_status pa_decode_contiguous_workspace_bytes(const pa_contig_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PA_E_INVAL, "bytes_out is null");
  Plan plan;
  pa_status st = check_contig(a, &plan);
  if (st != PA_OK) return st;
  *bytes_out = plan.workspace;
  return ok();
}

extern "C" pa_status pa_decode_contiguous(const pa_contig_args* a, pa_stream stream) {
  Plan plan;
  pa_status st = check_contig(a, &plan);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return ok();
  if (!a->out || !a->q || !a->k || !a->v || !a->ctx_lens) return fail(PA_E_INVAL, "null device pointer");
  st = check_workspace(plan, a->workspace, a->workspace_bytes);
  if (st != PA_OK) return st;
  const int eb = dtype_bytes(a->kv_dtype);
  DecodeParams p{};
  p.out = a->out;
  p.q = a->q;
  p.k = static_cast<const char*>(a->k);
  p.v = static_cast<const char*>(a->v);
  p.tables = nullptr;
  p.ctx_lens = a->ctx_lens;
  p.part_o = static_cast<float*>(a->workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + plan.part_o_bytes);
  p.num_seqs = a->num_seqs;
  p.tile_bytes = 0;
  p.region_bytes = int64_t(a->capacity) * a->head_dim * eb;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.block_size = 8;
  p.log2_block = 3;
  p.max_blocks = 0;
  p.num_blocks = 0;
  p.max_ctx = plan.max_ctx;
  p.part_tokens = plan.part_tokens;
  p.num_parts = plan.num_parts;
  p.out_f32 = a->out_dtype == PA_F32;
  p.scale_log2e = a->scale * 1.4426950408889634f;
  return launch<false>(p, a->kv_dtype, a->head_dim, a->num_q_heads / a->num_kv_heads, a->num_seqs,
                       a->num_kv_heads, static_cast<hipStream_t>(stream));
}
