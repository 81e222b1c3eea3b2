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
//     with the log-sum-exp identity, in partition order.  For 16-bit caches
//     the weighted sums are stored as f16 under a power-of-two scale per row
//     (record_scale_exp), half the lines of float32 records; float32 caches
//     keep float32 records.  (Merging inside the
//     same launch would need device-scope release/acquire fences per wave;
//     on this GPU those write back and invalidate the XCD's L2 and cost far
//     more than one short extra launch.)
// Loads are double-buffered: while one buffer of rows is being consumed the
// next is in flight, and the first V rows are requested before the softmax.
// Block ids of a partition are fetched once, one per lane, and broadcast
// with readlane, so each pass's base address is a scalar.
#include "decode_params.h"
#include "device_common.h"

#include <algorithm>
#include <cstdlib>
#include <string>
#include <cmath>
#include <map>
#include <mutex>

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
// partition_size 0: fixed partitions of the largest of 512 / 256 / 128 tokens
// that still yields at least this many (sequence, KV head, partition) units,
// about eight waves per compute unit of an MI355X (256 CUs).  Longer
// partitions amortise each wave's fixed costs; enough units keep every CU
// busy.
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

// Sum over the 8 lanes of each position c (lanes c, c + 8, ..., c + 56) of
// V values per lane, scattered: afterwards lane (r = lane / 8, c) holds in
// x[0, V / 8) the sums of values [r V / 8, (r + 1) V / 8).  Three halving
// steps across lane distance 32, 16 and 8; a step pairs value i with value
// i + n / 2 and keeps the first sum in the lanes with that lane bit clear,
// the second in the others.  The distance-32 and -16 steps use the gfx950
// permlane swaps (after swap(a, b) the two results add to a + a' in the low
// lanes and b' + b in the high ones), the distance-8 step a DPP rotation
// within 16-lane rows; all stay on the vector ALU.
template <int V>
__device__ __forceinline__ void reduce_scatter8(float (&x)[V], int lane) {
  static_assert(V % 8 == 0, "8 lanes share each position");
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + V / 2]), false, false);
    x[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i + V / 4]), false, false);
    x[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
  const bool hi = lane & 8;
#pragma unroll
  for (int i = 0; i < V / 8; ++i) {
    const float a = x[i], b = x[i + V / 8];
    x[i] = (hi ? b : a) + dpp<kRowRor8>(hi ? a : b);
  }
}

// x, hidden from the optimiser: values computed from it are recomputed where
// they are used instead of being hoisted out of loops and kept in registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// N consecutive float32 values a[i] * s to o (N a power of 2).
template <int N>
__device__ __forceinline__ void store_run(float* o, const float* a, float s) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(o + i) = make_float4(a[i] * s, a[i + 1] * s, a[i + 2] * s, a[i + 3] * s);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(o) = make_float2(a[0] * s, a[1] * s);
  } else {
    *o = a[0] * s;
  }
}
// The same, rounded to 16 bits.
template <class T, int N>
__device__ __forceinline__ void store_run(T, uint16_t* o, const float* a, float s) {
  if constexpr (N == 1) {
    *o = narrow(T{}, a[0] * s);
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      w[i] = uint32_t(narrow(T{}, a[2 * i] * s)) | (uint32_t(narrow(T{}, a[2 * i + 1] * s)) << 16);
    if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(o) = w[0];
    } else if constexpr (N == 4) {
      *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; i += 4) *reinterpret_cast<uint4*>(o + 2 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
    }
  }
}

// ---- kernels ----------------------------------------------------------------



// Scores run on the vector ALUs (v_dot2 on 16-bit pairs) for every group
// size: 8 lanes share a token row, so each 16-byte load instruction of a wave
// reads whole 128-byte lines.  The matrix-core form of q.K (A = 16 K rows in
// the v_mfma_f32_16x16x32 operand layout) reads only 64 bytes of each of 16
// rows per instruction, twice the L2 requests for the same bytes; measured on
// MI355X it made the shared-prefix batch (mostly L2 hits) 8% slower and gained
// at most 2% elsewhere, and decode has arithmetic to spare (removing the
// score and weighted-sum arithmetic altogether left its time unchanged).

// Passes (of 8 token rows) held by one load buffer; two buffers alternate,
// so up to 2 * passes_per_buffer * 8 rows are in flight per wave, for K and
// for V.
template <int G>
constexpr int passes_per_buffer() { return G <= 2 ? 4 : 2; }

// Rows of LDS scores a partition of `part_tokens` tokens needs: both passes
// run in pairs of buffers (at most 8 passes = 64 rows per pair), so the count
// is rounded up to 64 rows.
__host__ __device__ constexpr int lds_rows(int part_tokens) { return (part_tokens + 63) / 64 * 64; }
template <int G>
__host__ __device__ constexpr int lds_floats(int part_tokens) { return lds_rows(part_tokens) * G; }

// ---- schedule ------------------------------------------------------------------
//
// Fixed partitions: one wave per (partition, KV head, sequence), partition =
// a fixed number of tokens, as on the pages; the hardware dispatcher hands
// units to CUs as slots free up (grid order: unit_of).

// 16-bit caches with G <= 4 fit 128 registers, i.e. 4 waves per SIMD.
template <class T, int D, int G, bool PAGED>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(T::bytes == 2 && G <= 4 ? 4 : 1)))
void decode_kernel(DecodeParams p) {
  constexpr int EPC = 16 / T::bytes;          // elements per 16-byte chunk
  constexpr int ROW_BYTES = D * T::bytes;
  constexpr int NCH = ROW_BYTES / 128;        // chunks per lane per row
  constexpr int NV = NCH * EPC;               // values per lane per row (= D / 8)
  constexpr int U = passes_per_buffer<G>();
  static_assert(NCH >= 1, "row must span the 8 lanes");

  extern __shared__ float lds[];  // [rows][G] scores, then weights

  const int lane_id = threadIdx.x;
  // Lane coordinates (r, c) = (lane / 8, lane % 8) for row work.  They are
  // re-derived at the start of the partition's passes and at its finish
  // (refresh_lane) from an opaque copy of the lane id, so addresses built
  // from them are not hoisted to the top of the kernel, where they would hold
  // registers across every pass.
  int lane = lane_id, r = lane >> 3, c = lane & 7;

  // The partition being reduced: sequence s, KV head g, tokens [tok0, tok1)
  // (at most part_tokens of them).
  int s = 0, g = 0, tok0 = 0, tok1 = 0, npass = 0;
  int64_t head0 = 0;  // first query row of (s, g)
  int lane_block = 0;

  // Lane i keeps, for head i % G, the partition's max and weight sum; acc
  // holds each lane's rows' share of the weighted V sums.
  float acc[G * NV];  // [head][value]; after the reduction, PER sums per lane
  float run_m = -INFINITY, run_l = 0.f;
  // After the reduction lane (r, c) holds sums [r PER, (r + 1) PER) of the
  // flattened (head, value) index: head my_h, values e0 .. e0 + PER - 1 at
  // position c, i.e. PER / RUN runs of RUN consecutive elements of the row.
  constexpr int PER = G * NV / 8;
  constexpr int RUN = PER < EPC ? PER : EPC;
  int my_h = r * PER / NV;
  int e0 = r * PER % NV;
  auto refresh_lane = [&]() {
    const int l = opaque(lane_id);
    lane = l;
    r = l >> 3;
    c = l & 7;
    my_h = r * PER / NV;
    e0 = r * PER % NV;
  };
  auto elem = [&](int q) {  // row element of held sum q
    const int e = e0 + q;
    return (e / EPC) * (128 / T::bytes) + c * EPC + e % EPC;
  };

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
  // nt (a std::bool_constant): load with the non-temporal cache policy.
  auto load16 = [](__amdgpu_buffer_rsrc_t rs, uint32_t off, auto nt) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, decltype(nt)::value ? 2 : 0));
  };

  // Row loads are buffer loads: a scalar resource for a pass's rows plus a
  // per-lane offset (row r, chunk c) and an immediate per chunk; the hardware
  // range-checks every load against the resource.  Rows past the context are
  // never read: their lanes re-read the pass's last real row, and since their
  // scores are masked to -inf they get weight 0, so the (finite) duplicate
  // contributes exactly nothing.
  auto load_buf = [&](const char* base, uint4 (&buf)[U][NCH], int b, auto nt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int live;
      const auto rs = rsrc_of(pass_rows(base, b * U + u, live), kRowsPerPass);
      const uint32_t off = uint32_t(min(r, live - 1)) * ROW_BYTES + uint32_t(c) * 16;
#pragma unroll
      for (int j = 0; j < NCH; ++j) buf[u][j] = load16(rs, off + j * 128, nt);
    }
  };

  // Query registers of the current (s, g): lane (r, c) holds chunks
  // j * 128 + c * 16 of row r of each 8-row pass; the query chunks matching
  // them stay in registers.
  uint4 qc[G][NCH];
  auto load_q = [&]() {
    const char* qrow = reinterpret_cast<const char*>(p.q) + head0 * ROW_BYTES + c * 16;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        qc[h][j] = *reinterpret_cast<const uint4*>(qrow + h * ROW_BYTES + j * 128);
  };

  auto begin_range = [&]() {
    head0 = int64_t(s) * p.num_q_heads + int64_t(g) * G;
    run_m = -INFINITY;
    run_l = 0.f;
  };

  // Reduces tokens [tok0, tok1) into run_m, run_l and acc, loading the rows
  // with the cache policy nt.
  auto reduce = [&](auto nt) {
    refresh_lane();
    npass = (tok1 - tok0 + kRowsPerPass - 1) / kRowsPerPass;
    // Here, so the query registers are free during the V pass; the compiler
    // barrier keeps the loads from being hoisted to the top of the kernel,
    // which would pin them through the K pass set-up.
    asm volatile("" ::: "memory");
    load_q();
    // Physical ids of the partition's blocks, one per lane (clamped into the
    // pool so a corrupt table cannot read outside the caches).
    if constexpr (PAGED) {
      const int b0 = tok0 >> p.log2_block;
      const int nb = ((tok1 - 1) >> p.log2_block) - b0 + 1;
      lane_block = 0;
      if (lane < nb) {
        const int id = p.tables[int64_t(s) * p.max_blocks + b0 + lane];
        lane_block = min(max(id, 0), p.num_blocks - 1);
      }
    }

    // ---- pass 1: scores, scaled to the log2 domain, into LDS --------------
    float cmax = -INFINITY;
    uint4 bufA[U][NCH], bufB[U][NCH];
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
        cmax = fmaxf(cmax, mine);
      }
    };
    const int npairs = (npass + 2 * U - 1) / (2 * U);
    load_buf(p.k, bufA, 0, nt);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.k, bufB, 1, nt);
    __builtin_amdgcn_sched_barrier(0);
    // The scheduling barriers keep the order "consume one buffer, refill it,
    // consume the other, refill it", so one buffer is always in flight.
    for (int i = 0; i < npairs; ++i) {
      score_buf(bufA, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.k, bufA, 2 * i + 2, nt);
      __builtin_amdgcn_sched_barrier(0);
      score_buf(bufB, 2 * i + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.k, bufB, 2 * i + 3, nt);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first V rows start streaming while the weights are formed
    load_buf(p.v, bufA, 0, nt);
    __builtin_amdgcn_sched_barrier(0);
    load_buf(p.v, bufB, 1, nt);
    __builtin_amdgcn_sched_barrier(0);
    // lane i's cmax belongs to head i % G: reduce over that head's lanes
#pragma unroll
    for (int mm = G; mm < kWave; mm <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, mm));

    // ---- softmax weights against the partition's max --------------------------
    // Both passes run whole pairs of 2U passes, so every row the V pass
    // reaches has a score; rows past the context carry -inf and get weight 0.
    const float new_m = cmax;
    const int npass_v = (npass + 2 * U - 1) / (2 * U) * (2 * U);
    __syncthreads();
    float wsum = 0.f;
    const int nent = npass_v * kRowsPerPass * G;
    for (int e = lane; e < nent; e += kWave) {  // entry e belongs to head e % G = lane % G
      const float w = __builtin_amdgcn_exp2f(lds[e] - new_m);
      lds[e] = w;
      wsum += w;
    }
#pragma unroll
    for (int mm = G; mm < kWave; mm <<= 1) wsum += __shfl_xor(wsum, mm);
    run_l = wsum;
    run_m = new_m;
    __syncthreads();

    // ---- pass 2: weighted sum of V ------------------------------------------
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
            for (int e = 0; e < EPC; ++e) acc[h * NV + j * EPC + e] = fmaf(w[h], vv[e], acc[h * NV + j * EPC + e]);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < G * NV; ++i) acc[i] = 0.f;
    const int npairs_v = npass_v / (2 * U);
    for (int i = 0; i < npairs_v; ++i) {
      accumulate_buf(bufA, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.v, bufA, 2 * i + 2, nt);
      __builtin_amdgcn_sched_barrier(0);
      accumulate_buf(bufB, 2 * i + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_buf(p.v, bufB, 2 * i + 3, nt);
      __builtin_amdgcn_sched_barrier(0);
    }

    reduce_scatter8(acc, lane);
  };

  // Finishes the partition: the group's normalised output rows when it is
  // the whole context, else one record per head at rows rec0 + h * rec_stride
  // of the workspace: (max, sum, a) and the weighted sums divided by a (a = 1
  // and float32 values for float32 caches; f16 values under a power-of-two a
  // from record_scale_exp for 16-bit caches).
  auto finish = [&](bool whole, int64_t rec0, int64_t rec_stride) {
    refresh_lane();
    const float my_l = __shfl(run_l, my_h);  // lane h holds head h's max and sum
    const float my_m = __shfl(run_m, my_h);
    if (whole) {
      const float inv = 1.f / my_l;
      const int64_t row = (head0 + my_h) * D;
#pragma unroll
      for (int q = 0; q < PER; q += RUN) {
        float* of = reinterpret_cast<float*>(p.out) + row + elem(q);
        if constexpr (T::bytes == 4) {
          store_run<RUN>(of, acc + q, inv);
        } else {
          if (p.out_f32) store_run<RUN>(of, acc + q, inv);
          else store_run<T, RUN>(T{}, reinterpret_cast<uint16_t*>(p.out) + row + elem(q), acc + q, inv);
        }
      }
      return;
    }
    const int64_t prow = rec0 + my_h * rec_stride;
    float a = 1.f;  // the record's values times a are the weighted sums
    if constexpr (T::bytes == 4) {
#pragma unroll
      for (int q = 0; q < PER; q += RUN)
        store_run<RUN>(reinterpret_cast<float*>(p.part_o) + prow * D + elem(q), acc + q, 1.f);
    } else {
      // The head's row of D sums sits in 64 / G consecutive lanes.
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) amax = fmaxf(amax, fabsf(acc[i]));
#pragma unroll
      for (int mm = 1; mm < kWave / G; mm <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mm));
      const int k = record_scale_exp(amax);
      a = __builtin_ldexpf(1.f, -k);
#pragma unroll
      for (int q = 0; q < PER; q += RUN)
        store_run<F16, RUN>(F16{}, reinterpret_cast<uint16_t*>(p.part_o) + prow * D + elem(q), acc + q,
                            __builtin_ldexpf(1.f, k));
    }
    if (c == 0 && e0 == 0)  // one lane per head
      *reinterpret_cast<float4*>(p.part_ml + prow * 4) = make_float4(my_m, my_l, a, 0.f);
  };

  Unit unit;
  int ctx = 0;
  const int kind = unit_of(blockIdx.x, p, &unit, &ctx);
  if (kind == kUnitNone) return;
  g = unit.g;
  s = unit.s;
  if (kind == kUnitZeroRow) {
    // no context: defined as a zero output row
    const int64_t h0 = int64_t(s) * p.num_q_heads + int64_t(g) * G;
    for (int i = lane; i < G * D; i += kWave) {
      if (p.out_f32 || T::bytes == 4) reinterpret_cast<float*>(p.out)[h0 * D + i] = 0.f;
      else reinterpret_cast<uint16_t*>(p.out)[h0 * D + i] = 0;
    }
    return;
  }
  const int part = unit.part;
  const int from = part * p.part_tokens;
  const int nparts_seq = (ctx + p.part_tokens - 1) / p.part_tokens;
  begin_range();
  tok0 = from;
  tok1 = min(from + p.part_tokens, ctx);
  // Cache policy of the partition's row loads.  A partition that shares a
  // block with the previous or the next sequence at the same position (a
  // fork's or a beam's prefix: such sequences sit next to each other, and the
  // grid runs their units side by side on one XCD) is read again by that
  // unit at about the same time, so its rows take the default policy and the
  // re-reads hit the L2.  Every other partition is read once in the launch,
  // and its rows are loaded non-temporal (measured on MI355X: private
  // contexts stream 9-12% faster, while shared prefixes loaded that way miss
  // the L2 and run ~20% slower).  The contiguous layout holds no shared rows.
  bool stream = true;
  if constexpr (PAGED) {
    const int b0 = tok0 >> p.log2_block;
    const int nb = ((tok1 - 1) >> p.log2_block) - b0 + 1;
    bool mine = false;
    if (lane < nb) {
      const int64_t j = b0 + lane;
      const int id = p.tables[int64_t(s) * p.max_blocks + j];
      if (s > 0) mine = p.tables[int64_t(s - 1) * p.max_blocks + j] == id;
      if (s + 1 < p.num_seqs) mine = mine || p.tables[int64_t(s + 1) * p.max_blocks + j] == id;
    }
    stream = __builtin_amdgcn_ballot_w64(mine) == 0;
  }
  if (stream) reduce(std::true_type{});
  else reduce(std::false_type{});
  finish(nparts_seq == 1, head0 * p.num_parts + part, p.num_parts);
}

// Merges the records of each (sequence, query head):
//   M = max_i m_i,  L = sum_i l_i 2^(m_i - M),  out = sum_i 2^(m_i - M) o_i / L.
// One wave per (sequence, query head).  Lane i holds record i's (m, l)
// (64 records per round), so the max and the sum are wave reductions; each
// lane then owns D / 64 output elements and adds the records in token order,
// so the result never depends on the order in which the records were written.
// Every load address is known up front: with at most 64 records (the usual
// case) the (m, l) loads and the first 8 records' outputs are in flight
// together, so the merge waits on memory about once after the context length.
// Record i = partition i, row (head * num_parts + i): (m, l, a) and D values
// whose products with a are the weighted sums (float32 values and a = 1 for
// float32 caches, f16 values under a power-of-two a for the others).
template <class T, int D>
__global__ __launch_bounds__(kWave) void decode_combine_kernel(DecodeParams p) {
  const int64_t head = blockIdx.x;  // s * Hq + query head
  const int s = int(head / p.num_q_heads);
  const int lane = threadIdx.x;
  const int ctx = min(p.ctx_lens[s], p.max_ctx);
  constexpr int PER = D / kWave;  // output values per lane
  const int64_t obase = head * D + lane * PER;
  if (ctx <= 0) return;  // the partition kernel wrote the zero row
  const int np = (ctx + p.part_tokens - 1) / p.part_tokens;
  if (np <= 1) return;  // the partition kernel wrote this output itself
  const int64_t rec0 = head * p.num_parts;
  auto rec = [&](int i) -> int64_t { return rec0 + i; };
  const float4* ml = reinterpret_cast<const float4*>(p.part_ml);
  const int64_t po = lane * PER;  // this lane's first value in a record row
  auto value = [&](int64_t r, int k) -> float {
    if constexpr (T::bytes == 4) return reinterpret_cast<const float*>(p.part_o)[r * D + po + k];
    else return widen1(F16{}, reinterpret_cast<const uint16_t*>(p.part_o)[r * D + po + k]);
  };

  // Outputs are read kBatch records at a time, all loads of a batch issued
  // before any is used (an index past the round's last record re-reads that
  // record, and its term is skipped), so a batch costs one memory round trip;
  // records are added in token order.
  constexpr int kBatch = 8;
  float x[kBatch][PER];
  auto load_batch = [&](int base, int i0, int n) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t r = rec(base + min(i0 + u, n - 1));
#pragma unroll
      for (int k = 0; k < PER; ++k) x[u][k] = value(r, k);
    }
  };
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  // f: lane i holds the weight of the round's record i.  Terms past the
  // round's end are computed and dropped by a select (a branch would let the
  // compiler sink their loads behind it, one round trip each).
  auto add_batch = [&](int i0, int n, float f) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = i0 + u < n;
      const float fu = __shfl(f, min(i0 + u, kWave - 1));
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float y = fmaf(fu, x[u][k], o[k]);
        o[k] = live ? y : o[k];
      }
    }
  };
  auto wave_max = [](float v) {
#pragma unroll
    for (int mm = 1; mm < kWave; mm <<= 1) v = fmaxf(v, __shfl_xor(v, mm));
    return v;
  };

  float L = 0.f;
  if (np <= kWave) {
    // One round: lane i holds record i's (m, l).  Its load and the first
    // batch's output loads go out together, ahead of the reductions.
    const float4 mine = lane < np ? ml[rec(lane)] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
    load_batch(0, 0, np);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
    const float M = wave_max(mine.x);
    const float f = __builtin_amdgcn_exp2f(mine.x - M);  // 0 for lanes past np
    L = mine.y * f;
    add_batch(0, np, f * mine.z);
    for (int i0 = kBatch; i0 < np; i0 += kBatch) {
      load_batch(0, i0, np);
      add_batch(i0, np, f * mine.z);
    }
  } else {
    // Rounds of 64 records against the maximum over all of them.
    float M = -INFINITY;
    for (int i = lane; i < np; i += kWave) M = fmaxf(M, ml[rec(i)].x);
    M = wave_max(M);
    for (int base = 0; base < np; base += kWave) {
      const int n = min(np - base, kWave);
      const float4 mine = lane < n ? ml[rec(base + lane)] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
      const float f = __builtin_amdgcn_exp2f(mine.x - M);  // 0 for lanes past n
      L += mine.y * f;
      for (int i0 = 0; i0 < n; i0 += kBatch) {
        load_batch(base, i0, n);
        add_batch(i0, n, f * mine.z);
      }
    }
  }
#pragma unroll
  for (int mm = 1; mm < kWave; mm <<= 1) L += __shfl_xor(L, mm);
  const float inv = 1.f / L;
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

// ---- input validation (debug) -------------------------------------------------
//
// The decode kernels clamp table entries into the pool instead of checking
// them; these count what a correct caller never passes: contexts above the
// bound, and table entries j < ceil(ctx / B) outside [0, num_blocks).

__global__ __launch_bounds__(kWave) void clear_count_kernel(int32_t* count) {
  if (threadIdx.x == 0) *count = 0;
}

// One wave per sequence; lanes walk the table row.
__global__ __launch_bounds__(kWave) void validate_kernel(const int32_t* tables, const int32_t* ctx_lens,
                                                         int max_blocks, int block_size, int num_blocks,
                                                         int max_ctx, int32_t* count) {
  const int s = blockIdx.x;
  const int ctx = ctx_lens[s];
  int bad = 0;
  if (threadIdx.x == 0 && ctx > max_ctx) bad = 1;
  const int nb = ctx > 0 ? min((min(ctx, max_ctx) + block_size - 1) / block_size, max_blocks) : 0;
  for (int j = threadIdx.x; j < nb; j += kWave) {
    const int id = tables[int64_t(s) * max_blocks + j];
    bad += (id < 0 || id >= num_blocks) ? 1 : 0;
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) bad += __shfl_xor(bad, m);
  if (threadIdx.x == 0 && bad) atomicAdd(count, bad);
}

// ---- host side ---------------------------------------------------------------

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

struct Plan {
  int part_tokens = 0;   // partition length
  int num_parts = 0;     // partitions of the longest context
  int full_parts = 0;    // partitions that can be full under the bound
  int max_ctx = 0;
  size_t workspace = 0;
  size_t part_o_off = 0, part_ml_off = 0;
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
  if (int64_t(S) * Hq > INT32_MAX) return fail(PA_E_UNSUPPORTED, "too many (sequence, head) rows");
  plan->max_ctx = ctx_bound;
  plan->workspace = 0;
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
    return fail(PA_E_INVAL, "partition_size must be 0 or a multiple of 8 and of block_size, at most " +
                                std::to_string(cap));
  plan->part_tokens = pt;
  plan->num_parts = (ctx_bound + pt - 1) / pt;
  plan->full_parts = ctx_bound / pt;
  if ((int64_t(plan->full_parts) * padded_seqs(S) + S) * Hkv > INT32_MAX)
    return fail(PA_E_UNSUPPORTED, "too many (partition, sequence, head) units for one launch");
  if (plan->num_parts > 1 && S > 0) {
    const size_t rows = size_t(S) * Hq * plan->num_parts;
    // values: float32 for float32 caches, else f16; (m, l, a, unused) per row
    const size_t value_bytes = kv == PA_F32 ? sizeof(float) : sizeof(uint16_t);
    plan->part_o_off = 0;
    plan->part_ml_off = align256(rows * D * value_bytes);
    plan->workspace = plan->part_ml_off + align256(rows * 4 * sizeof(float));
  }
  return ok();
}

// Points the parameter block at the workspace regions of the plan.
void bind_workspace(const Plan& plan, void* ws, DecodeParams* p) {
  char* base = static_cast<char*>(ws);
  p->part_o = base + plan.part_o_off;
  p->part_ml = reinterpret_cast<float*>(base + plan.part_ml_off);
}

template <class T, int D, int G, bool PAGED>
void launch_decode(const DecodeParams& p, dim3 grid, hipStream_t st) {
  const size_t lds = size_t(lds_floats<G>(p.part_tokens)) * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<T, D, G, PAGED>), grid, dim3(kWave), lds, st, p);
}

template <class T, int D, int G, bool PAGED>
pa_status launch_group(DecodeParams p, const Plan& plan, int S, int Hkv, hipStream_t st) {
  const dim3 combine_grid(unsigned(int64_t(S) * p.num_q_heads));
  launch_decode<T, D, G, PAGED>(p, dim3(unsigned(grid_units(p))), st);
  pa_status ps = launch_status("decode partition kernel");
  if (ps != PA_OK || p.num_parts <= 1) return ps;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), combine_grid, dim3(kWave), 0, st, p);
  return launch_status("decode combine kernel");
}

template <class T, int D, bool PAGED>
pa_status launch_g(const DecodeParams& p, const Plan& plan, int G, int S, int Hkv, hipStream_t st) {
  switch (G) {
    case 1: return launch_group<T, D, 1, PAGED>(p, plan, S, Hkv, st);
    case 2: return launch_group<T, D, 2, PAGED>(p, plan, S, Hkv, st);
    case 4: return launch_group<T, D, 4, PAGED>(p, plan, S, Hkv, st);
    default: return launch_group<T, D, 8, PAGED>(p, plan, S, Hkv, st);
  }
}

template <bool PAGED>
pa_status launch(const DecodeParams& p, const Plan& plan, pa_dtype kv, int D, int G, int S, int Hkv,
                 hipStream_t st) {
  if (kv == PA_F32)
    return D == 64 ? launch_g<F32, 64, PAGED>(p, plan, G, S, Hkv, st) : launch_g<F32, 128, PAGED>(p, plan, G, S, Hkv, st);
  if (kv == PA_F16)
    return D == 64 ? launch_g<F16, 64, PAGED>(p, plan, G, S, Hkv, st) : launch_g<F16, 128, PAGED>(p, plan, G, S, Hkv, st);
  return D == 64 ? launch_g<BF16, 64, PAGED>(p, plan, G, S, Hkv, st) : launch_g<BF16, 128, PAGED>(p, plan, G, S, Hkv, st);
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
  pa_dtype compute = a->kv_dtype;
  if (a->kv_dtype == PA_FP8_E4M3) {
    if (a->q_dtype != PA_F16 && a->q_dtype != PA_BF16)
      return fail(PA_E_UNSUPPORTED, "E4M3 caches need q_dtype PA_F16 or PA_BF16");
    if (!(a->k_scale > 0.f) || !(a->v_scale > 0.f) || !std::isfinite(a->k_scale) || !std::isfinite(a->v_scale))
      return fail(PA_E_INVAL, "k_scale and v_scale must be finite and positive");
    compute = a->q_dtype;
  } else if (a->q_dtype != a->kv_dtype) {
    // the kernels read q at the cache's element size
    return fail(PA_E_INVAL, "q_dtype must equal kv_dtype for f32, f16 and bf16 caches");
  }
  return plan_decode(a->num_seqs, a->num_q_heads, a->num_kv_heads, a->head_dim, compute,
                     a->out_dtype, a->block_size, bound, a->partition_size, a->scale, plan);
}


pa_status check_contig(const pa_contig_args* a, Plan* plan) {
  if (!a) return fail(PA_E_INVAL, "args is null");
  if (a->capacity <= 0 || a->capacity % 8)
    return fail(PA_E_INVAL, "capacity must be a positive multiple of 8");
  if (a->max_ctx < 0 || a->max_ctx > a->capacity)
    return fail(PA_E_INVAL, "max_ctx must be in [0, capacity]");
  if (a->q_dtype != a->kv_dtype) return fail(PA_E_INVAL, "q_dtype must equal kv_dtype");
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

// Scratch for the debug check inside pa_decode: one counter per device,
// addressed through hipGetSymbolAddress (the host-side name is not a device
// address).
__device__ int32_t g_debug_count;

bool debug_checks() {
  static const bool on = [] {
    const char* v = std::getenv("PAGEDKV_DEBUG");
    return v && *v && std::string(v) != "0";
  }();
  return on;
}

pa_status launch_validate(const pa_decode_args* a, int max_ctx, int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(kWave), 0, st, count);
  pa_status ps = launch_status("validation clear kernel");
  if (ps != PA_OK) return ps;
  hipLaunchKernelGGL(validate_kernel, dim3(unsigned(a->num_seqs)), dim3(kWave), 0, st, a->block_tables, a->ctx_lens,
                     a->max_blocks, a->block_size, a->num_blocks, max_ctx, count);
  return launch_status("validation kernel");
}

// With PAGEDKV_DEBUG set, pa_decode validates its device inputs first: the
// stream is synchronised and the call fails with PA_E_INVAL, launching
// nothing else, if any context or table entry is out of range.
pa_status debug_validate(const pa_decode_args* a, int max_ctx, hipStream_t st) {
  int32_t* count = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&count), HIP_SYMBOL(g_debug_count)) != hipSuccess)
    return fail(PA_E_HIP, "hipGetSymbolAddress(debug counter) failed");
  pa_status ps = launch_validate(a, max_ctx, count, st);
  if (ps != PA_OK) return ps;
  int32_t bad = 0;
  if (hipMemcpyAsync(&bad, count, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(PA_E_HIP, "reading the validation count failed");
  if (bad) return fail(PA_E_INVAL, "PAGEDKV_DEBUG: " + std::to_string(bad) + " out-of-range context or table entries");
  return ok();
}

// ---- allocation-free decode ------------------------------------------------
//
// For callers that may not allocate device memory: the split-context records
// go to a file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy of the array until the process ends.
// The host-side name of the array is not a device address, so its address on
// each device is looked up once (hipGetSymbolAddress, with that device
// current) and only that pointer is handed to kernels.

constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

pa_status static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> by_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_E_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it == by_device.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    it = by_device.emplace(dev, p).first;
  }
  *ptr = it->second;
  return ok();
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pa_status pa_decode_validate(const pa_decode_args* a, int32_t* count, pa_stream stream) {
  Plan plan;
  pa_status st = check_paged(a, &plan);
  if (st != PA_OK) return st;
  if (!count) return fail(PA_E_INVAL, "count is null");
  if (a->num_seqs == 0) {
    hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(kWave), 0, static_cast<hipStream_t>(stream), count);
    return launch_status("validation clear kernel");
  }
  if (!a->block_tables || !a->ctx_lens) return fail(PA_E_INVAL, "null device pointer");
  return launch_validate(a, plan.max_ctx, count, static_cast<hipStream_t>(stream));
}

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
  if (debug_checks()) {
    st = debug_validate(a, plan.max_ctx, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
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
  bind_workspace(plan, a->workspace, &p);
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
  p.full_parts = plan.full_parts;
  p.out_f32 = a->out_dtype == PA_F32;
  p.scale_log2e = a->scale * 1.4426950408889634f;
  p.v_scale = 1.f;
  const int G = a->num_q_heads / a->num_kv_heads;
  if (a->kv_dtype == PA_FP8_E4M3) {
    p.scale_log2e = float(double(a->scale) * double(a->k_scale) * 1.4426950408889634);
    p.v_scale = a->v_scale;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    st = launch_decode_fp8_partitions(p, a->q_dtype, a->head_dim, G, hs);
    if (st != PA_OK || p.num_parts <= 1) return st;
    const dim3 cg(unsigned(int64_t(a->num_seqs) * a->num_q_heads));
    const bool d64 = a->head_dim == 64;
    if (a->q_dtype == PA_F16) {
      if (d64) hipLaunchKernelGGL((decode_combine_kernel<F16, 64>), cg, dim3(kWave), 0, hs, p);
      else hipLaunchKernelGGL((decode_combine_kernel<F16, 128>), cg, dim3(kWave), 0, hs, p);
    } else {
      if (d64) hipLaunchKernelGGL((decode_combine_kernel<BF16, 64>), cg, dim3(kWave), 0, hs, p);
      else hipLaunchKernelGGL((decode_combine_kernel<BF16, 128>), cg, dim3(kWave), 0, hs, p);
    }
    return launch_status("decode combine kernel");
  }
  return launch<true>(p, plan, a->kv_dtype, a->head_dim, G, a->num_seqs,
                      a->num_kv_heads, static_cast<hipStream_t>(stream));
}

extern "C" size_t pa_decode_static_max_bytes(void) { return kStaticScratchBytes; }

extern "C" pa_status pa_decode_static(const pa_decode_args* a, pa_stream stream) {
  Plan plan;
  pa_status st = check_paged(a, &plan);
  if (st != PA_OK) return st;
  if (plan.workspace > kStaticScratchBytes)
    return fail(PA_E_UNSUPPORTED, "this batch needs " + std::to_string(plan.workspace) +
                                      " bytes of split-context records, above the static maximum of " +
                                      std::to_string(kStaticScratchBytes));
  pa_decode_args local = *a;
  local.workspace = nullptr;
  local.workspace_bytes = 0;
  if (plan.workspace > 0 && a->num_seqs > 0) {
    st = static_scratch(&local.workspace);
    if (st != PA_OK) return st;
    local.workspace_bytes = kStaticScratchBytes;
  }
  return pa_decode(&local, stream);
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
  bind_workspace(plan, a->workspace, &p);
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
  p.full_parts = plan.full_parts;
  p.out_f32 = a->out_dtype == PA_F32;
  p.scale_log2e = a->scale * 1.4426950408889634f;
  return launch<false>(p, plan, a->kv_dtype, a->head_dim, a->num_q_heads / a->num_kv_heads, a->num_seqs,
                       a->num_kv_heads, static_cast<hipStream_t>(stream));
}

