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
//   * partitions of one sequence are merged by decode_combine_kernel with
//     the log-sum-exp identity.
// Block ids of a partition are fetched once, one per lane, and broadcast
// with readlane, so each pass's base address is a scalar.
#include "device_common.h"

#include <cmath>

namespace pkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kRowsPerPass = 8;
constexpr int kAutoPartition = 256;
constexpr int kMaxPartition = 512;

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

template <class T, int D, int G, bool PAGED>
__global__ __launch_bounds__(kWave) void decode_partition_kernel(DecodeParams p) {
  constexpr int EPC = 16 / T::bytes;          // elements per 16-byte chunk
  constexpr int ROW_BYTES = D * T::bytes;
  constexpr int NCH = ROW_BYTES / 128;        // chunks per lane per row
  constexpr int NV = NCH * EPC;               // values per lane per row (= D / 8)
  constexpr int U = (G >= 8) ? 2 : 4;         // passes per load group
  static_assert(NCH >= 1, "row must span the 8 lanes");

  extern __shared__ float lds[];  // [part_tokens][G]: scores, then weights

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
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

  // Query chunks matching this lane's K chunks.
  uint4 qc[G][NCH];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) + head0 * ROW_BYTES + c * 16;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        qc[h][j] = *reinterpret_cast<const uint4*>(qrow + h * ROW_BYTES + j * 128);
  }

  // Byte offset of this lane's row in pass `pass` (pass index is uniform).
  auto row_offset = [&](int pass) -> int64_t {
    const int t = tok0 + pass * kRowsPerPass;
    if constexpr (PAGED) {
      const int lb = (t >> p.log2_block) - (tok0 >> p.log2_block);
      const int phys = __builtin_amdgcn_readlane(lane_block, lb);
      return (int64_t(phys) * p.num_kv_heads + g) * p.tile_bytes +
             int64_t((t & (p.block_size - 1)) + r) * ROW_BYTES + c * 16;
    } else {
      return (int64_t(s) * p.num_kv_heads + g) * p.region_bytes + int64_t(t + r) * ROW_BYTES +
             c * 16;
    }
  };
  auto load_group = [&](const char* base, uint4 (&buf)[U][NCH], int first_pass) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pass = min(first_pass + u, npass - 1);  // re-read, never overrun
      const char* row = base + row_offset(pass);
#pragma unroll
      for (int j = 0; j < NCH; ++j) buf[u][j] = *reinterpret_cast<const uint4*>(row + j * 128);
    }
  };

  const int ngroups = (npass + U - 1) / U;

  // ---- pass 1: scores ------------------------------------------------------
  float run_max = -INFINITY;  // over this lane's rows, for head c % G
  {
    uint4 cur[U][NCH], nxt[U][NCH];
    load_group(p.k, cur, 0);
    for (int gi = 0; gi < ngroups; ++gi) {
      if (gi + 1 < ngroups) load_group(p.k, nxt, (gi + 1) * U);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pass = gi * U + u;
        if (pass >= npass) break;
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < NCH; ++j) a = dot_chunk(T{}, cur[u][j], qc[h][j], a);
          sc[h] = row8_sum(a);
        }
        float mine = sc[0];
#pragma unroll
        for (int h = 1; h < G; ++h) mine = (c % G == h) ? sc[h] : mine;
        mine *= p.scale_log2e;
        const int t = tok0 + pass * kRowsPerPass + r;
        if (t >= tok1) mine = -INFINITY;
        if (c < G) lds[(pass * kRowsPerPass + r) * G + c] = mine;
        run_max = fmaxf(run_max, mine);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NCH; ++j) cur[u][j] = nxt[u][j];
    }
  }

  // ---- softmax weights -----------------------------------------------------
  // Lane i's run_max belongs to head i % G; reduce over the lanes of that head.
#pragma unroll
  for (int m = G; m < kWave; m <<= 1) run_max = fmaxf(run_max, __shfl_xor(run_max, m));
  __syncthreads();
  float wsum = 0.f;
  const int nent = npass * kRowsPerPass * G;
  for (int e = lane; e < nent; e += kWave) {  // entry e belongs to head e % G = lane % G
    const float w = __builtin_amdgcn_exp2f(lds[e] - run_max);
    lds[e] = w;
    wsum += w;
  }
#pragma unroll
  for (int m = G; m < kWave; m <<= 1) wsum += __shfl_xor(wsum, m);
  __syncthreads();

  // ---- pass 2: weighted sum of V --------------------------------------------
  float acc[G][NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[h][e] = 0.f;
  {
    uint4 cur[U][NCH], nxt[U][NCH];
    load_group(p.v, cur, 0);
    for (int gi = 0; gi < ngroups; ++gi) {
      if (gi + 1 < ngroups) load_group(p.v, nxt, (gi + 1) * U);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pass = gi * U + u;
        if (pass >= npass) break;
        const float* wrow = lds + (pass * kRowsPerPass + r) * G;
        float w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) w[h] = wrow[h];
        const bool tail = tok0 + (pass + 1) * kRowsPerPass > tok1;
        const bool live = tok0 + pass * kRowsPerPass + r < tok1;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          float vv[EPC];
          widen(T{}, cur[u][j], vv);
          if (tail) {
            // rows past the context may hold anything (even NaN): select, never multiply
#pragma unroll
            for (int e = 0; e < EPC; ++e) vv[e] = live ? vv[e] : 0.f;
          }
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][j * EPC + e] = fmaf(w[h], vv[e], acc[h][j * EPC + e]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NCH; ++j) cur[u][j] = nxt[u][j];
    }
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

  // Lane (r, c) writes head r's values at its chunk positions.
  if (nparts_seq == 1) {
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
  } else {
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
}

// Merge the partitions of each (sequence, query head):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p 2^(m_p - M) o_p / L.
// Partitions are visited in index order, so the result is deterministic.
template <class T, int D>
__global__ __launch_bounds__(kWave) void decode_combine_kernel(DecodeParams p) {
  const int qh = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = min(p.ctx_lens[s], p.max_ctx);
  if (ctx <= 0) return;
  const int np = (ctx + p.part_tokens - 1) / p.part_tokens;
  if (np <= 1) return;
  const int64_t head = int64_t(s) * p.num_q_heads + qh;
  const float* ml = p.part_ml + head * p.num_parts * 2;
  const float* po = p.part_o + head * p.num_parts * D;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, ml[2 * i]);
  float L = 0.f;
  for (int i = 0; i < np; ++i) L += ml[2 * i + 1] * __builtin_amdgcn_exp2f(ml[2 * i] - M);
  const float inv = 1.f / L;
  constexpr int PER = D / kWave;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int i = 0; i < np; ++i) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * i] - M);
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = fmaf(f, po[int64_t(i) * D + k * kWave + threadIdx.x], o[k]);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int64_t idx = head * D + k * kWave + threadIdx.x;
    const float x = o[k] * inv;
    if constexpr (T::bytes == 4) {
      reinterpret_cast<float*>(p.out)[idx] = x;
    } else {
      if (p.out_f32) reinterpret_cast<float*>(p.out)[idx] = x;
      else reinterpret_cast<uint16_t*>(p.out)[idx] = narrow(T{}, x);
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
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared validation of the attention shape; fills the plan.
pa_status plan_decode(int S, int Hq, int Hkv, int D, pa_dtype kv, pa_dtype out, int block,
                      int ctx_bound, int partition, float scale, Plan* plan) {
  if (S < 0 || Hq <= 0 || Hkv <= 0) return fail(PA_E_INVAL, "num_seqs >= 0, heads > 0 required");
  if (S > 65535 || Hkv > 65535) return fail(PA_E_UNSUPPORTED, "at most 65535 sequences and KV heads per call");
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
  if (pt == 0) pt = kAutoPartition;
  if (pt <= 0 || pt % unit || pt > cap)
    return fail(PA_E_INVAL, "partition_size must be a multiple of 8 and of block_size, at most " +
                                std::to_string(cap));
  plan->part_tokens = pt;
  plan->max_ctx = ctx_bound;
  plan->num_parts = (ctx_bound + pt - 1) / pt;
  plan->workspace = 0;
  if (plan->num_parts > 1 && S > 0) {
    const size_t rows = size_t(S) * Hq * plan->num_parts;
    plan->part_o_bytes = align256(rows * D * sizeof(float));
    plan->workspace = plan->part_o_bytes + align256(rows * 2 * sizeof(float));
  }
  return ok();
}

template <class T, int D, bool PAGED>
pa_status launch_g(const DecodeParams& p, int G, int S, int Hkv, hipStream_t st) {
  const dim3 grid(p.num_parts, Hkv, S);
  const size_t lds = size_t(p.part_tokens) * G * sizeof(float);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_partition_kernel<T, D, 1, PAGED>), grid, dim3(kWave), lds, st, p); break;
    case 2: hipLaunchKernelGGL((decode_partition_kernel<T, D, 2, PAGED>), grid, dim3(kWave), lds, st, p); break;
    case 4: hipLaunchKernelGGL((decode_partition_kernel<T, D, 4, PAGED>), grid, dim3(kWave), lds, st, p); break;
    case 8: hipLaunchKernelGGL((decode_partition_kernel<T, D, 8, PAGED>), grid, dim3(kWave), lds, st, p); break;
  }
  pa_status ps = launch_status("decode partition kernel");
  if (ps != PA_OK) return ps;
  if (p.num_parts > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.num_q_heads, S), dim3(kWave), 0, st, p);
    return launch_status("decode combine kernel");
  }
  return ok();
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
