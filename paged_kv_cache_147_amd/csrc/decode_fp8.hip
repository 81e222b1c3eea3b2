// Paged decode attention over an E4M3 (8-bit float) KV cache, for gfx950.
//
// Same result as the 16-bit kernels, out[s][h] = sum_t softmax_t(scale q.K_t) V_t
// with K_t = value(code) * k_scale and V_t = value(code) * v_scale: a
// quantised cache halves the bytes decode must stream, the one lever on its
// byte floor besides fewer KV heads and shorter contexts ("Paged Attention"
// (daiw.org), 量化, the boxed warning).
//
// decode_fp8_kernel: one wave per (partition, KV head, sequence) unit of the
// fixed-partition schedule, writing the same outputs and records as
// decode_kernel, with both contractions on the matrix cores.  Every E4M3
// value is exactly a float16 and a bfloat16 value, so codes are widened
// without rounding: K to q's 16-bit type, V to f16 whatever q's type, so
// that p.V takes P rounded once to f16 (11 significant bits); the only other
// roundings are the float32 accumulation's.
//
// Per 32-token step, lane (m16 = lane % 16, q4 = lane / 16), written for
// head_dim 128 (at 64: two score steps, one 16-byte K piece, 4 V bytes per
// row and 4 output blocks):
//   * S^T = K Q^T per 16-token tile (v_mfma_f32_16x16x32): A = the tile's K
//     rows, lane m16 holding row m16, bytes 16 q4 .. +15 and 64 + 16 q4 ..
//     +15 (MFMA step kk takes bytes 64 (kk / 2) + 16 q4 + 8 (kk % 2) .. +7;
//     q's head_dim is read in the same order); B = the group's queries,
//     column m16 (zero for m16 >= G).  Lane (m16, q4) ends with tokens
//     16 h + 4 q4 + i of head m16, i < 4, of tiles h = 0, 1;
//   * softmax online, against a running max shared by the 4 lanes of a head
//     and moved only when a score passes it by more than kFp8Slack (log2
//     units), so most steps rescale nothing;
//   * O^T += V^T P^T: the 32 tokens of the contraction are ordered so that
//     lane group q4 holds tokens 4 q4 .. 4 q4 + 3 and 16 + 4 q4 .. +3 --
//     exactly the 8 probabilities the lane already owns, so P^T is formed
//     in place.  V^T needs those 8 tokens of one column in a lane: lane
//     (m16, q4) loads 8 bytes (columns 8 m16 .. 8 m16 + 7) of each of its 8
//     rows and regroups bytes into token pairs in registers, so output block
//     nn of O^T is head_dim column 8 m16 + nn.  V codes widen to f16 and P
//     enters rounded once to f16: one f16 MFMA per block.
// Rows are read with buffer loads from a scalar resource per 16-token span and
// a fixed per-lane offset (global loads with per-lane addresses when 8-token
// blocks put two blocks in a span); two steps of loads are in flight
// (register double buffering).  Rows past the partition's end are read from
// the last block (always inside the pool): their scores are masked and their
// V codes zeroed, so a stale NaN code there cannot reach the sums.
#include "decode_params.h"
#include "device_common.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr float kFp8Slack = 8.f;
// Word 3 of a raw (untyped) buffer resource on gfx9-family GPUs: 32-bit data
// format, no swizzle; loads through it are plain byte-addressed loads.
constexpr int kRawBufferWord3 = 0x00020000;

typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma(BF16, u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma(F16, u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                 0, 0, 0);
}

// Two E4M3 codes (bytes 0 and 1 of w, or 2 and 3 when HI) -> their values as
// two packed 16-bit floats of type T, in one gfx950 conversion with a scale
// of 1 (every E4M3 value is exactly a float16 and a bfloat16 value; checked
// on all byte pairs, NaN codes give NaN).  Issued as inline assembly: the
// compiler's own model of this instruction's two result halves has been
// seen to merge them wrongly when one half is extracted.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(BF16, uint32_t w) {
  uint32_t r;
  if constexpr (HI) asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  else asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(F16, uint32_t w) {
  uint32_t r;
  if constexpr (HI) asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  else asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}

// Bytes of two rows' words a (row e) and b (row e + 1), regrouped into token
// pairs: (a0, b0, a2, b2) and (a1, b1, a3, b3).
__device__ __forceinline__ uint32_t pair_even(uint32_t a, uint32_t b) {
  return (a & 0x00ff00ffu) | ((b & 0x00ff00ffu) << 8);
}
__device__ __forceinline__ uint32_t pair_odd(uint32_t a, uint32_t b) {
  return ((a >> 8) & 0x00ff00ffu) | (b & 0xff00ff00u);
}

// Max / sum with the lane 16 or 32 positions away (the same head's lanes).
__device__ __forceinline__ float fp8_max_xor16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float fp8_max_xor32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float fp8_sum_xor16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float fp8_sum_xor32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// One step's rows in registers: K of both tiles (D / 64 16-byte pieces each)
// and D / 16 bytes of each of the lane's 8 V rows.
template <int D>
struct Fp8Rows {
  uint4 k[2][D / 64];
  uint2 v[8];  // .y unused when D == 64
};

// SPLIT: 8-token blocks, so a 16-token span covers two blocks.
template <class T, int D, int G, bool SPLIT>
__global__ __launch_bounds__(kWave) void decode_fp8_kernel(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int KK = D / 32;  // score MFMA steps
  constexpr int NN = D / 16;  // output column blocks = V bytes per lane and row
  constexpr int KP = D / 64;  // 16-byte K pieces per lane and row
  constexpr int ROW = D;      // bytes per cached row
  const int lane = threadIdx.x, m16 = lane & 15, q4 = lane >> 4;
  Unit unit;
  int ctx = 0;
  const int kind = unit_of(blockIdx.x, p, &unit, &ctx);
  if (kind == kUnitNone) return;
  const int g = unit.g, s = unit.s, part = unit.part;
  const int64_t head0 = int64_t(s) * p.num_q_heads + int64_t(g) * G;
  if (kind == kUnitZeroRow) {  // no context: defined as a zero output row
    for (int i = lane; i < G * D; i += kWave) {
      if (p.out_f32) reinterpret_cast<float*>(p.out)[head0 * D + i] = 0.f;
      else reinterpret_cast<uint16_t*>(p.out)[head0 * D + i] = 0;
    }
    return;
  }
  const int tok0 = part * p.part_tokens;
  const int tok1 = min(tok0 + p.part_tokens, ctx);
  const int nsteps = (tok1 - tok0 + 31) >> 5;

  // Physical ids of the partition's blocks (at most 64), one per lane,
  // clamped into the pool.
  const int b0 = tok0 >> p.log2_block;
  const int lb_last = ((tok1 - 1) >> p.log2_block) - b0;
  int lane_block = 0;
  if (lane <= lb_last) {
    const int id = p.tables[int64_t(s) * p.max_blocks + b0 + lane];
    lane_block = min(max(id, 0), p.num_blocks - 1);
  }
  // Address of row k (0..15) of the 16-token span starting at token tb.
  auto row_ptr = [&](const char* cache, int tb, int k) -> const char* {
    const int lb = min((tb >> p.log2_block) - b0, lb_last);
    const int phys = __builtin_amdgcn_readlane(lane_block, lb);
    const char* base = cache + (int64_t(phys) * p.num_kv_heads + g) * p.tile_bytes +
                       int64_t(tb & (p.block_size - 1)) * ROW;
    if constexpr (!SPLIT) {
      return base + k * ROW;
    } else {
      const int phys2 = __builtin_amdgcn_readlane(lane_block, min(lb + 1, lb_last));
      const char* base2 = cache + (int64_t(phys2) * p.num_kv_heads + g) * p.tile_bytes;
      return (k < 8 ? base : base2) + (k & 7) * ROW;
    }
  };
  // Blocks of >= 16 tokens: a span is 16 consecutive rows of one block, read
  // as buffer loads from a scalar resource over those 16 rows plus a fixed lane
  // offset and an immediate (no per-lane address arithmetic).
  const uint32_t koff = uint32_t(m16) * ROW + 16u * q4;          // K: row m16, bytes 16 q4 (+64)
  const uint32_t voff = uint32_t(4 * q4) * ROW + uint32_t(NN) * m16;  // V: row 4 q4 (+j), bytes NN m16
  // Loads are issued for every step of the double-buffered loop, also the
  // one past the last: it gets a resource of zero bytes, so it moves nothing
  // and returns zeros, and the wait counts stay the same on every path (a
  // load under a branch would make the compiler drain all loads instead).
  auto span_rsrc = [&](const char* cache, int tb, bool live) {
    const int lb = min((tb >> p.log2_block) - b0, lb_last);
    const int phys = __builtin_amdgcn_readlane(lane_block, lb);
    const char* base = cache + (int64_t(phys) * p.num_kv_heads + g) * p.tile_bytes +
                       int64_t(tb & (p.block_size - 1)) * ROW;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, live ? 16 * ROW : 0, kRawBufferWord3);
  };
  auto load = [&](Fp8Rows<D>& b, int st_in) {
    const bool live = st_in < nsteps;
    const int st = min(st_in, nsteps - 1);
    const int t0 = tok0 + 32 * st;
    if constexpr (!SPLIT) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto rk = span_rsrc(p.k, t0 + 16 * h, live);
#pragma unroll
        for (int j = 0; j < KP; ++j)
          b.k[h][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * j, 0, 0));
        const auto rv = span_rsrc(p.v, t0 + 16 * h, live);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (D == 128)
            b.v[4 * h + j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff + j * ROW, 0, 0));
          else
            b.v[4 * h + j] = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(rv, voff + j * ROW, 0, 0), 0u);
        }
      }
    } else {
      // two blocks per span: per-lane addresses; a step past the last
      // re-reads the last step's rows (cached) instead
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* r = row_ptr(p.k, t0 + 16 * h, m16);
#pragma unroll
        for (int j = 0; j < KP; ++j) b.k[h][j] = *reinterpret_cast<const uint4*>(r + 64 * j + 16 * q4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const char* r0 = row_ptr(p.v, t0, 4 * q4 + j) + NN * m16;
        const char* r1 = row_ptr(p.v, t0 + 16, 4 * q4 + j) + NN * m16;
        if constexpr (D == 128) {
          b.v[j] = *reinterpret_cast<const uint2*>(r0);
          b.v[4 + j] = *reinterpret_cast<const uint2*>(r1);
        } else {
          b.v[j] = make_uint2(*reinterpret_cast<const uint32_t*>(r0), 0u);
          b.v[4 + j] = make_uint2(*reinterpret_cast<const uint32_t*>(r1), 0u);
        }
      }
    }
  };

  // Queries: lane (m16, q4), step kk holds head m16's elements
  // 64 (kk / 2) + 16 q4 + 8 (kk % 2) .. +7 (zero for padding heads); a
  // negative scale flips their signs so the score scale c is positive.
  const float sl = p.scale_log2e;
  const uint32_t flip = sl < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(sl), 1e-30f);
  const float slack = kFp8Slack / c;  // in raw score units
  u32x4_t qb[KK];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) + (head0 + min(m16, G - 1)) * (2 * D);
    const uint32_t keep = m16 < G ? ~0u : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 128 * (kk >> 1) + 32 * q4 + 16 * (kk & 1));
      qb[kk] = u32x4_t{(v.x ^ flip) & keep, (v.y ^ flip) & keep, (v.z ^ flip) & keep, (v.w ^ flip) & keep};
    }
  }

  float run_m = -INFINITY, run_mc = -INFINITY, run_l = 0.f;  // raw max, max * c, this lane's sum
  f32x4_t o[NN];
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Fp8Rows<D>& b, int st, auto masked_tag) {
    constexpr bool masked = decltype(masked_tag)::value;  // the step runs past tok1
    const int t0 = tok0 + 32 * st;
    f32x4_t sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 w = b.k[h][kk >> 1];
        const uint32_t lo = (kk & 1) ? w.z : w.x, hi = (kk & 1) ? w.w : w.y;
        const u32x4_t a = {e4m3_pair<false>(T{}, lo), e4m3_pair<true>(T{}, lo), e4m3_pair<false>(T{}, hi),
                           e4m3_pair<true>(T{}, hi)};
        sacc[h] = mfma(T{}, a, qb[kk], sacc[h]);
      }
    }
    // x[e]: token 16 (e / 4) + 4 q4 + e % 4 of the step, head m16
    float x[8], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = sacc[e >> 2][e & 3];
      if (masked && t0 + 16 * (e >> 2) + 4 * q4 + (e & 3) >= tok1) x[e] = -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    if (__builtin_amdgcn_ballot_w64(mx > run_m + slack)) {
      const float mnew = fmaxf(run_m, fp8_max_xor32(fp8_max_xor16(mx)));
      const float f = __builtin_amdgcn_exp2f((run_m - mnew) * c);
      run_m = mnew;
      run_mc = mnew * c;
      run_l *= f;
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) o[nn] *= f;
    }
    // P rounded once to f16 (11 significant bits), whatever q's type
    u32x4_t ph;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * e], c, -run_mc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * e + 1], c, -run_mc));
      run_l += p0 + p1;
      ph[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p0, p1}, f16x2_t));
    }
    // V rows e = 0..7 of the lane: tokens 4 q4 + e (e < 4), 16 + 4 q4 + e - 4
    uint2 vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vr[e] = b.v[e];
      if (masked && t0 + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4) >= tok1) vr[e] = make_uint2(0u, 0u);
    }
#pragma unroll
    for (int half = 0; half < NN / 4; ++half) {
      u32x4_t va[4];  // columns NN m16 + 4 half + n, n < 4
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = half ? vr[2 * i].y : vr[2 * i].x;
        const uint32_t bb = half ? vr[2 * i + 1].y : vr[2 * i + 1].x;
        const uint32_t ev = pair_even(a, bb), od = pair_odd(a, bb);
        va[0][i] = e4m3_pair<false>(F16{}, ev);
        va[1][i] = e4m3_pair<false>(F16{}, od);
        va[2][i] = e4m3_pair<true>(F16{}, ev);
        va[3][i] = e4m3_pair<true>(F16{}, od);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) o[4 * half + n] = mfma(F16{}, va[n], ph, o[4 * half + n]);
    }
  };
  auto step = [&](const Fp8Rows<D>& b, int st) {
    if (st == nsteps - 1) compute(b, st, std::true_type{});
    else compute(b, st, std::false_type{});
  };

  // The scheduling barriers keep every buffer's loads in the same order in
  // the prologue and the loop, so the waits before a buffer is used count
  // only its own loads (loads issued in another order on one path would make
  // the compiler drain everything at the loop head).
  Fp8Rows<D> bufA, bufB;
  load(bufA, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(bufB, 1);
  __builtin_amdgcn_sched_barrier(0);
  for (int st = 0; st < nsteps; st += 2) {
    step(bufA, st);
    __builtin_amdgcn_sched_barrier(0);
    load(bufA, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nsteps) step(bufB, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    load(bufB, st + 3);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Lane (m16, q4) holds head m16's columns NN (4 q4 + i) + nn in o[nn][i]:
  // NN consecutive values per i.
  const float l = fp8_sum_xor32(fp8_sum_xor16(run_l));
  const int nparts_seq = (ctx + p.part_tokens - 1) / p.part_tokens;
  const bool whole = nparts_seq == 1;  // the same for the whole wave
  // A record's values are stored as f16 under a power-of-two scale
  // (record_scale_exp) from the largest magnitude of the head's row, which
  // its 4 lanes m16 + 16 q4 hold; every lane still takes part here.
  int k = 0;
  if (!whole) {
    float amax = 0.f;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[nn][i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    k = record_scale_exp(amax * p.v_scale);
  }
  if (m16 >= G) return;
  const int64_t row = head0 + m16;
  const float f = whole ? p.v_scale / l : p.v_scale * __builtin_ldexpf(1.f, k);
  const int64_t orow = whole ? row : row * p.num_parts + part;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d0 = orow * D + NN * (4 * q4 + i);
    float y[NN];
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) y[nn] = o[nn][i] * f;
    if (whole && p.out_f32) {
      float* of = reinterpret_cast<float*>(p.out) + d0;
#pragma unroll
      for (int kk = 0; kk < NN; kk += 4) *reinterpret_cast<float4*>(of + kk) = make_float4(y[kk], y[kk + 1], y[kk + 2], y[kk + 3]);
    } else {
      // 16-bit output rows (q's type), or an f16 record row
      uint32_t w[NN / 2];
#pragma unroll
      for (int kk = 0; kk < NN / 2; ++kk) {
        if (whole) w[kk] = uint32_t(narrow(T{}, y[2 * kk])) | (uint32_t(narrow(T{}, y[2 * kk + 1])) << 16);
        else w[kk] = uint32_t(narrow(F16{}, y[2 * kk])) | (uint32_t(narrow(F16{}, y[2 * kk + 1])) << 16);
      }
      uint16_t* oh = reinterpret_cast<uint16_t*>(whole ? p.out : p.part_o) + d0;
      if constexpr (NN == 8) *reinterpret_cast<uint4*>(oh) = make_uint4(w[0], w[1], w[2], w[3]);
      else *reinterpret_cast<uint2*>(oh) = make_uint2(w[0], w[1]);
    }
  }
  if (whole) return;
  if (q4 == 0) *reinterpret_cast<float4*>(p.part_ml + orow * 4) = make_float4(run_mc, l, __builtin_ldexpf(1.f, -k), 0.f);
}

template <class T, int D, int G>
void launch_group(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(unsigned(grid_units(p)));
  if (p.block_size == 8) hipLaunchKernelGGL((decode_fp8_kernel<T, D, G, true>), grid, dim3(kWave), 0, st, p);
  else hipLaunchKernelGGL((decode_fp8_kernel<T, D, G, false>), grid, dim3(kWave), 0, st, p);
}

template <class T, int D>
void launch_g(const DecodeParams& p, int G, hipStream_t st) {
  switch (G) {
    case 1: launch_group<T, D, 1>(p, st); break;
    case 2: launch_group<T, D, 2>(p, st); break;
    case 4: launch_group<T, D, 4>(p, st); break;
    default: launch_group<T, D, 8>(p, st); break;
  }
}

}  // namespace

pa_status launch_decode_fp8_partitions(const DecodeParams& p, pa_dtype q_dtype, int D, int G, hipStream_t st) {
  if (q_dtype == PA_F16) {
    if (D == 64) launch_g<F16, 64>(p, G, st);
    else launch_g<F16, 128>(p, G, st);
  } else {
    if (D == 64) launch_g<BF16, 64>(p, G, st);
    else launch_g<BF16, 128>(p, G, st);
  }
  return launch_status("decode E4M3 partition kernel");
}

}  // namespace pkv
