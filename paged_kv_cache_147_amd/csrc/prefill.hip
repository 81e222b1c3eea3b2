// Chunked prefill attention over a paged KV cache, for gfx950 (CDNA4).
//
// What is computed: sequence s holds ctx[s] cached tokens, the last n_s of
// which are the chunk being prefilled (its K/V rows were written first, as
// any growth).  Chunk row i sits at position p = ctx[s] - n_s + i and attends
// causally over tokens 0..p, found through the block table as in decode:
//   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_t) V_t.
// The pages: prefill admits a prompt's tokens at once ("vLLM PagedAttention：
// 大模型推理的显存管理革命", 分配策略) and works on large blocks of queries
// ("vllm-pagedattention", 它和 FlashAttention 优化的是两张不同的账); a
// tiled kernel must read K/V through the block table to get both the paged
// layout and the tiled data flow ("Paged Attention" (daiw.org), 回顾与衔接).
//
// Work decomposition (a dense contraction, so the matrix cores do it):
//   * one workgroup of 4 waves per (KV head, sequence, block of chunk
//     tokens); each wave owns 16 (token, query head) rows -- 16/G tokens
//     times the G query heads of the KV head;
//   * the workgroup walks the keys its rows can see in steps of 32, staging
//     each step's K and V rows (gathered through the block table) in LDS,
//     double-buffered so the next step's loads fly during this one's math;
//   * scores are S^T = K Q^T (v_mfma_f32_16x16x32, A = 16 K rows from LDS,
//     B = the wave's queries, held in registers), so each lane ends up with
//     4 keys x 2 tiles of one row: the online softmax (running max, sum and
//     rescale) is lane-local plus two cross-lane steps;
//   * the same 8 probabilities per lane are, unchanged, the B operand of
//     O^T += V^T P^T -- with the contraction's 32 keys ordered so that lane
//     group q holds keys 4q..4q+3 and 16+4q..16+4q+3 -- and V^T comes from
//     the LDS tile through ds_read_b64_tr_b16, the gfx950 transposing load
//     (each 16-lane group reads 4 rows x 16 columns and every lane receives
//     one column of 4);
//   * P is split into a 16-bit high part and the 16-bit rounding of the
//     remainder, two MFMAs per block, so p.V keeps ~16 more bits than a
//     16-bit P would (a single rounded P alone exceeds the 1e-3 tolerance).
#include "device_common.h"

#include <cmath>

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kKeys = 32;                  // keys per step: two 16-key MFMA tiles
constexpr int kRows = 16;                  // (token, query head) rows per wave

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // staged chunk: a plain vector, kept in registers

__device__ __forceinline__ f32x4_t mfma(BF16, uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma(F16, uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                 0, 0, 0);
}

// LDS rows of staged K/V hold D elements plus 16 of padding: consecutive rows
// then start 8 banks apart, so the 16 rows a transposing read touches spread
// over the banks.
template <int D>
constexpr int lds_stride() { return D + 16; }

struct PrefillParams {
  void* out;
  const void* q;
  const char* k;
  const char* v;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* q_start;
  int64_t tile_bytes;    // bytes of one (block, KV head) tile: B * D * 2
  int32_t num_seqs;
  int32_t num_rows;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t log2_block;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t out_f32;
  float scale_log2e;     // scale * log2(e): scores in the log2 domain
};

template <class T, int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int RS = lds_stride<D>();
  constexpr int KK = D / 32;              // score MFMA steps over head_dim
  constexpr int NN = D / 16;              // 16-column blocks of the output
  constexpr int TPW = kRows / G;          // chunk tokens per wave
  constexpr int TPB = TPW * kWaves;       // chunk tokens per workgroup
  constexpr int CPR = D / 8;              // 16-byte chunks per K or V row
  constexpr int CPT = kKeys * CPR;        // chunks per 32-key tile
  constexpr int NLD = 2 * CPT / kThreads; // K + V chunks each thread stages per step
  static_assert(2 * CPT % kThreads == 0, "staging must divide evenly");

  __shared__ __align__(16) uint16_t kbuf[2][kKeys * RS];
  __shared__ __align__(16) uint16_t vbuf[2][kKeys * RS];

  // Workgroup id -> (block of chunk tokens, sequence, KV head).  KV heads of
  // one sequence and then sequences vary fastest, so with S * Hkv a multiple
  // of 8 every (sequence, KV head) keeps its workgroups on one XCD.
  const int units = p.num_seqs * p.num_kv_heads;
  const int rb = blockIdx.x / units;
  const int unit = blockIdx.x % units;
  const int s = unit / p.num_kv_heads;
  const int g = unit % p.num_kv_heads;
  const int r0 = p.q_start[s];
  const int n = p.q_start[s + 1] - r0;
  const int tok0 = rb * TPB;
  if (tok0 >= n) return;                  // the whole workgroup: no barrier is left waiting
  // Contexts are clamped to the table's capacity, and rows outside
  // [0, num_rows) are padding, so bad lengths or offsets never reach outside
  // the tables, q or out (their results are then meaningless).
  const int ctx = min(p.ctx_lens[s], p.max_blocks << p.log2_block);

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int m16 = lane & 15;              // MFMA column: this lane's (token, head) row
  const int q4 = lane >> 4;               // MFMA k-group
  const int tok = tok0 + wave * TPW + m16 / G;
  const bool row_ok = tok < n && r0 + tok >= 0 && r0 + tok < p.num_rows;
  const int head = g * G + m16 % G;

  if (ctx <= 0) {                         // no context: zero rows (whole workgroup)
    if (row_ok) {
      const int64_t orow = (int64_t(r0 + tok) * p.num_q_heads + head) * D;
      for (int d = q4; d < D; d += 4) {
        if (p.out_f32) reinterpret_cast<float*>(p.out)[orow + d] = 0.f;
        else reinterpret_cast<uint16_t*>(p.out)[orow + d] = 0;
      }
    }
    return;
  }
  const int base = ctx - n;               // position of chunk row 0
  const int pos = row_ok ? max(base + tok, 0) : 0;
  const int last_tok = min(tok0 + TPB, n) - 1;
  const int kmax = max(base + last_tok, 0);   // last key any row here sees (<= ctx - 1)
  const int nsteps = kmax / kKeys + 1;

  // Queries: the B operand of S^T = K Q^T.  Lane (q4, m16) holds elements
  // [32 kk + 8 q4, +8) of row m16 for step kk.
  uint4 qb[KK];
  {
    const int qr = row_ok ? r0 + tok : 0;  // padding rows read row 0; never written
    const char* qrow = reinterpret_cast<const char*>(p.q) + (int64_t(qr) * p.num_q_heads + head) * D * 2 + q4 * 16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb[kk] = *reinterpret_cast<const uint4*>(qrow + kk * 64);
  }

  // Staging: thread tid moves chunks tid + kThreads * c of the step's K tile
  // (chunk index < CPT) and V tile, each chunk 16 bytes of one key row.
  // Keys past the context re-read the last token (their scores are masked).
  const int32_t* table = p.tables + int64_t(s) * p.max_blocks;
  u32x4_t ld[NLD];
  auto stage_load = [&](int t0) {
#pragma unroll
    for (int c = 0; c < NLD; ++c) {
      const int idx = tid + kThreads * c;
      const bool is_v = idx >= CPT;
      const int cc = is_v ? idx - CPT : idx;
      const int key = min(t0 + cc / CPR, ctx - 1);
      const int blk = min(max(table[key >> p.log2_block], 0), p.num_blocks - 1);
      const char* src = (is_v ? p.v : p.k) + (int64_t(blk) * p.num_kv_heads + g) * p.tile_bytes +
                        int64_t(key & ((1 << p.log2_block) - 1)) * D * 2 + (cc % CPR) * 16;
      ld[c] = *reinterpret_cast<const u32x4_t*>(src);
    }
  };
  auto stage_store = [&](int b) {
#pragma unroll
    for (int c = 0; c < NLD; ++c) {
      const int idx = tid + kThreads * c;
      const bool is_v = idx >= CPT;
      const int cc = is_v ? idx - CPT : idx;
      uint16_t* dst = (is_v ? vbuf[b] : kbuf[b]) + (cc / CPR) * RS + (cc % CPR) * 8;
      *reinterpret_cast<u32x4_t*>(dst) = ld[c];
    }
  };

  float run_m = -INFINITY, run_l = 0.f;   // this lane's row (m16)
  f32x4_t o[NN];                          // O^T: lane holds columns 16 nn + 4 q4 + i of row m16
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int b, int t0) {
    // S^T tiles: element i of tile j is key t0 + 16 j + 4 q4 + i of row m16.
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = kbuf[b] + (16 * j + m16) * RS + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = mfma(T{}, *reinterpret_cast<const uint4*>(krow + 32 * kk), qb[kk], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * j + 4 * q4 + i;
        const float x = t > pos ? -INFINITY : acc[i] * p.scale_log2e;   // causal mask (and t >= ctx)
        sc[4 * j + i] = x;
        mx = fmaxf(mx, x);
      }
    }
    // The row's 32 scores sit in lanes m16, m16 + 16, m16 + 32, m16 + 48.
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(run_m, mx);        // finite: key 0 is in every row's first step
    const float f = __builtin_amdgcn_exp2f(run_m - mnew);
    float pr[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(sc[e] - mnew);
      psum += pr[e];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    run_l = run_l * f + psum;
    run_m = mnew;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) o[nn] *= f;

    // P^T operands: contraction index 8 q4 + e is key 4 q4 + e (e < 4) or
    // 16 + 4 q4 + e - 4 (e >= 4), i.e. exactly pr[e]; high and low parts.
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h0 = narrow(T{}, pr[2 * e]), h1 = narrow(T{}, pr[2 * e + 1]);
      const uint16_t l0 = narrow(T{}, pr[2 * e] - widen1(T{}, h0));
      const uint16_t l1 = narrow(T{}, pr[2 * e + 1] - widen1(T{}, h1));
      ph[e] = uint32_t(h0) | (uint32_t(h1) << 16);
      pl[e] = uint32_t(l0) | (uint32_t(l1) << 16);
    }
    const uint4 PH = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const uint4 PL = make_uint4(pl[0], pl[1], pl[2], pl[3]);

    // V^T operands by transposing reads: lane m16 of group q4 points at row
    // 4 q4 + m16 / 4 (then 16 + that), columns 16 nn + 4 (m16 % 4) .. +3, and
    // receives column 16 nn + m16 of the 4 rows its group addressed.
    const uint16_t* vlo = vbuf[b] + (4 * q4 + (m16 >> 2)) * RS + 4 * (m16 & 3);
    const uint16_t* vhi = vlo + 16 * RS;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vlo + 16 * nn));
      const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vhi + 16 * nn));
      const uint2 w0 = __builtin_bit_cast(uint2, a0), w1 = __builtin_bit_cast(uint2, a1);
      const uint4 A = make_uint4(w0.x, w0.y, w1.x, w1.y);
      o[nn] = mfma(T{}, A, PH, o[nn]);
      o[nn] = mfma(T{}, A, PL, o[nn]);
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int b = st & 1;
    // The next step's rows fly during this step's math (after the last step
    // this re-reads clamped rows into the idle buffer; nothing uses them).
    stage_load((st + 1) * kKeys);
    compute(b, st * kKeys);
    stage_store(b ^ 1);   // buffer b ^ 1 was last read before the previous barrier
    __syncthreads();
  }

  if (!row_ok) return;
  const float inv = 1.f / run_l;
  const int64_t orow = (int64_t(r0 + tok) * p.num_q_heads + head) * D;
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) {
    const int d0 = 16 * nn + 4 * q4;
    const float x0 = o[nn][0] * inv, x1 = o[nn][1] * inv, x2 = o[nn][2] * inv, x3 = o[nn][3] * inv;
    if (p.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow + d0) = make_float4(x0, x1, x2, x3);
    } else {
      const uint32_t w0 = uint32_t(narrow(T{}, x0)) | (uint32_t(narrow(T{}, x1)) << 16);
      const uint32_t w1 = uint32_t(narrow(T{}, x2)) | (uint32_t(narrow(T{}, x3)) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + orow + d0) = make_uint2(w0, w1);
    }
  }
}

// ---- host side ---------------------------------------------------------------

int log2_of(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

int tokens_per_workgroup(int G) { return kRows / G * kWaves; }

pa_status check_prefill(const pa_prefill_args* a) {
  if (!a) return fail(PA_E_INVAL, "args is null");
  if (a->num_seqs < 0 || a->num_rows < 0) return fail(PA_E_INVAL, "num_seqs and num_rows must be >= 0");
  if (a->num_q_heads <= 0 || a->num_kv_heads <= 0) return fail(PA_E_INVAL, "heads must be positive");
  if (a->kv_dtype != PA_F16 && a->kv_dtype != PA_BF16)
    return fail(PA_E_UNSUPPORTED, "prefill needs a 16-bit (f16 or bf16) cache");
  if (a->out_dtype != PA_F32 && a->out_dtype != a->kv_dtype)
    return fail(PA_E_UNSUPPORTED, "out dtype must be f32 or the cache dtype");
  if (a->num_q_heads % a->num_kv_heads) return fail(PA_E_INVAL, "num_q_heads must be a multiple of num_kv_heads");
  const int G = a->num_q_heads / a->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(PA_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (a->block_size != 8 && a->block_size != 16 && a->block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size must be 8, 16 or 32");
  if (a->max_blocks <= 0 || a->num_blocks <= 0) return fail(PA_E_INVAL, "max_blocks and num_blocks must be positive");
  if (a->max_chunk < 0) return fail(PA_E_INVAL, "max_chunk must be >= 0");
  if (!std::isfinite(a->scale)) return fail(PA_E_INVAL, "scale must be finite");
  const int64_t rbs = (int64_t(a->max_chunk) + tokens_per_workgroup(G) - 1) / tokens_per_workgroup(G);
  if (rbs * a->num_seqs * a->num_kv_heads > INT32_MAX) return fail(PA_E_UNSUPPORTED, "grid too large");
  return ok();
}

template <class T, int D>
void launch_prefill(const PrefillParams& pp, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<T, D, 1>), grid, dim3(kThreads), 0, st, pp); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<T, D, 2>), grid, dim3(kThreads), 0, st, pp); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<T, D, 4>), grid, dim3(kThreads), 0, st, pp); break;
    default: hipLaunchKernelGGL((prefill_kernel<T, D, 8>), grid, dim3(kThreads), 0, st, pp); break;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pa_status pa_prefill(const pa_prefill_args* a, pa_stream stream) {
  pa_status st = check_prefill(a);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0 || a->num_rows == 0 || a->max_chunk == 0) return ok();
  if (!a->out || !a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->ctx_lens || !a->q_start)
    return fail(PA_E_INVAL, "null device pointer");
  const int G = a->num_q_heads / a->num_kv_heads;
  PrefillParams pp{};
  pp.out = a->out;
  pp.q = a->q;
  pp.k = static_cast<const char*>(a->k_cache);
  pp.v = static_cast<const char*>(a->v_cache);
  pp.tables = a->block_tables;
  pp.ctx_lens = a->ctx_lens;
  pp.q_start = a->q_start;
  pp.tile_bytes = int64_t(a->block_size) * a->head_dim * 2;
  pp.num_seqs = a->num_seqs;
  pp.num_rows = a->num_rows;
  pp.num_q_heads = a->num_q_heads;
  pp.num_kv_heads = a->num_kv_heads;
  pp.log2_block = log2_of(a->block_size);
  pp.max_blocks = a->max_blocks;
  pp.num_blocks = a->num_blocks;
  pp.out_f32 = a->out_dtype == PA_F32;
  pp.scale_log2e = a->scale * 1.4426950408889634f;
  const int64_t rbs = (int64_t(a->max_chunk) + tokens_per_workgroup(G) - 1) / tokens_per_workgroup(G);
  const dim3 grid(unsigned(rbs * a->num_seqs * a->num_kv_heads));
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (a->kv_dtype == PA_BF16) {
    if (a->head_dim == 64) launch_prefill<BF16, 64>(pp, G, grid, hs);
    else launch_prefill<BF16, 128>(pp, G, grid, hs);
  } else {
    if (a->head_dim == 64) launch_prefill<F16, 64>(pp, G, grid, hs);
    else launch_prefill<F16, 128>(pp, G, grid, hs);
  }
  return launch_status("prefill kernel");
}
