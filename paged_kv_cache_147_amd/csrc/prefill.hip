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
//     tokens); each wave owns 32 (token, query head) rows -- 32/G tokens
//     times the G query heads of the KV head -- as two 16-row MFMA tiles
//     that share every K and V operand read from LDS;
//   * the workgroup walks the keys its rows can see in steps of 32.  Each
//     step's K and V rows are gathered through the block table straight into
//     LDS by global_load_lds_dwordx4 (16 bytes per lane, no registers on the
//     way), into a ring of 4 stages used two steps at a time: while a pair
//     of steps is computed the next pair's loads are in flight, and the
//     waves meet once per pair; the block ids come from scalar loads, which
//     keeps the vector-memory counter for the ring alone;
//   * rows sit in LDS unpadded, their 16-byte chunks permuted by an XOR of
//     the row index, so the K reads and the transposing V reads below spread
//     over the banks;
//   * scores are S^T = K Q^T (v_mfma_f32_16x16x32, A = 16 K rows from LDS,
//     B = the wave's queries, held in registers), so each lane ends up with
//     4 keys x 2 tiles of one row and the softmax is lane-local: the running
//     max moves only when a score exceeds it by more than 2^8 (until then the
//     probabilities are exponentials against the stale max, at most 2^8, and
//     the final division by the sum, taken against the same max, cancels
//     it); the row sums of the probabilities come from the matrix cores,
//     one more block of the p.V product with V^T replaced by ones, so they
//     sum exactly the rounded probabilities that went into O;
//   * the same 8 probabilities per lane are, unchanged, the B operand of
//     O^T += V^T P^T -- with the contraction's 32 keys ordered so that lane
//     group q holds keys 4q..4q+3 and 16+4q..16+4q+3 -- and V^T comes from
//     the LDS tile through ds_read_b64_tr_b16, the gfx950 transposing load
//     (each 16-lane group reads 4 rows x 16 columns and every lane receives
//     one column of 4);
//   * P enters p.V rounded once to f16 (11 significant bits; one bf16
//     rounding, 8 bits, would leave a relative L2 error near 1e-3), one MFMA
//     per block.  A bf16 cache's V rows are turned into f16 in LDS once per
//     step by the whole workgroup (exact inside the f16 range).  A V value
//     beyond that range becomes inf and leaves a non-finite O; a workgroup
//     that ends so runs again on bf16 V rows with P split into a bf16 high
//     part and the bf16 rounding of the rest (~16 bits), two MFMAs per block;
//   * workgroups are issued longest first (the last chunk blocks see the
//     most keys), so the short ones fill the tail.
#include "device_common.h"

#include <cmath>
#include <type_traits>

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kKeys = 32;                  // keys per step: two 16-key MFMA tiles
constexpr int kSub = 2;                    // 16-row MFMA tiles per wave
constexpr int kRows = 16 * kSub;           // (token, query head) rows per wave
constexpr int kStages = 4;                 // LDS ring depth, in steps
constexpr int kXcds = 8;                   // workgroups are dealt to the XCDs round robin
constexpr int kRankMax = 256;              // units per XCD ranked by context length (else taken in order)
constexpr float kSlack = 8.f;              // log2 headroom before the running max moves

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* const_i32_p;   // read through the scalar cache

__device__ __forceinline__ f32x4_t mfma(BF16, u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma(F16, u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                 0, 0, 0);
}

// Two probabilities -> a packed bf16 high part (round to nearest even) and
// the packed bf16 rounding of what the high part leaves out.
__device__ __forceinline__ void split(BF16, float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){ra, rb}, bf16x2_t));
}

// Max with the lane 16 or 32 positions away: after a permlane swap of x with
// itself the two results hold x of the lane and of its partner.
__device__ __forceinline__ float max_xor16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// Chunk permutation of a staged row: a row of CPR 16-byte chunks keeps chunk
// c at position c ^ swizzle(row).  Rows 0..7 get 8 different values (the 8
// rows one K read serves at a time use 8 different bank groups) and rows
// 4k..4k+3 differ above bit 0 (the 4 rows of one transposing read, 32 bytes
// each, land on different chunk pairs).  Adding 16 to the row leaves it alone.
template <int CPR>
__device__ __forceinline__ int swizzle(int row) {
  return ((row & (CPR / 2 - 1)) << 1) | ((row / (CPR / 2)) & 1);
}

// Wait until this wave has at most N vector-memory operations outstanding
// (the LDS ring's loads are the only ones in the loop), then meet the other
// waves: after it, every wave's loads of the awaited step are in LDS and
// every wave is done reading the stage the next loads overwrite.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_and_meet() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

// A wave-uniform 64-bit address in scalar registers.  readfirstlane returns
// a signed int: each half is taken back through uint32_t, so the low half is
// zero-extended, never sign-extended into the high half.
__device__ __forceinline__ uint64_t sgpr64(const char* p) {
  const uint64_t b = uint64_t(uintptr_t(p));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b >> 32))));
  return (uint64_t(hi) << 32) | uint64_t(lo);
}

// The two ring loads of one piece: 16 bytes per lane from kb + off into LDS
// at lds + 16 * lane, and from vb + off into LDS at lds + VOFF + 16 * lane
// (kb, vb and lds, an LDS byte address, the same for the whole wave; off per
// lane), by global_load_lds_dwordx4 with scalar bases, whose LDS address is
// M0 (saved once and restored here).  They are issued from asm so that the
// compiler, which cannot tell which stage a load targets, adds no waits of
// its own for them in front of the LDS reads: the ring's waits are explicit.
// Hazards: each base is copied by a scalar move inside the asm, so no load
// reads a scalar register that a vector instruction (a readfirstlane) wrote
// just before, and that move is also the one wait state a load-to-LDS needs
// after the scalar write of M0.
template <uint32_t VOFF>
__device__ __forceinline__ void ring_load_kv(const char* kb, const char* vb, uint32_t off, uint32_t lds) {
  const uint32_t l = uint32_t(__builtin_amdgcn_readfirstlane(int(lds)));
  const uint64_t ks = sgpr64(kb), vs = sgpr64(vb);
  uint32_t saved;
  uint64_t kc, vc;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %6\n\t"
               "s_mov_b64 %1, %4\n\t"
               "global_load_lds_dwordx4 %3, %1\n\t"
               "s_add_u32 m0, %6, %7\n\t"
               "s_mov_b64 %2, %5\n\t"
               "global_load_lds_dwordx4 %3, %2\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved), "=&s"(kc), "=&s"(vc) : "v"(off), "s"(ks), "s"(vs), "s"(l), "n"(VOFF) : "memory");
}

// float32 pair -> packed 16-bit pair, round to nearest even.
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

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
  int32_t row_blocks;    // chunk blocks per (sequence, KV head)
  int32_t out_f32;
  float scale_log2e;     // scale * log2(e): scores in the log2 domain
};

// A ring stage known at compile time, so that LDS addresses of a stage fold
// into the instructions' offsets.
template <int S>
using Stage = std::integral_constant<int, S>;

template <class T, int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int KK = D / 32;              // score MFMA steps over head_dim
  constexpr int NN = D / 16;              // 16-column blocks of the output
  constexpr int CPR = D / 8;              // 16-byte chunks per K or V row
  constexpr int ROW = D * 2;              // bytes per staged row
  constexpr int TILE = kKeys * ROW;       // bytes of one step's K (or V) rows
  constexpr int NDMA = TILE / (kThreads * 16);   // 16-byte pieces per thread per tile
  constexpr int TPW = kRows / G;          // chunk tokens per wave
  constexpr int TPB = TPW * kWaves;       // chunk tokens per workgroup
  static_assert(TILE % (kThreads * 16) == 0, "a step's tile must split into whole wave loads");
  static_assert(kStages == 4, "steps go in pairs: two stages computed while two fill");

  // bf16 caches: each step's V rows are turned into f16 in LDS once per
  // workgroup, so that p.V takes P rounded once to f16 (one MFMA per block).
  // A workgroup whose V holds a value beyond the f16 range runs again on
  // bf16 V rows with P split into two bf16 parts.
  constexpr bool kConvV = std::is_same<T, BF16>::value;

  __shared__ __align__(16) char lds[kStages][2][TILE];   // [stage][K, V][32 rows]
  __shared__ int vflag;                                  // some O not finite after the f16 pass

  const int tid = threadIdx.x;

  // Workgroup id -> (unit = (sequence, KV head), block of chunk tokens).
  // Workgroup ids go to the XCDs round robin; XCD x takes the units
  // u = x + 8 m.  It runs them one after another in order of decreasing
  // context, and all chunk blocks of a unit in a row, the last (which see
  // the most keys) first, so that a unit's K and V rows are fetched into
  // that XCD's L2 once while its blocks run side by side, and the longest
  // units do not start last.
  const int units = p.num_seqs * p.num_kv_heads;
  const int xcd = blockIdx.x % kXcds;
  const int local = blockIdx.x / kXcds;
  const int nx = (units - xcd + kXcds - 1) / kXcds;       // units of this XCD
  const int rank = local / p.row_blocks;
  const int rb = p.row_blocks - 1 - local % p.row_blocks;
  if (rank >= nx) return;                 // grid padding (the whole workgroup)
  int m = rank;                           // unit xcd + 8 m has this rank
  if (nx > 1 && nx <= kRankMax) {
    // rank of each unit: how many of the XCD's units have a longer context
    // (ties: the lower index first); scratch in the last ring stage, which
    // the first loads below leave alone
    int* len = reinterpret_cast<int*>(lds[kStages - 1][1]);
    int* pick = len + kRankMax;
    if (tid < nx) len[tid] = p.ctx_lens[(xcd + kXcds * tid) / p.num_kv_heads];
    __syncthreads();
    if (tid < nx) {
      const int mine = len[tid];
      int r = 0;
      for (int t = 0; t < nx; ++t) {
        const int o = len[t];
        r += o > mine || (o == mine && t < tid);
      }
      if (r == rank) *pick = tid;
    }
    __syncthreads();
    m = *pick;
  }
  const int unit = xcd + kXcds * m;
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

  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int m16 = lane & 15;              // MFMA column: this lane's row within a tile
  const int q4 = lane >> 4;               // MFMA k-group
  const int tokw = tok0 + wave * TPW;     // first chunk token of this wave
  const int head = g * G + m16 % G;       // the same in both tiles (16 is a multiple of G)

  int tok[kSub];
  bool row_ok[kSub];
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    tok[j] = tokw + (16 * j + m16) / G;
    row_ok[j] = tok[j] < n && r0 + tok[j] >= 0 && r0 + tok[j] < p.num_rows;
  }

  if (ctx <= 0) {                         // no context: zero rows (whole workgroup)
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if (!row_ok[j]) continue;
      const int64_t orow = (int64_t(r0 + tok[j]) * p.num_q_heads + head) * D;
      for (int d = q4; d < D; d += 4) {
        if (p.out_f32) reinterpret_cast<float*>(p.out)[orow + d] = 0.f;
        else reinterpret_cast<uint16_t*>(p.out)[orow + d] = 0;
      }
    }
    return;
  }
  const int base = ctx - n;               // position of chunk row 0
  // Visible keys: row at chunk token t sees positions 0..base + t.  Padding
  // rows (past the chunk) see the whole context; nothing of them is written.
  int pos[kSub];
#pragma unroll
  for (int j = 0; j < kSub; ++j) pos[j] = tok[j] < n ? max(base + tok[j], 0) : ctx - 1;
  const int wave_first = tokw < n ? max(base + tokw, 0) : ctx - 1;          // fewest keys in the wave
  const int wave_last = tokw < n ? max(base + min(tokw + TPW, n) - 1, 0) : -1;  // most keys; -1: no rows
  const int kmax = max(base + min(tok0 + TPB, n) - 1, 0);   // last key any row here sees (<= ctx - 1)
  const int nsteps = kmax / kKeys + 1;

  // Ring loads.  One wave-wide load moves 1 KB, RPI whole rows: load c of
  // wave w fills tile rows [(c kWaves + w) RPI, +RPI), which lie in one cache
  // block (RPI divides B), so its block id is one scalar load.  Lane l of it
  // fills LDS slot 16 l of those rows: row lrow[c] of its block (within the
  // tile), chunk position l % CPR, which holds chunk (l % CPR) ^ swizzle(row).
  constexpr int RPI = kWave * 16 / ROW;   // rows per wave-wide load: 4 or 8
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int bmask = (1 << p.log2_block) - 1;
  int lrow[NDMA];
  uint32_t lbyte[NDMA];
#pragma unroll
  for (int c = 0; c < NDMA; ++c) {
    const int row = (c * kWaves + wv) * RPI + lane / CPR;
    lrow[c] = row & bmask;
    lbyte[c] = ((lane % CPR) ^ swizzle<CPR>(row)) * 16;
  }
  const const_i32_p table = (const_i32_p)(p.tables + int64_t(s) * p.max_blocks);
  const int last_blk = (ctx - 1) >> p.log2_block;
  const int last_row = (ctx - 1) & bmask;
  const int64_t head_off = int64_t(g) * p.tile_bytes;
  const char* const kbase = p.k + head_off;
  const char* const vbase = p.v + head_off;
  const uint32_t blk_stride = uint32_t(p.num_kv_heads) * uint32_t(p.tile_bytes);   // < 2^32 (checked on the host)
  const uint32_t lds0 = uint32_t(size_t((__attribute__((address_space(3))) const char*)&lds[0][0][0]));
  // The block ids of a step are fetched (scalar loads) a pair of steps
  // before its loads are issued, so their latency hides behind the math.
  // ids[step % 2] holds them.
  int ids[2][NDMA];
  auto block_index = [&](int step, int c) {
    // a step spans whole blocks (B divides 32); keys past the context
    // re-read rows of the last block (their scores are masked)
    return min(((step * kKeys) >> p.log2_block) + (((c * kWaves + wv) * RPI) >> p.log2_block), last_blk);
  };
  auto fetch = [&](int step, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;   // step % kStages
#pragma unroll
    for (int c = 0; c < NDMA; ++c) ids[stage & 1][c] = table[uint32_t(block_index(step, c))];
  };
  auto issue = [&](int step, auto stage_c) {   // ids hold this step's block ids
    constexpr int stage = decltype(stage_c)::value;   // step % kStages
#pragma unroll
    for (int c = 0; c < NDMA; ++c) {
      const int bidx = block_index(step, c);
      const int blk = min(max(ids[stage & 1][c], 0), p.num_blocks - 1);
      const int cap = bidx == last_blk ? last_row : bmask;
      const uint32_t off = uint32_t(min(lrow[c], cap) * ROW) + lbyte[c];
      const uint64_t at = uint64_t(uint32_t(blk)) * blk_stride;
      const uint32_t dst = lds0 + uint32_t(stage * 2 * TILE) + uint32_t((c * kWaves + wv) * kWave * 16);
      ring_load_kv<TILE>(kbase + at, vbase + at, off, dst);
    }
  };

  // Step 0's ring loads go first; the query loads follow, and one wait the
  // compiler sees covers both, so that no wait for the queries is left for
  // it to place inside the loop (where it would drain the ring).
  fetch(0, Stage<0>{});
  issue(0, Stage<0>{});
  // Queries: the B operand of S^T = K Q^T.  Lane (q4, m16) of tile j holds
  // elements [32 kk + 8 q4, +8) of row 16 j + m16 for step kk.
  u32x4_t qb[kSub][KK];
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    const int qr = row_ok[j] ? r0 + tok[j] : 0;   // padding rows read row 0; never written
    const char* qrow = reinterpret_cast<const char*>(p.q) + (int64_t(qr) * p.num_q_heads + head) * ROW + q4 * 16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qb[j][kk] = *reinterpret_cast<const u32x4_t*>(qrow + kk * 64);
  }

  __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0); expcnt and lgkmcnt left alone
  // Scores are kept raw (q . k) and scaled inside the exponent, which needs
  // a positive factor: a negative scale is moved into the queries by flipping
  // their sign bits (exact), and a zero one is raised to 1e-30 (every
  // exponent then still rounds to 0).
  if (p.scale_log2e < 0.f) {
#pragma unroll
    for (int j = 0; j < kSub; ++j)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qb[j][kk] ^= 0x80008000u;
  }
  if (1 < nsteps) {
    fetch(1, Stage<1>{});
    issue(1, Stage<1>{});
  }
  if (2 < nsteps) fetch(2, Stage<2>{});
  if (3 < nsteps) fetch(3, Stage<3>{});

  // LDS read offsets.  K (A operand of S^T): lane (q4, m16) reads key row
  // m16 (+16 for the second tile), chunk 4 kk + q4.  V^T (transposing reads):
  // lane m16 of group q4 points at row 4 q4 + m16 / 4 (+16 for keys 16..31),
  // columns 16 nn + 4 (m16 % 4) .. +3, i.e. chunk 2 nn + (m16 % 4) / 2, and
  // receives column 16 nn + m16 of the 4 rows its group addressed.
  int koff[KK], voff[NN];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = m16 * ROW + ((4 * kk + q4) ^ swizzle<CPR>(m16)) * 16;
  {
    const int vr = 4 * q4 + (m16 >> 2);
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
      voff[nn] = vr * ROW + ((2 * nn + ((m16 & 3) >> 1)) ^ swizzle<CPR>(vr)) * 16 + 8 * (m16 & 1);
  }

  const float c = fmaxf(fabsf(p.scale_log2e), 1e-30f);
  const float slack = kSlack / c;         // kSlack in raw score units
  float run_m[kSub], run_mc[kSub];        // running max (raw), and times c
  float run_top[kSub];                    // run_m + slack: a score above it moves the max
  // Running sums of the probabilities, from the matrix cores: one more block
  // of the p.V product with an all-ones V^T, so every element of run_l[j]
  // is row m16's sum of the very (rounded) P that went into O.
  f32x4_t run_l[kSub];
  f32x4_t o[kSub][NN];                    // O^T: lane holds columns 16 nn + 4 q4 + i of row m16
  auto clear_state = [&]() {
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      run_m[j] = run_mc[j] = run_top[j] = -INFINITY;
      run_l[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) o[j][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  clear_state();

  auto compute = [&](int step, auto stage_c, auto masked_step, auto split_step, const u32x4_t& one) {
    constexpr int stage = decltype(stage_c)::value;         // step % kStages
    constexpr bool masked = decltype(masked_step)::value;   // some row of the wave stops inside this step
    constexpr bool psplit = decltype(split_step)::value;    // bf16 V rows: P as two bf16 parts
    const int t0 = step * kKeys;
    const char* kt = lds[stage][0];
    const char* vt = lds[stage][1];
    // S^T tiles: element i of acc[j][h] is key t0 + 16 h + 4 q4 + i of row 16 j + m16.
    f32x4_t acc[kSub][2];
#pragma unroll
    for (int j = 0; j < kSub; ++j) acc[j][0] = acc[j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(kt + koff[kk]);
      const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(kt + koff[kk] + 16 * ROW);
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        acc[j][0] = mfma(T{}, k0, qb[j][kk], acc[j][0]);
        acc[j][1] = mfma(T{}, k1, qb[j][kk], acc[j][1]);
      }
    }
    u32x4_t PH[kSub], PL[kSub];
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      float x[8], mx = -INFINITY;
      const int lim = pos[j] - t0 - 4 * q4;   // element e is visible when 16 (e / 4) + e % 4 <= lim
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = acc[j][e >> 2][e & 3];
        if (masked && 16 * (e >> 2) + (e & 3) > lim) x[e] = -INFINITY;
        mx = fmaxf(mx, x[e]);
      }
      // The max moves only when some score of the wave's rows exceeds it by
      // more than kSlack in log2 units (always in the first step, where it
      // is -inf).
      if (__builtin_amdgcn_ballot_w64(mx > run_top[j])) {
        const float mnew = fmaxf(run_m[j], max_xor32(max_xor16(mx)));
        const float f = __builtin_amdgcn_exp2f((run_m[j] - mnew) * c);
        run_m[j] = mnew;
        run_mc[j] = mnew * c;
        run_top[j] = mnew + slack;
        run_l[j] *= f;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) o[j][nn] *= f;
      }
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -run_mc[j]));
      }
      // P^T operand: contraction index 8 q4 + e is key 4 q4 + e (e < 4) or
      // 16 + 4 q4 + e - 4 (e >= 4), i.e. exactly pr[e].
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (psplit) {
          uint32_t hi, lo;
          split(BF16{}, pr[2 * e], pr[2 * e + 1], hi, lo);
          PH[j][e] = hi;
          PL[j][e] = lo;
        } else {
          PH[j][e] = pack2(F16{}, pr[2 * e], pr[2 * e + 1]);
        }
      }
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vt + voff[nn]));
      const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vt + voff[nn] + 16 * ROW));
      const uint2 w0 = __builtin_bit_cast(uint2, a0), w1 = __builtin_bit_cast(uint2, a1);
      const u32x4_t va = {w0.x, w0.y, w1.x, w1.y};
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        if constexpr (psplit) {
          o[j][nn] = mfma(BF16{}, va, PH[j], o[j][nn]);
          o[j][nn] = mfma(BF16{}, va, PL[j], o[j][nn]);
        } else {
          o[j][nn] = mfma(F16{}, va, PH[j], o[j][nn]);
        }
      }
    }
    // the row sums: V^T replaced by ones
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if constexpr (psplit) {
        run_l[j] = mfma(BF16{}, one, PH[j], run_l[j]);
        run_l[j] = mfma(BF16{}, one, PL[j], run_l[j]);
      } else {
        run_l[j] = mfma(F16{}, one, PH[j], run_l[j]);
      }
    }
  };

  // Ring: step st lives in stage st % kStages, and steps go in pairs.  Before
  // computing steps st and st + 1 the wave waits for all its loads (those of
  // the pair) and meets the others; the two stages it then refills, with
  // steps st + 2 and st + 3, held the previous pair, which every wave has
  // finished.  The next pair's loads are in flight while this pair is
  // computed, and there is one barrier per two steps.
  // bf16 -> f16 of the pair's V rows in place, exact for every bf16 value
  // inside the f16 range; a value beyond it becomes inf.  Each thread turns
  // the very 16-byte pieces that its own ring loads wrote (a piece holds 8
  // elements of one row wherever the swizzle put it), so it needs only its
  // own wait for them, before the pair's barrier, and the barrier then
  // publishes the converted rows too.
  auto convert_v = [&](int st, auto stage_c) {
    constexpr int s0 = decltype(stage_c)::value;      // st % kStages
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (st + h >= nsteps) break;
      char* vt = lds[s0 + h][1];
#pragma unroll
      for (int cch = 0; cch < TILE / (kThreads * 16); ++cch) {
        u32x4_t* w = reinterpret_cast<u32x4_t*>(vt + (cch * kThreads + tid) * 16);
        const u32x4_t x = *w;
        u32x4_t y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = pack2(F16{}, __uint_as_float(x[e] << 16), __uint_as_float(x[e] & 0xffff0000u));
        *w = y;
      }
    }
  };

  // All steps of the workgroup, pair by pair; for a bf16 cache in the first
  // mode the V rows of each pair are turned into f16 first.  The loop runs
  // two pairs per turn, so that every stage index is a compile-time constant
  // and LDS addresses take it as an instruction offset.  A pair's block ids
  // for the pair after next are fetched once its steps are issued: a scalar
  // load in flight would otherwise hold up the steps' first LDS reads (both
  // count on the same wait counter).
  auto ring_loop = [&](auto split_mode) {
    constexpr bool psplit = decltype(split_mode)::value;
    // the all-ones V^T of the row sums (1.0 in the operand's type), held in
    // registers for the whole loop
    u32x4_t one = psplit ? u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                         : u32x4_t{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
    asm volatile("" : "+v"(one));
    auto one_step = [&](int s2, auto stage_c) {
      if (s2 < nsteps && s2 * kKeys <= wave_last) {
        if (s2 * kKeys + kKeys - 1 > wave_first) compute(s2, stage_c, std::true_type{}, split_mode, one);
        else compute(s2, stage_c, std::false_type{}, split_mode, one);
      }
    };
    // steps st and st + 1, held in stages S0 and S0 + 1
    auto pair = [&](int st, auto stage_c) {
      constexpr int S0 = decltype(stage_c)::value;
      constexpr int S2 = (S0 + 2) % kStages;
      if constexpr (kConvV && !psplit) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's pieces of the pair
        convert_v(st, stage_c);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        wait_and_meet<0>();
      }
      if (st + 2 < nsteps) issue(st + 2, Stage<S2>{});
      if (st + 3 < nsteps) issue(st + 3, Stage<S2 + 1>{});
      one_step(st, Stage<S0>{});
      one_step(st + 1, Stage<S0 + 1>{});
      if (st + 4 < nsteps) fetch(st + 4, Stage<S0>{});
      if (st + 5 < nsteps) fetch(st + 5, Stage<S0 + 1>{});
    };
    for (int st = 0; st < nsteps; st += 4) {
      pair(st, Stage<0>{});
      if (st + 2 < nsteps) pair(st + 2, Stage<2>{});
    }
  };

  if constexpr (kConvV) {
    if (tid == 0) vflag = 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ring_loop(std::false_type{});
    // A V value beyond the f16 range became inf, and every V row of a staged
    // step is multiplied by some probability (0 for masked keys, and
    // 0 * inf is NaN), so it leaves a non-finite value in O.  If any wave's
    // O is not finite, the workgroup runs its steps again with bf16 V rows
    // and P split in two bf16 parts (inputs that hold NaN or inf themselves
    // take that path too, and give its result).  The loop ended on a drained
    // ring.
    float osum = 0.f;
#pragma unroll
    for (int j = 0; j < kSub; ++j)
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) osum += (o[j][nn][0] + o[j][nn][1]) + (o[j][nn][2] + o[j][nn][3]);
    if (__builtin_amdgcn_ballot_w64(!__builtin_isfinite(osum))) vflag = 1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (__builtin_amdgcn_readfirstlane(vflag)) {
      clear_state();
      fetch(0, Stage<0>{});
      issue(0, Stage<0>{});
      if (1 < nsteps) {
        fetch(1, Stage<1>{});
        issue(1, Stage<1>{});
      }
      if (2 < nsteps) fetch(2, Stage<2>{});
      if (3 < nsteps) fetch(3, Stage<3>{});
      ring_loop(std::true_type{});
    }
  } else {
    ring_loop(std::false_type{});
  }

  // the loop's last wait drained the ring; rows of the wave now end
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    const float l = run_l[j][0];
    if (!row_ok[j]) continue;
    const float inv = 1.f / l;
    const int64_t orow = (int64_t(r0 + tok[j]) * p.num_q_heads + head) * D;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d0 = 16 * nn + 4 * q4;
      const float x0 = o[j][nn][0] * inv, x1 = o[j][nn][1] * inv, x2 = o[j][nn][2] * inv, x3 = o[j][nn][3] * inv;
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow + d0) = make_float4(x0, x1, x2, x3);
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + orow + d0) =
            make_uint2(pack2(T{}, x0, x1), pack2(T{}, x2, x3));
      }
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
  if (a->q_dtype != a->kv_dtype) return fail(PA_E_INVAL, "q_dtype must equal kv_dtype");
  if (a->num_q_heads % a->num_kv_heads) return fail(PA_E_INVAL, "num_q_heads must be a multiple of num_kv_heads");
  const int G = a->num_q_heads / a->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(PA_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (a->block_size != 8 && a->block_size != 16 && a->block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size must be 8, 16 or 32");
  if (a->max_blocks <= 0 || a->num_blocks <= 0) return fail(PA_E_INVAL, "max_blocks and num_blocks must be positive");
  if (a->max_chunk < 0) return fail(PA_E_INVAL, "max_chunk must be >= 0");
  if (int64_t(a->num_kv_heads) * a->block_size * a->head_dim * 2 > int64_t(UINT32_MAX))
    return fail(PA_E_UNSUPPORTED, "a cache block must stay under 4 GiB");
  if (!std::isfinite(a->scale)) return fail(PA_E_INVAL, "scale must be finite");
  const int64_t rbs = (int64_t(a->max_chunk) + tokens_per_workgroup(G) - 1) / tokens_per_workgroup(G);
  const int64_t units = int64_t(a->num_seqs) * a->num_kv_heads;
  if (rbs * kXcds * ((units + kXcds - 1) / kXcds) > INT32_MAX) return fail(PA_E_UNSUPPORTED, "grid too large");
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
  pp.row_blocks = int(rbs);
  const int64_t units = int64_t(a->num_seqs) * a->num_kv_heads;
  const dim3 grid(unsigned(rbs * kXcds * ((units + kXcds - 1) / kXcds)));
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
