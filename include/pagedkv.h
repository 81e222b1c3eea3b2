/*
 * pagedkv.h -- C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * What the library does.  A sequence's KV cache lives in fixed-size physical
 * blocks of B tokens; a per-sequence block table maps logical block i // B to
 * a physical block id ("Paged Attention" (daiw.org), 直觉 and 定义).  The host
 * block pool hands blocks out and takes them back, shares them between
 * sequences by reference count and copies a still-shared last block before a
 * sequence writes into it ("vllm-pagedattention" (chenyuan1125.github.io),
 * 页表真正解开的… and 一块内存，如何安全地属于多条序列).  Three device
 * operations serve one decode step: pa_copy_blocks (those copies),
 * pa_write_kv (the new token's K/V into its slot) and pa_decode
 * (single-query attention whose K/V rows are found through the tables).
 * pa_decode_contiguous computes the same attention on the contiguous
 * one-region-per-sequence layout the pages compare paging against.
 *
 * Conventions shared by every call
 * - Status: every call returns a pa_status; PA_OK is 0, errors are negative.
 *   No C++ exception and no abort crosses this boundary.  pa_last_error()
 *   gives a human-readable detail of the calling thread's last failure.
 * - Device memory: every device pointer is owned by the caller (for instance
 *   a torch tensor's data_ptr()).  The library never allocates, frees or
 *   synchronises device memory; device calls only enqueue work on the given
 *   stream (a hipStream_t passed as pa_stream; NULL = the null stream) and
 *   return once it is enqueued.
 * - Host memory: the pool owns its host state until pa_pool_destroy.  Output
 *   arrays are caller-owned and written only on PA_OK unless a call says
 *   otherwise.
 * - Shapes are checked on the host before anything is enqueued: a bad
 *   argument gives PA_E_INVAL, a shape or dtype outside the supported set
 *   gives PA_E_UNSUPPORTED; neither launches anything.
 * - Threading: a pool is not thread-safe (callers serialise calls on one
 *   pool); device calls are reentrant.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_E_INVAL (-1)        /* bad argument (null pointer, negative size, ...) */
#define PA_E_NOBLOCKS (-2)     /* pool exhausted: the request is refused, nothing changed */
#define PA_E_NOSEQ (-3)        /* unknown sequence id */
#define PA_E_EXISTS (-4)       /* sequence id already in use */
#define PA_E_UNSUPPORTED (-5)  /* shape / dtype outside the compiled set */
#define PA_E_HIP (-6)          /* the HIP runtime refused a launch */

typedef int32_t pa_dtype;
#define PA_F32 0
#define PA_F16 1
#define PA_BF16 2
/* One-byte E4M3 codes of a quantised KV cache (OCP 8-bit float, "FN": 1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7F / 0xFF NaN,
 * no infinities, largest finite 448), each cache with one float32 scale:
 * element = value(code) * scale.  Cache dtype only: written by
 * pa_write_kv_fp8, read by pa_decode, moved by the bit-copy calls. */
#define PA_FP8_E4M3 3

typedef void* pa_stream; /* a hipStream_t */

/* Static text for a status code ("unknown status" for other values). */
const char* pa_strerror(pa_status status);
/* Detail of the calling thread's last failing call ("" if none). */
const char* pa_last_error(void);
/* Library ABI version, currently 1. */
int32_t pa_version(void);

/* ------------------------------------------------------------------------- */
/* Host block pool                                                            */
/* ------------------------------------------------------------------------- */
/*
 * Rules ("vLLM PagedAttention：大模型推理的显存管理革命" (horeb.top), 分配策略
 * and 内存共享：写时复制; "vllm-paged-attention-engine" (aiqz.cc), 分页存储设计
 * and the allocator of Python 演示; "vllm-pagedattention", 一块内存…):
 * - a sequence of n tokens holds ceil(n / B) blocks;
 * - free blocks are taken from the front of the free list and released blocks
 *   are appended at its back, in table order;
 * - a token goes into the last block while it has room; a full last block
 *   makes the pool append one more block to the table;
 * - fork shares every block of the parent (reference count + 1 each);
 * - writing into a last block whose count is > 1 first copies it: the
 *   sequence's last entry is remapped to a fresh block (taken from the front)
 *   and the caller must copy src -> dst on the device (pa_copy_blocks)
 *   before writing the token; full blocks are never copied;
 * - a block returns to the free list when its count reaches 0;
 * - a request the pool cannot cover is refused with PA_E_NOBLOCKS and leaves
 *   the pool unchanged ("Paged Attention", 读者问答 / 运维提示: an exhausted
 *   pool rejects requests rather than failing).
 * The slot of logical token i of a sequence is table[i / B] * B + i % B; it
 * indexes the device caches' [num_blocks * B] token rows (see pa_write_kv).
 */
typedef struct pa_pool pa_pool;

typedef struct pa_pool_stats_t {
  int32_t num_blocks;
  int32_t block_size;
  int32_t free_blocks;    /* blocks on the free list */
  int32_t used_blocks;    /* blocks with reference count >= 1 */
  int32_t shared_blocks;  /* blocks with reference count >= 2 */
  int32_t num_seqs;
  int64_t tokens;         /* sum of sequence lengths */
  int64_t waste_tokens;   /* sum over sequences of empty slots in their tables
                             (each < B; "Paged Attention", 定义: waste is
                             confined to the last block) */
} pa_pool_stats_t;

/* Create a pool of num_blocks blocks of block_size tokens (both > 0 and
 * num_blocks < 2^31 / block_size).  initial_free_order: NULL for 0..n-1, else
 * a permutation of 0..n-1 (PA_E_INVAL otherwise), copied. */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* initial_free_order, pa_pool** out);
void pa_pool_destroy(pa_pool* pool); /* NULL is a no-op */

/* Admit seq with n_tokens >= 0 prompt tokens, taking ceil(n/B) blocks at
 * once.  slots_out (nullable) receives the n_tokens slots.  PA_E_EXISTS if seq
 * is live, PA_E_NOBLOCKS if the pool is short (nothing taken). */
pa_status pa_seq_alloc(pa_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out);

/* Grow seq by one token and return its slot.  If the token lands in a
 * still-shared last block, *cow_src / *cow_dst receive the block pair the
 * caller must copy on the device first; otherwise both are -1.  Output
 * pointers are nullable. */
pa_status pa_seq_append(pa_pool* pool, int64_t seq, int64_t* slot_out,
                        int32_t* cow_src, int32_t* cow_dst);

/* n >= 0 successive pa_seq_append calls as one all-or-nothing request:
 * slots_out (nullable, n entries); at most the first token can need a copy,
 * reported as in pa_seq_append. */
pa_status pa_seq_extend(pa_pool* pool, int64_t seq, int32_t n, int64_t* slots_out,
                        int32_t* cow_src, int32_t* cow_dst);

/* child shares all of parent's blocks and its length.  PA_E_NOSEQ if parent
 * is unknown, PA_E_EXISTS if child is live (including child == parent). */
pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t child);

/* Release seq: reference counts drop in table order; blocks reaching 0 go to
 * the back of the free list. */
pa_status pa_seq_free(pa_pool* pool, int64_t seq);

pa_status pa_seq_len(const pa_pool* pool, int64_t seq, int32_t* len_out);

/* Block tables of n sequences as an n x max_blocks int32 row-major array,
 * padded with -1, and their lengths (ctx_out, nullable).  PA_E_NOSEQ for an
 * unknown id, PA_E_INVAL when a table is wider than max_blocks; on error the
 * output arrays hold unspecified values. */
pa_status pa_pool_block_tables(const pa_pool* pool, const int64_t* seqs, int32_t n,
                               int32_t max_blocks, int32_t* tables_out, int32_t* ctx_out);

/* Swap-out / swap-in for preemption: a request's blocks are moved to host
 * memory and back later ("vllm-paged-attention-engine" (aiqz.cc),
 * 连续批处理：随到随走的新秩序: under memory pressure a request's whole set of
 * blocks is copied back to CPU memory and copied in again when there is
 * room).
 * pa_seq_swap_out writes seq's table (block ids, logical order) to
 * blocks_out (cap entries; *n_out = their number), releases the blocks as
 * pa_seq_free would, and marks seq swapped out.  The caller copies those
 * blocks to host memory (pa_swap_out) on the stream before any later device
 * write can reach them.  pa_seq_swap_in takes ceil(len / B) fresh blocks
 * from the front of the free list (all-or-nothing, PA_E_NOBLOCKS), returns
 * them in logical order and makes seq resident again; the caller copies the
 * contents back (pa_swap_in).  Blocks shared with other sequences before the
 * swap come back as private copies.  A swapped-out sequence keeps its id and
 * length; growth, fork and pa_pool_block_tables refuse it (PA_E_INVAL),
 * pa_seq_free drops it.  pa_pool_stats counts resident sequences only. */
pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq, int32_t* blocks_out, int32_t cap, int32_t* n_out);
pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq, int32_t* blocks_out, int32_t cap, int32_t* n_out);

pa_status pa_pool_stats(const pa_pool* pool, pa_pool_stats_t* out);
/* Reference count of a block, or -1 for an id outside [0, num_blocks). */
int32_t pa_pool_refcount(const pa_pool* pool, int32_t block);
/* Free list front to back into out[0 .. min(cap, free)-1]; *n_out = free count. */
pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/*
 * Prefix cache (automatic prefix caching on top of the pool: a full block is
 * identified by its parent block, its token ids and extra keys such as a
 * cache salt, so a request whose prompt starts with a cached prefix reuses
 * those blocks and skips their prefill -- "vllm-pagedattention"
 * (chenyuan1125.github.io), the passage on automatic prefix caching after
 * 一块内存，如何安全地属于多条序列; the salt keeps tenants' prefixes apart, same
 * page, closing remarks).  Rules:
 * - the key of a full block is (its parent block's id, salt, its B token
 *   ids); lookups walk a prompt's full blocks from the first and stop at the
 *   first miss, so a hit is always a whole-block prefix;
 * - a block is registered when it becomes full -- at admission for the
 *   prompt's full blocks, or when pa_seq_append_token fills it -- provided
 *   its parent is registered (or it is a first block) and no block holds its
 *   key yet;
 * - a registered block whose reference count drops to 0 stays cached on the
 *   free list; allocation still takes from the front, and a cached block
 *   taken there is evicted (least recently released first); a hit takes a
 *   free cached block back off the list;
 * - with the cache on, pa_seq_free releases a sequence's blocks last to
 *   first (descendants are evicted before their ancestors);
 * - pa_seq_alloc, pa_seq_append and pa_seq_extend still work; they leave the
 *   sequence's later blocks unregistered (their token ids are not known).
 * The caller writes the K/V of the uncached tokens (slots from cached_tokens
 * on) before any other request can hit the blocks it registered.
 */
typedef struct pa_prefix_stats_t {
  int64_t lookups;       /* block keys looked up by pa_seq_alloc_prefix */
  int64_t hit_blocks;    /* of them found and reused */
  int64_t registered;    /* blocks registered */
  int64_t evictions;     /* cached blocks taken off the free list for new contents */
  int32_t cached_blocks; /* blocks registered now */
} pa_prefix_stats_t;

/* Switch the prefix cache on; only before the first sequence is admitted
 * (PA_E_INVAL otherwise). */
pa_status pa_pool_enable_prefix_cache(pa_pool* pool);

/* Admit seq with its n_tokens >= 0 prompt token ids (host array) under salt.
 * The longest cached whole-block prefix is reused; the rest takes fresh
 * blocks.  *cached_tokens_out (nullable) = tokens whose K/V is already in
 * the cache (a multiple of B, possibly n_tokens); slots_out (nullable)
 * receives all n_tokens slots.  All-or-nothing: PA_E_NOBLOCKS when the free
 * list (cached blocks included, the hits excepted) is short; PA_E_EXISTS,
 * and PA_E_INVAL when the cache is off. */
pa_status pa_seq_alloc_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens, int32_t n_tokens,
                              uint64_t salt, int32_t* cached_tokens_out, int64_t* slots_out);

/* pa_seq_append for a token whose id is known: as pa_seq_append, and when the
 * token fills the last block, that block is registered (rules above). */
pa_status pa_seq_append_token(pa_pool* pool, int64_t seq, int32_t token, int64_t* slot_out,
                              int32_t* cow_src, int32_t* cow_dst);

pa_status pa_prefix_cache_stats(const pa_pool* pool, pa_prefix_stats_t* out);
/* 1 if the block is registered in the prefix cache, 0 if not, -1 for an id
 * outside [0, num_blocks). */
int32_t pa_pool_block_cached(const pa_pool* pool, int32_t block);

/* ------------------------------------------------------------------------- */
/* Device operations                                                          */
/* ------------------------------------------------------------------------- */
/*
 * Cache layout (both K and V): [num_blocks][num_kv_heads][block_size][head_dim],
 * dense, row-major, elements of the cache dtype.  One (block, kv head) tile
 * of block_size * head_dim elements is contiguous, so a block is contiguous
 * inside and blocks sit anywhere ("Paged Attention", 定义).
 * Supported set: head_dim in {64, 128}; block_size in {8, 16, 32};
 * dtype in {PA_F32, PA_F16, PA_BF16}, and PA_FP8_E4M3 for the bit copies
 * (pa_write_kv of codes, pa_copy_blocks, pa_swap_*), pa_write_kv_fp8 and
 * pa_decode.
 */

/* Scatter num_tokens new tokens into their slots ("vllm-pagedattention",
 * 页表真正解开的…: a new token is written into the last block while it has
 * room).  k_new, v_new: [num_tokens][num_kv_heads][head_dim] device arrays;
 * slot_mapping: num_tokens int64 device array; token t goes to block
 * slot / B, row slot % B.  A negative slot is padding and is skipped; a slot
 * >= num_blocks * B is skipped as well (never written out of bounds).  Bit
 * copy: no arithmetic on the values.  Slots must be distinct (duplicates
 * race). */
pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      pa_dtype dtype, pa_stream stream);

/* Quantising scatter into an E4M3 cache (PA_FP8_E4M3 layout above).  Same
 * slots and skipping rules as pa_write_kv; k_new, v_new hold src_dtype
 * values (PA_F32, PA_F16 or PA_BF16).  Each element x is stored as the E4M3
 * code nearest to y = x * r, r = 1 / k_scale (v_scale for V) rounded to
 * float32 once and the product rounded to float32: ties go to the even code,
 * |y| >= 448 saturates to +-448, NaN gives 0x7F.  Scales must be finite and
 * positive (PA_E_INVAL otherwise).  Quantised caches are one lever on the
 * cache's byte floor besides fewer KV heads and shorter contexts
 * ("Paged Attention" (daiw.org), 量化, the boxed warning); serving systems
 * ship FP8 caches ("vLLM PagedAttention：大模型推理的显存管理革命", 生态现状).
 * The pages fix no format; E4M3 with a per-cache scale is this library's
 * choice. */
pa_status pa_write_kv_fp8(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          pa_dtype src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          float k_scale, float v_scale, pa_stream stream);

/* Copy-on-write block copies ("vllm-pagedattention", 一块内存…: the shared last
 * block is copied before the branch writes).  pairs: n_pairs x 2 int32 device
 * array of (src, dst); each copies the whole block, every KV head, in K and in
 * V.  Pairs whose ids fall outside [0, num_blocks) are skipped.  Pairs run
 * concurrently: no block may be both a source and a destination in one call. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, pa_dtype dtype, pa_stream stream);

/* Swap copies for preemption (see pa_seq_swap_out / pa_seq_swap_in):
 * pa_swap_out copies blocks[0..n) (device int32 ids, the table pa_seq_swap_out
 * returned) -- every KV head, K and V -- into host, laid out
 * [n][K, V][num_kv_heads][block_size][head_dim]; pa_swap_in copies such a
 * buffer back into blocks[0..n) (the table pa_seq_swap_in returned).  host
 * must be pinned host memory (hipHostMalloc, e.g. a torch pin_memory
 * tensor; PA_E_INVAL otherwise) of at least 2 * n * block bytes; the kernel
 * reads or writes it directly over the host link.  Ids outside
 * [0, num_blocks) are skipped (their host rows are not touched).  Bit copy.
 * The caller keeps host alive and unchanged until the copy has run
 * (stream-ordered). */
pa_status pa_swap_out(const void* k_cache, const void* v_cache, const int32_t* blocks, int32_t n, void* host,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      pa_dtype dtype, pa_stream stream);
pa_status pa_swap_in(void* k_cache, void* v_cache, const int32_t* blocks, int32_t n, const void* host,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     pa_dtype dtype, pa_stream stream);

/*
 * Decode attention, one query token per sequence.  For sequence s and query
 * head h (KV head g = h / (Hq / Hkv), consecutive grouping):
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) * V_t,  t in [0, ctx_lens[s]),
 * with token t's rows in block block_tables[s][t / B], row t % B
 * ("Paged Attention", 直觉; "vllm-pagedattention", 页表真正解开的…: the kernel
 * fetches each block through the table and does scores, softmax and the
 * weighted sum of V; the attention itself is unchanged).  The new token must
 * have been written already (it attends to itself).
 *
 * Contexts are cut into fixed partitions of partition_size tokens, one wave
 * each, as on the pages (vLLM's partitioned kernel), reduced independently
 * and merged with the log-sum-exp identity (which needs the workspace); a
 * sequence's result depends only on its own inputs.  partition_size 0 picks
 * the length automatically (512, 256 or 128 tokens: the largest giving
 * >= 2048 sequence x KV head x partition units).
 * Arithmetic is float32 (16-bit inputs are widened exactly); results do not
 * depend on which physical blocks hold the tokens, and are bitwise
 * reproducible for the same inputs on the same GPU with the same
 * partition_size (the contiguous entry point cuts identically, so it agrees
 * bit for bit when both use the same score path).
 */
typedef struct pa_decode_args {
  void* out;                   /* [S][Hq][head_dim], out_dtype */
  pa_dtype out_dtype;          /* PA_F32 or kv_dtype */
  const void* q;               /* [S][Hq][head_dim], q_dtype */
  const void* k_cache;         /* layout above, kv_dtype */
  const void* v_cache;
  pa_dtype kv_dtype;
  const int32_t* block_tables; /* [S][max_blocks] device; entries j < ceil(ctx/B) are read */
  const int32_t* ctx_lens;     /* [S] device */
  int32_t num_seqs;            /* S >= 0 (0: nothing to do) */
  int32_t num_q_heads;         /* Hq, a multiple of Hkv with Hq / Hkv in {1, 2, 4, 8} */
  int32_t num_kv_heads;        /* Hkv > 0 */
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks;          /* table row width > 0 */
  int32_t num_blocks;          /* physical blocks in the caches */
  int32_t max_ctx;             /* 0 or an upper bound on ctx_lens; sizes the grid
                                  (0 means max_blocks * block_size) */
  float scale;                 /* finite, e.g. 1/sqrt(head_dim) */
  int32_t partition_size;      /* 0 = automatic, else partitions of that many
                                  tokens: a multiple of 8 and of block_size, at
                                  most min(512, 64 * block_size) (PA_E_INVAL
                                  otherwise, negative values included) */
  void* workspace;             /* device scratch, >= pa_decode_workspace_bytes,
                                  256-byte aligned */
  size_t workspace_bytes;
  pa_dtype q_dtype;            /* q's element type.  f32 / f16 / bf16 caches: must equal
                                  kv_dtype (PA_E_INVAL otherwise: the kernels read q at the
                                  cache's element size).  E4M3 caches: PA_F16 or PA_BF16,
                                  and out_dtype is PA_F32 or q_dtype. */
  /* E4M3 caches (kv_dtype PA_FP8_E4M3) only; ignored otherwise: */
  float k_scale;               /* finite, > 0: K element = value(code) * k_scale */
  float v_scale;               /* finite, > 0 */
} pa_decode_args;
/*
 * E4M3 caches: codes are widened exactly to q_dtype, q.K and p.V run on the matrix cores
 * with float32 accumulation (p as a 16-bit value plus the 16-bit rounding of
 * its remainder), k_scale is folded into the score scale and v_scale into
 * the weighted sums.
 */
/*
 * Device-side data: a ctx_lens entry <= 0 yields a zero output row; entries
 * above max_ctx are clamped to it (the caller guarantees they do not occur);
 * table entries are clamped into [0, num_blocks) so that a corrupt table can
 * never read outside the caches (its sequence's output is then meaningless).
 */

/* Workspace bytes pa_decode needs for these arguments.  Validates the
 * arguments like pa_decode; needs no GPU.
 *
 * One record per (sequence, query head, partition) of the longest context,
 * or 0 bytes when every context fits one partition: the partition's max, sum
 * of weights and a scale a (4 floats), and its head_dim weighted sums divided
 * by a.  The sums are float32 for float32 caches; for 16-bit and E4M3 caches
 * they are f16 under a power-of-two a chosen per record so that the record's
 * largest magnitude lands in [2^14, 2^15) (relative rounding at most 2^-11 per
 * value; the half-size records halve the lines the partition kernel writes,
 * which measured 3.5% faster on the Llama-3.1-8B batch without sharing).  A
 * short launch after the decode kernel merges the records.  The contents need
 * no initialisation and are rewritten by each call, so one workspace serves
 * any number of calls ordered on one stream; two calls running at the same
 * time must not share one. */
pa_status pa_decode_workspace_bytes(const pa_decode_args* args, size_t* bytes_out);
pa_status pa_decode(const pa_decode_args* args, pa_stream stream);

/*
 * pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split-context records go to a static device array inside the library
 * instead of a caller workspace; args->workspace and workspace_bytes are
 * ignored.  The call allocates nothing.
 *
 * Limit: pa_decode_static_max_bytes() bytes (64 MiB).  A batch whose
 * pa_decode_workspace_bytes exceeds it is refused with PA_E_UNSUPPORTED
 * before anything is launched.  Each GPU the library runs on holds one such
 * array until the process ends.
 *
 * Sharing: every call on one GPU uses that GPU's array, which keeps the last
 * call's contents.  The contents need no initialisation, since each call
 * rewrites all it reads.  Calls ordered on one stream are safe.  Two calls
 * that may run at the same time on one GPU (different streams, no ordering
 * between them) race on the array and give undefined results.  Otherwise the
 * same as pa_decode: same checks, same kernels, bit-identical output.
 */
size_t pa_decode_static_max_bytes(void);
pa_status pa_decode_static(const pa_decode_args* args, pa_stream stream);

/*
 * Chunked prefill attention.  Sequence s holds ctx_lens[s] cached tokens, the
 * last n_s = q_start[s+1] - q_start[s] of which are the chunk being
 * prefilled: their K/V rows have been written (pa_write_kv) before the call.
 * Chunk row i of s sits at position ctx_lens[s] - n_s + i and attends
 * causally over tokens 0..position, gathered through the block table:
 *     out[row][h] = sum_{t <= pos} softmax_t(scale * q[row][h] . K_t) * V_t
 * ("vLLM PagedAttention：大模型推理的显存管理革命", 分配策略: prefill admits a
 * prompt at once; "vllm-pagedattention", 它和 FlashAttention 优化的是两张不同的账:
 * prefill works on large query blocks; "Paged Attention" (daiw.org), 回顾与衔接:
 * a tiled kernel must read K/V through the block table).  Scores and p.V run
 * on the matrix cores with float32 accumulation; the probabilities enter p.V
 * rounded once to f16, against V rows in f16 (a bf16 cache's rows are
 * converted exactly in on-chip memory).  A workgroup whose bf16 V rows hold a
 * value beyond the f16 range recomputes its rows with bf16 V and each
 * probability as a bf16 value plus the bf16 rounding of its remainder.
 * PA_E_UNSUPPORTED also when one cache block (Hkv * B * head_dim * 2 bytes)
 * reaches 4 GiB.
 */
typedef struct pa_prefill_args {
  void* out;                   /* [T][Hq][head_dim], out_dtype */
  pa_dtype out_dtype;          /* PA_F32 or kv_dtype */
  const void* q;               /* [T][Hq][head_dim], kv_dtype: the chunks' rows, grouped by sequence */
  const void* k_cache;         /* [num_blocks][Hkv][B][head_dim] */
  const void* v_cache;
  pa_dtype kv_dtype;           /* PA_F16 or PA_BF16 */
  const int32_t* block_tables; /* [S][max_blocks] device */
  const int32_t* ctx_lens;     /* [S] device: cached tokens, chunk included; <= 0 gives zero rows */
  const int32_t* q_start;      /* [S + 1] device: rows of s are q_start[s] .. q_start[s+1]-1,
                                  non-decreasing, q_start[S] = T, and each chunk no longer
                                  than its context */
  int32_t num_seqs;            /* S >= 0 */
  int32_t num_rows;            /* T >= 0 */
  int32_t num_q_heads;         /* Hq, a multiple of Hkv with Hq / Hkv in {1, 2, 4, 8} */
  int32_t num_kv_heads;
  int32_t head_dim;            /* 64 or 128 */
  int32_t block_size;          /* 8, 16 or 32 */
  int32_t max_blocks;          /* table row width > 0 */
  int32_t num_blocks;          /* physical blocks in the caches */
  int32_t max_chunk;           /* >= every n_s; sizes the grid */
  float scale;
  pa_dtype q_dtype;            /* q's element type: must equal kv_dtype (PA_E_INVAL otherwise) */
} pa_prefill_args;
pa_status pa_prefill(const pa_prefill_args* args, pa_stream stream);

/*
 * Debug check of pa_decode's device inputs.  The decode kernels clamp table
 * entries into the pool rather than check them (a corrupt table gives a
 * meaningless row, never an out-of-bounds read); this counts what a correct
 * caller never passes: ctx_lens entries above the context bound (max_ctx, or
 * max_blocks * block_size), and table entries j < ceil(ctx / block_size)
 * outside [0, num_blocks).  The count goes to *count (device int32),
 * asynchronously on stream.  Arguments are validated as for pa_decode
 * (out, q and the caches are not read).
 *
 * With the environment variable PAGEDKV_DEBUG set (and not "0"), pa_decode
 * runs this check first, synchronises the stream, and returns PA_E_INVAL
 * without launching the decode when the count is not zero.
 */
pa_status pa_decode_validate(const pa_decode_args* args, int32_t* count, pa_stream stream);

/*
 * The same attention on the contiguous layout the pages contrast paging with
 * ("Paged Attention", 定义: one region per sequence reserved for its maximum
 * length): K and V are [S][Hkv][capacity][head_dim]; no block table.  Used to
 * measure what the table indirection costs.
 */
typedef struct pa_contig_args {
  void* out;
  pa_dtype out_dtype;
  const void* q;
  const void* k;               /* [S][Hkv][capacity][head_dim] */
  const void* v;
  pa_dtype kv_dtype;
  const int32_t* ctx_lens;     /* [S] device, each <= capacity */
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t capacity;            /* token rows reserved per (sequence, KV head) */
  int32_t max_ctx;             /* 0 or an upper bound on ctx_lens (0 = capacity) */
  float scale;
  int32_t partition_size;      /* as in pa_decode_args; fixed partitions a
                                  multiple of 8, at most 512 */
  void* workspace;
  size_t workspace_bytes;
  pa_dtype q_dtype;            /* q's element type: must equal kv_dtype (PA_E_INVAL otherwise) */
} pa_contig_args;

pa_status pa_decode_contiguous_workspace_bytes(const pa_contig_args* args, size_t* bytes_out);
pa_status pa_decode_contiguous(const pa_contig_args* args, pa_stream stream);


#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
