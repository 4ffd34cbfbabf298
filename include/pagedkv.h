/*
 * pagedkv.h -- C ABI of the MI355X paged-KV decode library (libpagedkv.so).
 *
 * The library has two halves:
 *   1. a host-side block allocator: a pool of fixed-size physical blocks,
 *      per-sequence block tables, prefix sharing with reference counts and
 *      copy-on-write, release and truncate. It owns host metadata only.
 *   2. device operations on caller-owned GPU memory, issued asynchronously
 *      on the caller's HIP stream: the slot-mapped cache write, the
 *      copy-on-write block copy, and paged attention (decode, and causal
 *      multi-query verify).
 *
 * Sources of the method (cited by section, as on the pages):
 *   [vLLM]       PagedAttention / vLLM abstract, papers search page for
 *                "external vector cache": attention over a KV cache kept in
 *                fixed-size blocks like OS pages, with sharing of blocks
 *                within and across requests.
 *   [NeuralOps]  "NeuralOps v1.3.4: Serving Primitives & KV Cache
 *                Optimization", Architectural Breakdown, 1. Paged KV Cache
 *                Engine (16-token physical blocks, block table, growth one
 *                block at a time) and Highlights (slot mapping, block
 *                reclamation when generation ends).
 *   [KVNB s5]    course page "Module 10. KV Caches and Efficient Inference",
 *                notebook "KV cache and serving: bytes, pages, and
 *                ceilings", section 5 "Page pool: prefix sharing and
 *                copy-on-write" (allocation order, preflight, COW, release,
 *                counters, invariants); section 2 (causal visibility: query
 *                j of a suffix sees prefix + j + 1 keys); section 9
 *                (negative tests: errors leave the pool unchanged).
 *
 * Conventions for every call:
 *   - Return value: PKV_OK (0) or one of the PKV_E* codes below. On error a
 *     human-readable message is available from paged_kv_last_error() (per
 *     calling thread) and, for allocator calls, the pool is unchanged.
 *   - All arguments are checked before anything is mutated or launched.
 *   - Host pointers are plain host memory; "device" pointers are GPU memory
 *     (for example torch tensors' data pointers). The caller owns all of it.
 *   - A pool handle is not thread-safe: one thread at a time per pool.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls only enqueue work: no host synchronisation, no device
 *     allocation.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,   /* bad size, pointer, dtype, count or unsupported shape */
  PKV_ENOENT = 2,   /* unknown sequence id                                   */
  PKV_EEXIST = 3,   /* sequence id already exists (create, fork target)      */
  PKV_ENOMEM = 4,   /* not enough free blocks; the pool is unchanged         */
  PKV_ECORRUPT = 5, /* paged_kv_validate found a broken invariant            */
  PKV_EHIP = 6      /* a HIP runtime or launch error                         */
};

/* ---- element types of caches and queries ------------------------------ */
/* PKV_I8: int8 codes of a cache holding per-row integer codes (see
 * paged_cache_write_q8); accepted by paged_kv_copy_blocks (codes) and as the
 * byte type of such caches, never as a query type. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_I8 = 2 };

/* Thread-local text describing the last error of this thread's calls. */
const char *paged_kv_last_error(void);

/* ======================================================================
 * Host allocator  ([KVNB s5], [NeuralOps], [vLLM] sharing)
 * ====================================================================== */

typedef struct pkv_pool pkv_pool; /* opaque */

/* A device block copy the caller must perform (paged_kv_copy_blocks) before
 * writing the new tokens: physical block `src` -> `dst`, K and V. */
typedef struct {
  int32_t src;
  int32_t dst;
} pkv_cow_t;

/* The counters of [KVNB s5]. A block's fill is the most tokens any live
 * sequence keeps in it; payload sums fills once per physical block. */
typedef struct {
  int64_t allocated_blocks;         /* blocks with at least one reference  */
  int64_t free_blocks;              /* blocks on the free stack            */
  int64_t physical_capacity_tokens; /* allocated_blocks * block_size       */
  int64_t physical_payload_tokens;  /* sum of fills of allocated blocks    */
  int64_t logical_tokens;           /* sum of sequence lengths             */
  int64_t internal_waste_tokens;    /* capacity - payload                  */
  int64_t sharing_savings_tokens;   /* logical - payload                   */
} pkv_stats_t;

/* Create a pool of `total_blocks` blocks of `block_size` token slots.
 * initial_free_stack: NULL for the order N-1, ..., 0 (block 0 is handed out
 * first), or a permutation of 0..N-1 (host array of N ints) whose LAST entry
 * is handed out first. Requires total_blocks * block_size <= INT32_MAX so
 * every slot fits an int32. *out receives the handle. */
int paged_kv_pool_create(int32_t total_blocks, int32_t block_size,
                         const int32_t *initial_free_stack, pkv_pool **out);
/* Free the pool and every sequence in it (NULL is a no-op); the handle is
 * invalid afterwards. */
void paged_kv_pool_destroy(pkv_pool *pool);

/* Register an empty sequence. EEXIST if the id is taken. */
int paged_kv_seq_create(pkv_pool *pool, int64_t seq_id);

/* Append `n_tokens` logical tokens to a sequence ([KVNB s5] append).
 * Order: preflight the blocks needed (one extra when the last block is
 * partial and shared with another sequence) -> ENOMEM with no change if too
 * few are free; then, if the last block is partial and shared, take a
 * replacement block and report the pair (old, new) in cow_out; fill the last
 * block's free slots; then take new blocks from the free stack.
 * slot_mapping_out: host array of n_tokens ints; token k of this append gets
 *   slot = block * block_size + offset (block id from the sequence's table).
 * cow_out: host array of at least 1 pair; *n_cow_out gets 0 or 1.
 * n_tokens == 0 is a no-op that succeeds. */
int paged_kv_alloc(pkv_pool *pool, int64_t seq_id, int32_t n_tokens,
                   int32_t *slot_mapping_out, pkv_cow_t *cow_out,
                   int32_t *n_cow_out);

/* paged_kv_alloc for n_seqs sequences in order, with the results separate
 * calls would give (an id may repeat; a copy made for one member counts when
 * a later member writes into the same shared block). All or nothing
 * ([KVNB s5]: allocation is preflighted so a failure changes nothing): the
 * whole batch is checked first -- unknown ids (ENOENT), negative counts or a
 * length past INT32_MAX (EINVAL), and the free blocks all members take
 * together (ENOMEM) -- and on any error the pool is unchanged and *n_done
 * is 0. On success slots are written back to back into slot_mapping_out
 * (sum of n_tokens entries), copy pairs back to back into cow_out (capacity
 * n_seqs), *n_cow_out gets their count and *n_done = n_seqs. */
int paged_kv_alloc_batch(pkv_pool *pool, const int64_t *seq_ids,
                         const int32_t *n_tokens, int32_t n_seqs,
                         int32_t *slot_mapping_out, pkv_cow_t *cow_out,
                         int32_t *n_cow_out, int32_t *n_done);

/* Create `child` sharing the first ceil(prefix_tokens / block_size) blocks
 * of `parent` (each gains a reference); child length = prefix_tokens
 * ([KVNB s5] share_prefix). EINVAL if prefix_tokens > parent length,
 * EEXIST if child exists, ENOENT if parent does not. */
int paged_kv_fork(pkv_pool *pool, int64_t parent, int64_t child,
                  int32_t prefix_tokens);

/* Release a sequence: drop one reference per table entry in table order;
 * blocks reaching zero go on top of the free stack ([KVNB s5] release).
 * ENOENT (pool unchanged) if the id is unknown. */
int paged_kv_free(pkv_pool *pool, int64_t seq_id);

/* Shorten a sequence to new_length (0 <= new_length <= length): table
 * entries past ceil(new_length / block_size) are released in table order; a
 * kept partial block that is shared stays shared, so the next append copies
 * it. (Rollback of rejected speculative tokens.) ENOENT if the id is
 * unknown, EINVAL if new_length is outside [0, length]; the pool is then
 * unchanged. */
int paged_kv_truncate(pkv_pool *pool, int64_t seq_id, int32_t new_length);

/* The sequence's length in *len; ENOENT if the id is unknown, EINVAL if len
 * is NULL. */
int paged_kv_seq_length(const pkv_pool *pool, int64_t seq_id, int32_t *len);

/* Number of live sequences in *n_out, and (when ids_out is not NULL) their
 * ids in ascending order in ids_out[capacity]; EINVAL if capacity is too
 * small. */
int paged_kv_seq_ids(const pkv_pool *pool, int64_t *ids_out, int32_t capacity,
                     int32_t *n_out);

/* One sequence's block table (host array of `capacity` ints). */
int paged_kv_page_table(const pkv_pool *pool, int64_t seq_id,
                        int32_t *blocks_out, int32_t capacity, int32_t *n_out);

/* The free stack bottom to top (the top is handed out next). */
int paged_kv_free_stack(const pkv_pool *pool, int32_t *out, int32_t capacity,
                        int32_t *n_out);

/* Row-major block tables for n_seqs sequences into host memory:
 * tables_out[n_seqs * max_blocks], each row padded with -1, and
 * context_lens_out[n_seqs]. EINVAL if a table is longer than max_blocks. */
int paged_kv_block_tables(const pkv_pool *pool, const int64_t *seq_ids,
                          int32_t n_seqs, int32_t max_blocks,
                          int32_t *tables_out, int32_t *context_lens_out);

int paged_kv_stats(const pkv_pool *pool, pkv_stats_t *out);

/* Check the invariants of [KVNB s5] validate: no duplicate or out-of-range
 * id on the free stack; table length = ceil(length / block_size); no block
 * twice in one table; reference count = number of table entries naming the
 * block; referenced <=> not free; 1 <= fill <= block_size for referenced
 * blocks; logical >= payload. ECORRUPT with the broken rule as message. */
int paged_kv_validate(const pkv_pool *pool);

/* ======================================================================
 * Device operations (gfx950)
 *
 * Cache layout ([NeuralOps] blocks; layout chosen here): K and V pools are
 * separate row-major arrays [num_blocks, Hkv, block_size, D] of the cache
 * dtype, so one (block, KV head) is a contiguous block_size * D run.
 * Supported on the device: D in {64, 128, 256}; block_size a multiple of 16
 * for attention (any positive size for the cache write and block copy).
 * ====================================================================== */

/* Slot-mapped cache write ([NeuralOps] slot mapping): for every t < T with
 * s = slot_mapping[t] in [0, num_blocks * block_size):
 *   k_cache[s / bs, h, s % bs, :] = k_new[t, h, :]   (and V), all h < Hkv.
 * Bit-exact copy. Slots < 0 or >= num_blocks * block_size are skipped.
 * k_new, v_new: device [T, Hkv, D]; slot_mapping: device int32 [T].
 * Two tokens must not name the same slot (the allocator never does; see
 * paged_kv_check_slots). */
int paged_cache_write(const void *k_new, const void *v_new, void *k_cache,
                      void *v_cache, const int32_t *slot_mapping, int32_t T,
                      int32_t num_blocks, int32_t Hkv, int32_t D,
                      int32_t block_size, int dtype, void *stream);

/* Check a slot mapping in HOST memory before a cache write: PKV_EINVAL if
 * two of its T tokens name the same slot in [0, num_slots) -- the write's
 * result would then depend on which token lands last -- with the later
 * token's index in *first_dup (NULL allowed; -1 when there is none); PKV_OK
 * otherwise. Slots < 0 or >= num_slots are ignored, as the write skips
 * them. The allocator never emits a repeated slot; this is a debugging aid.
 * A build with PKV_DEBUG_SLOTS defined runs it inside paged_cache_write and
 * its 8-bit and 3-bit variants (copying the mapping to the host and waiting
 * for the stream first) and returns its error instead of launching. */
int paged_kv_check_slots(const int32_t *slots, int32_t T, int64_t num_slots,
                         int32_t *first_dup);

/* Copy-on-write device copy: for each of the n pairs (device array), copy
 * block src -> dst in both pools (all Hkv * block_size * D elements). Pairs
 * with an id outside [0, num_blocks) are skipped. Must run before the cache
 * write of the same step, on the same stream. v_cache may be NULL: then only
 * k_cache is copied (a single-pool array, such as the scales of an 8-bit or
 * 3-bit cache). */
int paged_kv_copy_blocks(void *k_cache, void *v_cache, const pkv_cow_t *pairs,
                         int32_t n, int32_t num_blocks, int32_t Hkv, int32_t D,
                         int32_t block_size, int dtype, void *stream);

/* Workspace bytes paged_attention_decode needs for these sizes and
 * partition_tokens (0 when the chosen launch keeps everything on chip).
 * partition_tokens:
 *    0  the library chooses (one partition per (sequence, KV head) when
 *       those pairs fill the GPU, else as many equal partitions per
 *       context as fill it);
 *   -1  balanced stream: all sequences' tiles are shared equally among the
 *       wavefronts whatever their lengths (for batches of mixed lengths);
 *   >0  split every context into partitions of that many tokens (a multiple
 *       of 16), merged by a log-sum-exp reduce launch.
 * The workspace holds partial results only for the duration of one call;
 * it need not be initialised. */
int paged_attention_workspace_size(int32_t B, int32_t nq, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t max_blocks,
                                   int32_t block_size,
                                   int32_t partition_tokens, size_t *bytes);

/* Paged attention ([vLLM]; causal rule of [KVNB s2]).
 * For sequence b, query i < nq, query head h (KV head g = h / (Hq / Hkv)):
 * the query sees its first n = context_lens[b] - nq + i + 1 tokens, token t
 * being slot t % bs of block block_tables[b * max_blocks + t / bs];
 *   out = softmax(scale * q . K^T) V   over those n tokens,
 *   lse = log(sum exp(scale * q . k))  (natural log; optional).
 * context_lens includes this step's tokens (write them first).
 *   out:          device float32 [B, nq, Hq, D]
 *   q:            device `dtype` [B, nq, Hq, D]
 *   k_cache/v_cache: device `dtype` [num_blocks, Hkv, block_size, D]
 *   block_tables: device int32 [B, max_blocks]; entries past the used ones
 *                 are ignored
 *   context_lens: device int32 [B]
 *   lse_out:      device float32 [B, nq, Hq] or NULL
 *   workspace:    device buffer of paged_attention_workspace_size() bytes
 *                 (may be NULL when that size is 0)
 * Accumulation is float32. Rows that see no token (n <= 0), rows of a
 * sequence with context_lens[b] > max_blocks * block_size, and rows whose
 * visible tokens meet a table entry outside [0, num_blocks) produce NaN in
 * out and lse instead of reading out of bounds.
 * Kernels: bf16 caches with one query token and D <= 128 run on a matrix-
 * core decode kernel (all G rows of a KV head in one wavefront; with
 * partition_tokens = -1 and B <= 4096 in its stream mode, as do the code
 * caches below); fp32 caches and
 * the other single-token cases run on VALU kernels (up to 16 rows per KV
 * head: G * nq rounded up to a power of two, 8 per wavefront); bf16 caches
 * with nq > 1 run on an MFMA tile of 16 query rows
 * per KV head (G * nq <= 16), e.g. 4 query heads x 4 draft tokens for
 * verification. With bf16 caches and G * nq > 16 the call is a chunked
 * prefill (a chunk of nq prompt tokens over the cached prefix plus the chunk
 * itself, whose K/V were written first; the chunk decomposition of
 * [KVNB s7]): an MFMA kernel over 16-row tiles of the chunk's rows, the
 * context cut into partitions (partition_tokens > 0 fixes their length; 0
 * and -1 let the library choose), then the log-sum-exp reduce; a workspace
 * is always needed. fp32 caches take at most 16 rows per KV head.
 * Host-checked: sizes, Hq % Hkv == 0, D and block_size supported, rows per
 * KV head within those limits, scale finite, workspace large enough ->
 * EINVAL. */
int paged_attention_decode(float *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           int32_t max_blocks, const int32_t *context_lens,
                           int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t block_size, int32_t num_blocks,
                           float scale, int dtype, int32_t partition_tokens,
                           void *workspace, size_t workspace_bytes,
                           float *lse_out, void *stream);

/* paged_attention_decode for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same arguments without the workspace, the same kernels and
 * results. Partials that need a workspace go to a device array inside the
 * library of 64 MiB (every graded workload fits: the 131072-token split-K
 * call with 512-token partitions needs 32.5 MiB), one per GPU, held until
 * the process ends; its address on the calling thread's current device is
 * looked up once (hipGetSymbolAddress) and kept. Nothing is allocated and
 * nothing in it needs to start at zero. Every call on one GPU uses the same
 * array, so calls on one GPU that may overlap (other streams, other host
 * threads) race on it: issue them on one stream. EINVAL, before anything is
 * launched, when paged_attention_workspace_size() for these sizes exceeds
 * 64 MiB; other errors as paged_attention_decode. */
int paged_attention_decode_noalloc(float *out, const void *q, const void *k_cache,
                                   const void *v_cache, const int32_t *block_tables,
                                   int32_t max_blocks, const int32_t *context_lens,
                                   int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t block_size, int32_t num_blocks,
                                   float scale, int dtype, int32_t partition_tokens,
                                   float *lse_out, void *stream);

/* ---- caches of 8-bit per-row codes --------------------------------------
 * The teaching quantizer of [KVNB demo] Demo 2 (symmetric integer codes,
 * one scale per row), 8 bits, applied to every (token, KV head) row of K
 * and of V as it is written: scale = max |x| / 127 (1 for a row of zeros),
 * code = clip(round-half-even(x / scale), -127, 127), computed in float64;
 * the scale is stored as float32. Such a cache is three device arrays:
 *   k_codes, v_codes: int8    [num_blocks, Hkv, block_size, D]
 *   scales:           float32 [num_blocks, Hkv, 2, block_size]
 * where scales[b, h, 0, :] are the K rows' scales and scales[b, h, 1, :]
 * the V rows' (D + 4 bytes per token and head instead of 2 D for bf16).
 * K and V scales sit side by side so that one (block, KV head) reads one
 * contiguous 2 * block_size * 4 bytes: a single 128-byte line at
 * block_size 16 when the array is 128-byte aligned (any array from the HIP
 * allocator is). */

/* Quantize and scatter T new rows: k_new, v_new device `dtype` (f32 or
 * bf16) [T, Hkv, D]; slot_mapping as in paged_cache_write (-1 or out of
 * range: skipped). D in {64, 128, 256}. Asynchronous on `stream`.
 * Copy-on-write for such a cache: paged_kv_copy_blocks on the codes
 * (dtype PKV_I8) and on the scales alone (k_cache = scales, v_cache NULL,
 * dtype PKV_F32, Hkv as the cache's, D = 2). */
int paged_cache_write_q8(const void *k_new, const void *v_new, int8_t *k_codes,
                         int8_t *v_codes, float *scales,
                         const int32_t *slot_mapping, int32_t T, int32_t num_blocks,
                         int32_t Hkv, int32_t D, int32_t block_size, int dtype,
                         void *stream);

/* paged_attention_decode over a cache of 8-bit codes: the same attention
 * with each K and V element taken as code * its row's scale ([KVNB demo]
 * Demo 2 reconstruction), dequantized inside the kernel. q is bf16
 * [B, nq, Hq, D]; out, lse, tables, lengths, partition_tokens and workspace
 * as there (paged_attention_workspace_size gives the size; -1 is taken as 0
 * here). Rows per KV head: G * nq rounded up to a power of two <= 16 (one
 * matrix-core wavefront holds them all). The scale array 16-byte aligned.
 * Host-checked as paged_attention_decode -> EINVAL. */
int paged_attention_decode_q8(float *out, const void *q, const int8_t *k_codes,
                              const int8_t *v_codes, const float *scales,
                              const int32_t *block_tables,
                              int32_t max_blocks, const int32_t *context_lens,
                              int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t block_size, int32_t num_blocks,
                              float scale, int32_t partition_tokens,
                              void *workspace, size_t workspace_bytes,
                              float *lse_out, void *stream);

/* ---- caches of 3-bit per-row codes --------------------------------------
 * The same quantizer with 3 bits ([KVNB demo] Demo 2; the 3-bit storage
 * scenario of [KVNB s8]): limit 3, scale = max |x| / 3, code in [-3, 3].
 * Codes are stored two per byte (dim 2 i in the low nibble of byte i), each
 * as its 4-bit float e2m1 bits (sign, 2 exponent bits with bias 1, 1
 * mantissa bit), which hold every code exactly: 0 -> 0x0, 1 -> 0x2,
 * 2 -> 0x4, 3 -> 0x5, and bit 3 set for -1, -2, -3 (0xA, 0xC, 0xD). Half a
 * byte per element, byte-aligned for the decode kernels (the pages' 3 bits
 * per element would not give whole bytes per lane), and a native operand
 * of the gfx950 matrix cores:
 *   k_codes, v_codes: uint8   [num_blocks, Hkv, block_size, D / 2]
 *   scales:           float32 [num_blocks, Hkv, 2, block_size] (as above)
 * D in {128, 256}. paged_cache_write_q3 / paged_attention_decode_q3 are the
 * 8-bit calls' counterparts (same arguments, errors and copy-on-write: codes
 * as PKV_I8 with D / 2 bytes per row). */
int paged_cache_write_q3(const void *k_new, const void *v_new, uint8_t *k_codes,
                         uint8_t *v_codes, float *scales,
                         const int32_t *slot_mapping, int32_t T, int32_t num_blocks,
                         int32_t Hkv, int32_t D, int32_t block_size, int dtype,
                         void *stream);
int paged_attention_decode_q3(float *out, const void *q, const uint8_t *k_codes,
                              const uint8_t *v_codes, const float *scales,
                              const int32_t *block_tables,
                              int32_t max_blocks, const int32_t *context_lens,
                              int32_t B, int32_t nq, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t block_size, int32_t num_blocks,
                              float scale, int32_t partition_tokens,
                              void *workspace, size_t workspace_bytes,
                              float *lse_out, void *stream);

/* ----------------------------------------------------------------------
 * Shared prefixes ([vLLM]: blocks shared within and across requests;
 * [KVNB s5] share_prefix forks a parent's leading blocks).
 * ---------------------------------------------------------------------- */

/* Groups of a batch that share leading physical blocks, from host copies of
 * the block tables [B, max_blocks] and context_lens [B]. Sequences are
 * grouped by their first block id; a group's prefix is the longest run of
 * leading block ids common to all its members, capped so that every query
 * row of every member sees all of it (prefix <= context_lens[b] - nq + 1)
 * and rounded down to a multiple of 16 tokens. Groups with fewer than
 * min_members members (>= 2) or a prefix under min_tokens (>= 16) are
 * dropped. Host outputs, caller-allocated:
 *   seq_prefix[B]       tokens of sequence b in its group's prefix (0: none)
 *   group_start[B + 1]  members of group i are members[group_start[i] ..
 *                       group_start[i + 1])
 *   members[B]          sequence indices, grouped, in ascending order
 *   group_tokens[B]     prefix tokens of group i (first *n_groups entries)
 *   *n_groups, *max_members (largest group), *max_prefix (longest prefix)
 * EINVAL on NULL pointers or bad sizes; nothing is allocated. */
int paged_kv_prefix_groups(const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *context_lens, int32_t B, int32_t nq,
                           int32_t block_size, int32_t min_members,
                           int32_t min_tokens, int32_t *seq_prefix,
                           int32_t *group_start, int32_t *members,
                           int32_t *group_tokens, int32_t *n_groups,
                           int32_t *max_members, int32_t *max_prefix);

/* Workspace bytes paged_attention_decode_shared needs (the larger of what
 * it and paged_attention_decode need for these sizes). */
int paged_attention_shared_workspace_size(int32_t B, int32_t nq, int32_t Hq,
                                          int32_t Hkv, int32_t D,
                                          int32_t max_blocks,
                                          int32_t block_size,
                                          int32_t partition_tokens,
                                          int32_t n_groups, int32_t max_members,
                                          int32_t max_prefix, size_t *bytes);

/* paged_attention_decode with each group's shared prefix read once per KV
 * head for all its members: the query rows of a group's members are
 * stacked into 16-row MFMA tiles that stream the prefix blocks together,
 * the rest of every context (from seq_prefix[b] on) runs on the ordinary
 * kernels, and a log-sum-exp merge joins the parts. Same results as
 * paged_attention_decode (up to float32 rounding order and, in the prefix
 * part, weights rounded to bf16 for the MFMA product, as in its nq > 1
 * path). bf16 caches only; G * nq rounded up to a power of two <= 16.
 *   seq_prefix, group_start, members, group_tokens: device int32 copies of
 *     paged_kv_prefix_groups' outputs (members' tables must hold the same
 *     block ids over the group's prefix, and seq_prefix[b] must be the
 *     group's prefix for members and 0 otherwise);
 *   n_groups, n_members = group_start[n_groups], max_members, max_prefix:
 *     the host-side values of the same call (they size the launch).
 * Inconsistent group arrays give wrong or NaN results but no access
 * outside the arrays. With n_groups = 0 this is paged_attention_decode.
 * Host-checked: as paged_attention_decode, plus dtype bf16, the group
 * sizes, and a workspace of paged_attention_shared_workspace_size(). */
int paged_attention_decode_shared(
    float *out, const void *q, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks,
    const int32_t *context_lens, int32_t B, int32_t nq, int32_t Hq,
    int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
    float scale, int dtype, int32_t partition_tokens,
    const int32_t *seq_prefix, const int32_t *group_start,
    const int32_t *members, const int32_t *group_tokens, int32_t n_groups,
    int32_t n_members, int32_t max_members, int32_t max_prefix,
    void *workspace, size_t workspace_bytes, float *lse_out, void *stream);

/* ======================================================================
 * Measurement aid (not part of the attention path)
 * ====================================================================== */

/* Read n_chunks chunks of chunk_bytes bytes (1, 2, 4 or 8 KiB) from the
 * device buffer buf (buf_bytes long, 16-byte aligned): chunk k at byte
 * order[k] * chunk_bytes (order: device int32; an entry at or past
 * buf_bytes / chunk_bytes reads the last whole chunk). n_wg workgroups of
 * eight wavefronts; wavefront w of workgroup x takes chunks x * 8 + w,
 * + 8 n_wg, ... Each lane loads 16 bytes per 1 KiB, as the decode kernels
 * load K/V rows: mode 0 into registers, mode 1 into registers with
 * non-temporal loads, mode 2 with the non-temporal direct-to-LDS gathers
 * the decode kernels use into a ring of ring_bytes (4, 8 or 16 KiB, at
 * least one chunk; ignored by modes 0 and 1) per wavefront, read back from
 * LDS: ring_bytes is what each wavefront keeps in flight. sink (device,
 * n_wg uint32) receives each workgroup's XOR of every
 * 32-bit word it read. With order = 0, 1, 2, ... it measures a sequential
 * read stream; with a random permutation, the reads of a cache whose blocks
 * came from a shuffled free list. Returns PKV_EINVAL for sizes or a mode out
 * of range, PKV_EHIP if the launch fails. */
int paged_kv_read_probe(const void *buf, size_t buf_bytes, const int32_t *order,
                        int32_t n_chunks, int32_t chunk_bytes, int mode, int32_t ring_bytes,
                        int32_t n_wg, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
