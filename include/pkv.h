/*
 * pkv.h -- C ABI of libpkv: a paged KV cache for MI355X (gfx950) whose write
 * side injects precomputed, unrotated K/V into fixed 16-token blocks (rotating
 * each key to its destination position as it is written) and whose read side
 * runs grouped-query decode attention through per-sequence block tables.
 *
 * Sources, cited by page title and section:
 *   [InferScale]     "InferScale: GPU-Native KV Injection for Personalized LLM
 *                    Serving"
 *   [KV essay]       "LLM Inference: KV Caching"
 *   [Inside engines] "Inside LLM Inference Engines: KV Caching,
 *                    PagedAttention, and Continuous Batching"
 *   [KV management]  "Latency Optimization > KV Cache Management"
 *
 * Conventions for every entry point:
 *   - Returns a pkv_status (0 = PKV_OK, negative = error) unless noted.
 *   - All argument checks run on the host before anything is enqueued; on an
 *     error nothing is enqueued, no host state changes, and pkv_last_error()
 *     describes the problem.
 *   - "device" pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or retains them beyond the enqueued work, which
 *     must complete before the caller frees them.  "host" pointers are read or
 *     written before the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously; no call synchronises the
 *     device except where stated.
 *   - Element strides and offsets are in elements of the stated dtype.
 *   - Index data that lives on the device (block tables, positions) is
 *     range-checked inside the kernels: an out-of-range block id or position
 *     is never dereferenced; the element it would have produced is skipped.
 *   - A pkv_cache or pkv_plan is not thread-safe: one host thread at a time.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 9
/* Tokens per physical block ([InferScale] §2; [KV essay] "Paged attention"). */
#define PKV_BLOCK_TOKENS 16

typedef int32_t pkv_status;
#define PKV_OK             0
#define PKV_E_INVALID     -1  /* bad argument, unknown sequence, bad state   */
#define PKV_E_OOM         -2  /* the free list cannot cover a reservation    */
#define PKV_E_RANGE       -3  /* position/length beyond capacity or table    */
#define PKV_E_OVERLAP     -4  /* two tokens of one inject call, one slot     */
#define PKV_E_WORKSPACE   -5  /* device workspace missing or too small       */
#define PKV_E_HIP         -6  /* a HIP runtime call or launch failed         */
#define PKV_E_UNSUPPORTED -7  /* shape/dtype combination not implemented     */

/* Element formats.  A pool holds F32, BF16, F16 or FP8E4M3; injected and
 * appended K/V and q are F32, BF16 or F16.  FP8E4M3 is the OCP 8-bit E4M3
 * format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
 * finite value 448, no infinities): a quantised cache, which the int8/int4
 * paragraph of [KV management] motivates, halving decode bytes. */
#define PKV_F32     0
#define PKV_BF16    1
#define PKV_F16     2
#define PKV_FP8E4M3 3

/* RoPE pairings ([InferScale] §2: R_p is block-diagonal with 2x2 rotations).
 * PAIRS rotates dimensions (2i, 2i+1); HALVES rotates (i, i+d/2); NONE stores
 * keys as given (already rotated by the caller). */
#define PKV_ROPE_PAIRS  0
#define PKV_ROPE_HALVES 1
#define PKV_ROPE_NONE   2

typedef struct pkv_cache pkv_cache; /* host allocator state (opaque)      */
typedef struct pkv_plan pkv_plan;   /* host decode split plan (opaque)    */

/* ---------------------------------------------------------------------------
 * Data descriptors
 * ------------------------------------------------------------------------- */

/* The paged pool of one model ([KV essay] "Paged attention": a shared pool of
 * fixed blocks).  For every (layer, physical block, KV head) there is one K
 * plane and one V plane of 16*head_dim elements each:
 *   K plane base = k + layer*layer_stride + block*block_stride + head*head_stride
 *   V plane base = v + (same offset)
 * Inside a K plane, element (token t in block, dim j) is at
 *   ((j / X) * 16 + t) * X + (j % X),   X = 16 bytes / element size,
 * i.e. d/X chunks of X consecutive dims for all 16 tokens.  Inside a V plane,
 * element (t, j) is at j * 16 + t (dimension-major).  Planes must be 16-byte
 * aligned (base pointers and every stride times the element size a multiple
 * of 16).  dtype is PKV_F32, PKV_BF16, PKV_F16 or PKV_FP8E4M3; head_dim is 64
 * or 128.  An FP8E4M3 pool stores code = e4m3(x / scale) (round to nearest
 * even, saturating at 448) with float scales for K and for V ("Latency
 * Optimization > KV Cache Management": a quantised cache keeps a scale
 * beside its codes), chosen by scale_mode:
 *   0: one per (layer, KV head); k_scale, v_scale are device
 *      float [n_layers][n_kv_heads];
 *   1: one per (layer, block, KV head); k_scale, v_scale are device
 *      float [n_layers][num_blocks][n_kv_heads].  A block's entries must hold
 *      its scales before anything is written to it (the caller sets them,
 *      e.g. from the magnitudes the block will hold); pkv_copy_blocks copies
 *      a block's entries along with its planes, so in this mode it writes
 *      through k_scale and v_scale.
 * The scale pointers are NULL and scale_mode 0 for the other formats. */
typedef struct {
  int32_t n_layers;
  int32_t num_blocks;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t scale_mode;   /* FP8E4M3 pools: 0 per (layer, head), 1 per (layer, block, head) */
  void* k;              /* device */
  void* v;              /* device */
  int64_t layer_stride; /* elements */
  int64_t block_stride; /* elements */
  int64_t head_stride;  /* elements */
  const float* k_scale; /* device, FP8E4M3 pools only */
  const float* v_scale; /* device, FP8E4M3 pools only */
} pkv_pool;

/* The store of precomputed, unrotated K/V ([InferScale] §3: keys captured
 * before the rotary embedding, kept with their values, per layer).  Element
 * (layer, token, kv head, dim) is at layer*layer_stride + token*token_stride +
 * head*head_dim + dim, for K at k and V at v.  Same n_kv_heads and head_dim
 * as the pool; 16-byte aligned rows.  dtype is the pool's, or PKV_BF16 /
 * PKV_F16 for an FP8E4M3 pool.
 *
 * The store may live in device memory or in pinned host memory (allocated
 * with hipHostMalloc, or a torch tensor with pin_memory=True): [InferScale]
 * §6 keeps the pre-RoPE store in pinned host DRAM and streams only the
 * retrieved facts over PCIe.  The inject kernel then reads exactly the rows
 * its runs name straight from host memory over PCIe while it writes the
 * pool, so transfer and scatter overlap in one pass.  Any other host pointer
 * (pageable memory) is rejected with PKV_E_INVALID before work is enqueued;
 * pinned memory must stay allocated and unchanged until the call's kernels
 * finish. */
typedef struct {
  const void* k;        /* device, or pinned host */
  const void* v;        /* device, or pinned host */
  int64_t layer_stride; /* elements */
  int64_t token_stride; /* elements */
  int64_t n_tokens;     /* tokens per layer (for range checks) */
  int32_t dtype;        /* format of the stored K/V */
  int32_t _reserved;
} pkv_src;

/* One injected run: source tokens src_token .. src_token+n_tokens-1 land at
 * positions dst_pos .. dst_pos+n_tokens-1 of sequence seq. */
typedef struct {
  int32_t seq;
  int32_t n_tokens;
  int32_t dst_pos;
  int32_t _reserved;
  int64_t src_token;
} pkv_run;

/* Host allocator configuration. free_list_seed 0 = ascending initial order;
 * otherwise the Fisher-Yates shuffle (i from N-1 down to 1, j = next() mod
 * (i+1)) driven by splitmix64 seeded with free_list_seed.
 *
 * block_tokens: tokens per allocation block, 16 (or 0) or 32 ([Inside
 * engines] "PagedAttention": blocks of e.g. 16 or 32 tokens).  A 32-token
 * block b is the pair of 16-token planes 2b and 2b+1 of the pool (which then
 * holds 2 * num_blocks planes); allocation, sharing, copy-on-write, prefix
 * entries and window trimming work in blocks of block_tokens, while
 * pkv_block_table exports the table of 16-token planes every kernel reads. */
typedef struct {
  int32_t num_blocks;
  int32_t max_seqs;
  int32_t max_blocks_per_seq;
  int32_t block_tokens;
  uint64_t free_list_seed;
} pkv_cache_config;

/* ---------------------------------------------------------------------------
 * Library
 * ------------------------------------------------------------------------- */

/* PKV_ABI_VERSION of the built library. */
int32_t pkv_abi_version(void);

/* Message of the last error on this thread ("" if none).  Valid until the next
 * pkv_* call on the same thread. */
const char* pkv_last_error(void);

/* Bytes of K plus V for n_tokens tokens: 2 * n_layers * n_kv_heads * head_dim
 * * elem_bytes * n_tokens ([Inside engines] "The KV Cache: Mathematical
 * Formulation & Memory Footprint"; [KV essay] "What the cache costs";
 * [InferScale] §3, per-fact storage).  Returns 0 for a negative argument. */
uint64_t pkv_kv_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                      int32_t elem_bytes, int64_t n_tokens);

/* ---------------------------------------------------------------------------
 * Host block allocator ([KV essay] "Paged attention": free list, per-sequence
 * block table, a new block handed out when a sequence reaches it;
 * [Inside engines] "PagedAttention", "Continuous Batching": blocks return to
 * the pool when a sequence ends).  Blocks are taken from the head of a FIFO
 * free list and returned to its tail in table order.
 *
 * Blocks may be shared ([KV essay] "Paged attention", "Prefix caching";
 * [KV management] on beam search, parallel sampling and prefix caching;
 * [Inside engines] "Zero-Copy Page Sharing"): every block has a reference
 * count, the number of table entries naming it, and is on the free list
 * exactly when that count is 0 (a block leaves the free list when handed out
 * or taken back by pkv_prefix_match, and rejoins its tail when its count
 * drops to 0).  Before a sequence writes into a block whose count exceeds 1,
 * it takes a fresh block from the free list's head (copy-on-write): the pair
 * (old, new) is queued, the sequence's table entry becomes the new block and
 * the old block's count drops by one.  Queued copies must be carried out,
 * in queue order, before the written positions are used: pkv_inject does so
 * itself; after pkv_extend call pkv_copy_blocks before appending.
 * ------------------------------------------------------------------------- */

/* Create an allocator. *out receives the handle. Errors: INVALID. */
pkv_status pkv_cache_create(const pkv_cache_config* cfg, pkv_cache** out);

/* Destroy an allocator (NULL is ignored). */
void pkv_cache_destroy(pkv_cache* cache);

/* Grow seq's blocks until it can hold n_tokens positions (its length is
 * unchanged).  All-or-nothing.  Errors: INVALID (seq, n_tokens < 0),
 * RANGE (more than max_blocks_per_seq blocks), OOM. */
pkv_status pkv_alloc_blocks(pkv_cache* cache, int32_t seq, int64_t n_tokens);

/* Give an empty sequence an explicit table (host ids[n_ids], each currently
 * free, no repeats) and length len <= 16*n_ids.  The ids leave the free list,
 * whose remaining order is kept.  Errors: INVALID, RANGE. */
pkv_status pkv_set_blocks(pkv_cache* cache, int32_t seq, const int32_t* ids,
                          int32_t n_ids, int64_t len);

/* Append n_new positions to each of seqs[n_seqs] (host, distinct), reserving
 * a block whenever a sequence crosses a 16-token boundary.  Every block
 * already in a sequence's table that will hold one of its new positions (the
 * partly filled block at its length, and reserved blocks past it, which a
 * fork shares as well) and that other sequences share is copied first
 * (queued; see pkv_copy_blocks), sequences in list order, blocks in table
 * order.  All-or-nothing over the whole list (the copies count as
 * reservations).
 * first_pos_out (host, may be NULL) receives each sequence's first new
 * position (its old length).  Errors: INVALID, RANGE, OOM. */
pkv_status pkv_extend(pkv_cache* cache, const int32_t* seqs, int32_t n_seqs,
                      int32_t n_new, int64_t* first_pos_out);

/* Drop seq's reference to each of its blocks in table order; blocks whose
 * count reaches 0 join the tail of the free list.  Its length becomes 0. */
pkv_status pkv_free_seq(pkv_cache* cache, int32_t seq);

/* Export block tables of 16-token planes: table_out (host, n_seqs rows of
 * pkv_table_width(cache) int32, padded with -1; a 32-token block b appears
 * as planes 2b, 2b+1) and lens_out (host, n_seqs int64; may be NULL). */
pkv_status pkv_block_table(const pkv_cache* cache, const int32_t* seqs, int32_t n_seqs,
                           int32_t* table_out, int64_t* lens_out);

/* Entries per exported table row: max_blocks_per_seq * block_tokens / 16;
 * -1 for a NULL cache. */
int32_t pkv_table_width(const pkv_cache* cache);

/* Number of free blocks. Returns -1 for a NULL cache. */
int32_t pkv_num_free_blocks(const pkv_cache* cache);

/* Copy the free list, head first, into out (host, capacity cap).  Returns the
 * number of entries copied, or a negative status. */
int32_t pkv_free_list(const pkv_cache* cache, int32_t* out, int32_t cap);

/* Give the empty sequence dst_seq the table and length of src_seq (every
 * block's count + 1), as beams or parallel samples share their prompt
 * ([KV management]).  No device work.  Errors: INVALID (bad or equal ids,
 * dst_seq not empty). */
pkv_status pkv_fork(pkv_cache* cache, int32_t src_seq, int32_t dst_seq);

/* Reference count of a block (>= 0), or a negative status. */
int32_t pkv_block_refcount(const pkv_cache* cache, int32_t block);

/* Copy the queued copy-on-write pairs (src, dst), oldest first, into
 * pairs_out (host, cap pairs of two int32).  Returns the number queued (which
 * may exceed cap), or a negative status. */
int32_t pkv_pending_copies(const pkv_cache* cache, int32_t* pairs_out, int32_t cap);

/* Carry out the queued copies on `stream` and empty the queue: for each pair,
 * every layer's K and V planes (all KV heads) of block src are copied into
 * block dst; for an FP8E4M3 pool with scale_mode 1, block dst's scale
 * entries (every layer and KV head, K and V) are set to block src's.  The
 * result equals doing them one after another in queue order.
 * The pool's blocks must include every queued id.  Device work only; the
 * pool must not be written by other work until the copies finish (stream
 * order suffices).  Errors: INVALID, RANGE (an id outside the pool), HIP. */
pkv_status pkv_copy_blocks(pkv_cache* cache, const pkv_pool* pool, void* stream);

/* Prefix cache ([KV essay] "Prefix caching"; [KV management]: engines look
 * prefixes up by a hash, and reuse needs identical tokens from position 0
 * on).  The caller names what each position holds by a 64-bit key
 * (a token id of a prompt, or the store row of injected memory).  A full
 * block is registered under (the block registered for the preceding 16
 * positions, or -1 at position 0; its 16 keys), compared exactly.  An entry
 * lasts until its block is handed out again by the free list, given out by
 * pkv_set_blocks, or written in place by pkv_inject; it then goes together
 * with every entry registered under it. */

/* For an empty sequence: share the longest chain of registered blocks that
 * matches keys[0 .. n_keys) (host) block by block from position 0 (a block
 * with count 0 is taken back off the free list); the sequence's length
 * becomes the matched token count, written to *matched_out (host, may be
 * NULL), a multiple of 16.  Errors: INVALID (sequence not empty, bad keys). */
pkv_status pkv_prefix_match(pkv_cache* cache, int32_t seq, const uint64_t* keys,
                            int64_t n_keys, int64_t* matched_out);

/* Register the full blocks of seq covered by keys[0 .. n_keys) (host,
 * n_keys <= length): a block whose (predecessor, keys) is already registered
 * is skipped (later blocks chain off the registered one).  Errors: INVALID
 * (a block already registered under other keys; nothing is registered),
 * RANGE (n_keys beyond the length). */
pkv_status pkv_prefix_commit(pkv_cache* cache, int32_t seq, const uint64_t* keys,
                             int64_t n_keys);

/* Number of registered blocks, or -1 for a NULL cache. */
int32_t pkv_prefix_cached_blocks(const pkv_cache* cache);

/* Sliding window ([KV essay] "Capping the window instead of shrinking the
 * rows": entries older than the window can be discarded, so the cache's size
 * is bounded by the window).  For each of seqs[n_seqs] (host), drop the references to
 * the blocks lying wholly before its last `window` positions, in table order
 * (blocks reaching count 0 join the free list's tail); their table entries
 * become -1.  Lengths and positions are unchanged; writing a dropped position
 * later is refused (RANGE).  *dropped_out (host, may be NULL) receives the
 * number of entries dropped.  Errors: INVALID (bad ids, window <= 0). */
pkv_status pkv_trim_window(pkv_cache* cache, const int32_t* seqs, int32_t n_seqs,
                           int32_t window, int64_t* dropped_out);

/* ---------------------------------------------------------------------------
 * Rotary table ([InferScale] §2 and §3.3: keys are rotated with the model's
 * own rotary tables).  theta_i = base^(-2i/d); cos_out[p][i] and sin_out[p][i]
 * (host, max_pos x d/2 float each) are cos and sin of p*theta_i evaluated in
 * double precision and rounded once to float.
 * ------------------------------------------------------------------------- */
pkv_status pkv_rope_table(int32_t head_dim, double base, int32_t max_pos,
                          float* cos_out, float* sin_out);

/* ---------------------------------------------------------------------------
 * Inject ([InferScale] §3, connector steps 2-3 and the worker-side scatter
 * copy through the slot mapping; §3.3 and §5.1, chunked RoPE): for every run
 * token and every layer in [layer_begin, layer_end):
 *   K[slot(seq, p)] = round(R_p * k_src),  V[slot(seq, p)] = v_src  (bit copy)
 * with slot(seq, p) = table[seq][p / 16] * 16 + p % 16 taken from the host
 * allocator, R_p the rotation by the rotary table (cos, sin: device, max_pos
 * x d/2 float) applied in float32 without fused multiply-add, and round the
 * round-to-nearest-even store into the pool dtype.  Each run must lie within
 * its sequence's reserved blocks and below max_pos; two tokens of one call
 * may not target one position of one sequence (PKV_E_OVERLAP).  Destination
 * blocks shared with other sequences are copied first (copy-on-write, blocks
 * in order of first touch: runs in order, positions ascending; OOM when the
 * free list cannot cover the copies), a written block loses its prefix-cache
 * entry, and every queued copy is carried out on `stream` before the write.
 * Afterwards each sequence's length is max(length, dst_pos + n_tokens) over its
 * non-empty runs.  An empty run (n_tokens = 0) writes nothing: past the sequence
 * and sign checks it is neither range-checked nor counted.  Runs are host memory.  The device
 * workspace (d_ws, ws_bytes >= pkv_inject_workspace_bytes(runs, n_runs)) holds
 * the per-block write plan; it must not be reused by other work until this
 * call's kernels finish (stream order suffices).
 * ------------------------------------------------------------------------- */
size_t pkv_inject_workspace_bytes(const pkv_run* runs, int32_t n_runs);

/* Page-locked host memory for a host-resident source store ([InferScale] §6:
 * the pre-RoPE store kept in pinned host DRAM, only the retrieved rows read
 * over PCIe).  *out receives n_bytes (> 0) of pinned host memory that
 * pkv_inject can read directly; the caller fills it and releases it with
 * pkv_host_free.  Errors: INVALID, HIP (the allocation failed). */
pkv_status pkv_host_alloc(size_t n_bytes, void** out);

/* Release memory from pkv_host_alloc (NULL is ignored).  No enqueued kernel
 * may still read it.  Errors: HIP. */
pkv_status pkv_host_free(void* p);

pkv_status pkv_inject(pkv_cache* cache, const pkv_pool* pool, const pkv_src* src,
                      const pkv_run* runs, int32_t n_runs, int32_t layer_begin,
                      int32_t layer_end, int32_t rope_mode, const float* d_cos,
                      const float* d_sin, int32_t max_pos, void* d_ws, size_t ws_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Append ([InferScale] §2 and [KV essay] "The fix": decoding appends one K/V
 * entry per generated token): for b < n_seqs and t < n_new, token t of
 * sequence b lands at position p = d_first_pos[b] + t through row b of the
 * device block table (d_tables, int32, row stride table_stride):
 *   K[slot] = round(R_p * k_new[b][t]),  V[slot] = v_new[b][t]
 * k_new, v_new: device, [n_seqs][n_new][n_kv_heads][head_dim] in new_dtype
 * (the pool's, or PKV_BF16 / PKV_F16 for an FP8E4M3 pool).
 * d_first_pos: device int32[n_seqs] (the first_pos_out of pkv_extend), with
 * d_first_pos[b] + n_new <= INT32_MAX.  The table and the first positions are
 * device data and are range-checked: a token is skipped (not written) when
 * its position is negative, lies past the table row (p / 16 >= table_stride),
 * has no rotary row under a rotary pairing (p >= max_pos, rope_mode other
 * than PKV_ROPE_NONE), or when its table entry is not a block id in
 * [0, num_blocks).
 * ------------------------------------------------------------------------- */
pkv_status pkv_append_kv(const pkv_pool* pool, int32_t layer, const int32_t* d_tables,
                         int32_t table_stride, const int32_t* d_first_pos, int32_t n_seqs,
                         int32_t n_new, const void* d_k_new, const void* d_v_new,
                         int32_t new_dtype, int32_t rope_mode, const float* d_cos,
                         const float* d_sin, int32_t max_pos, void* stream);

/* ---------------------------------------------------------------------------
 * Decode attention ([KV essay] "First, what K and V are": softmax(q K^T /
 * sqrt(d)) V for one query row per head; "Paged attention": K/V read through
 * the block table; "What the cache costs" and [KV management]: query head h
 * reads KV head h / (n_q_heads / n_kv_heads)).  Sequence b attends to its
 * lens[b] cached tokens (positions 0 .. lens[b]-1, no mask), or, under a
 * sliding window (window > 0; [KV essay] "Capping the window instead of
 * shrinking the rows": attention covers a trailing span of W positions), to
 * positions max(0, lens[b] - window) .. lens[b]-1; blocks before those
 * positions are never read, so a table trimmed by pkv_trim_window with a
 * window >= this one decodes the same.
 *
 * A plan fixes the lengths (host, int64 lens[n_seqs]) and splits every
 * sequence longer than part_tokens (a multiple of 16; 0 = chosen from the
 * total work) into ranges of part_tokens tokens, which run on separate
 * workgroups; their softmax states (running max, sum, unnormalised output)
 * are merged by log-sum-exp in ascending range order.  Upload the plan into a device workspace once, then
 * call pkv_decode_attention for every layer that shares the lengths.
 *
 * Outputs: d_out (device float [n_seqs][n_q_heads][head_dim]) and, if not
 * NULL, d_lse (device float [n_seqs][n_q_heads], ln of the sum of exp of the
 * scaled scores).  A sequence of length 0 gets out = 0, lse = -inf.  A plan
 * of no sequences (n_seqs = 0) is valid: decode calls with it check the pool
 * and layer, enqueue nothing and read none of their device pointers.
 * q: device [n_seqs][n_q_heads][head_dim] in q_dtype (the pool's; PKV_BF16 or
 * PKV_F16 for an FP8E4M3 pool), already rotated to its own position.
 * scale <= 0 selects 1/sqrt(head_dim).  An FP8E4M3 pool takes up to 64 query
 * heads per KV head (PKV_E_UNSUPPORTED beyond); other pools take any group.
 * ------------------------------------------------------------------------- */
pkv_status pkv_decode_plan_create(const int64_t* lens, int32_t n_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t part_tokens,
                                  int32_t window, pkv_plan** out);

void pkv_decode_plan_destroy(pkv_plan* plan);

/* Number of work items (sequence token ranges) of a plan; -1 for NULL. */
int32_t pkv_decode_plan_items(const pkv_plan* plan);

/* Token range length the plan chose; -1 for NULL. */
int32_t pkv_decode_plan_part_tokens(const pkv_plan* plan);

/* Waves per workgroup the plan chose (1, 2, 4 or 8): the waves of one
 * workgroup take turns over the blocks of one token range and merge their
 * softmax states in LDS; -1 for NULL. */
int32_t pkv_decode_plan_waves(const pkv_plan* plan);

/* Device workspace a plan needs (work list, each sequence's newest position,
 * float partials). */
size_t pkv_decode_workspace_bytes(const pkv_plan* plan);

/* Copy the plan's work list into the workspace (asynchronous on stream; the
 * host copy is kept in library-owned pinned memory until it has landed).
 * A plan of at most 128 work items that splits no sequence, and whose
 * launches have fewer than 16 workgroups (items x KV heads) per compute unit
 * of the current device, travels in each decode launch's kernel arguments
 * instead: for it this call validates the workspace and enqueues nothing. */
pkv_status pkv_decode_plan_upload(pkv_plan* plan, void* d_ws, size_t ws_bytes, void* stream);

pkv_status pkv_decode_attention(const pkv_plan* plan, const pkv_pool* pool, int32_t layer,
                                const void* d_q, int32_t q_dtype, float scale,
                                const int32_t* d_tables,
                                int32_t table_stride, float* d_out, float* d_lse, void* d_ws,
                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One decode step's append and attention, in one launch ([KV essay] "The
 * fix": each generated token's K/V entry is appended and the step attends
 * over the cache including it; [InferScale] §2: the key is stored rotated at
 * its own position).  Launches of many workgroups on 16-bit pools (at least
 * 16 per CU, e.g. ragged batches of short sequences) run it as two launches,
 * the append and then attention alone, which measured faster there; the
 * results are the same.  Equal, byte for byte in the pool and in d_out/d_lse, to
 *   pkv_append_kv(pool, layer, d_tables, table_stride, first_pos = lens - 1,
 *                 n_seqs, 1, d_k_new, d_v_new, q_dtype, rope_mode, d_cos,
 *                 d_sin, max_pos)
 * followed by pkv_decode_attention with the same plan: every sequence b of
 * the plan with lens[b] >= 1 gets its newest token, at position lens[b] - 1,
 * written (K rotated by R_p, V as given) and attended to.  Sequences of
 * length 0 get no write.
 * k_new, v_new: device [n_seqs][n_kv_heads][head_dim] in q_dtype, 16-byte
 * aligned, unrotated.  The slot of position lens[b] - 1 must be reserved
 * (pkv_extend); a block id out of range in its table entry skips the write,
 * as pkv_append_kv does.  The block holding that slot may be written back
 * whole (its other slots with the bytes they held), so, as for any write, it must
 * belong to this sequence alone: pkv_extend copies a shared block first.
 * Errors, all before anything is enqueued: those of
 * pkv_decode_attention; PKV_E_INVALID for misaligned k_new/v_new, for null
 * ones when the plan has a sequence, or for bad rotary arguments; PKV_E_RANGE when a newest position has no rotary row
 * (>= max_pos, rope_mode other than PKV_ROPE_NONE).
 * ------------------------------------------------------------------------- */
pkv_status pkv_append_decode_attention(const pkv_plan* plan, const pkv_pool* pool, int32_t layer,
                                       const void* d_q, int32_t q_dtype, float scale,
                                       const int32_t* d_tables, int32_t table_stride,
                                       const void* d_k_new, const void* d_v_new,
                                       int32_t rope_mode, const float* d_cos,
                                       const float* d_sin, int32_t max_pos, float* d_out,
                                       float* d_lse, void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The decode step without any allocation, for callers that cannot allocate
 * device or pinned memory at the call: code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * checks, results and stream behaviour as pkv_append_decode_attention, except
 * that there is no workspace argument and no separate plan upload: the
 * plan's work list (24 bytes per item, 16 per split sequence, 4 per
 * sequence for its newest position) is copied from
 * the plan's host memory into a static device scratch buffer on `stream`,
 * and the kernels use that buffer for the work list and the partial states
 * of split sequences.  The scratch holds PKV_NOALLOC_SCRATCH_BYTES (16 MiB)
 * per device, reserved on each device the library runs on until the process
 * ends; a plan whose pkv_decode_workspace_bytes exceeds it is refused with
 * PKV_E_WORKSPACE before anything is enqueued.  The call makes no device or
 * pinned-host allocation and no library allocation (pkv_kernel_timing does
 * not apply to it).  Every call on one device shares that device's scratch:
 * calls on one device that overlap in time (different streams, or host
 * threads) race on it, so order them on one stream.  Nothing in the scratch
 * needs clearing between calls: each call rewrites the work list, and every
 * partial state is written before it is read.
 * ------------------------------------------------------------------------- */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status pkv_append_decode_attention_noalloc(const pkv_plan* plan, const pkv_pool* pool,
                                               int32_t layer, const void* d_q, int32_t q_dtype,
                                               float scale, const int32_t* d_tables,
                                               int32_t table_stride, const void* d_k_new,
                                               const void* d_v_new, int32_t rope_mode,
                                               const float* d_cos, const float* d_sin,
                                               int32_t max_pos, float* d_out, float* d_lse,
                                               void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helper: kernel durations from the dispatches themselves.
 * pkv_kernel_timing(1) makes every following decode launch on the calling
 * thread (pkv_decode_attention, pkv_append_decode_attention; the attention
 * kernel, not a split sequence's merge kernel) carry a start/stop event pair
 * attached to its own dispatch, so that the pair spans that dispatch and the
 * kernel's execution, not the neighbouring work on the stream (on MI355X
 * about 4 us more than the kernel's own start and end timestamps);
 * pkv_kernel_timing(0) stops that.  pkv_kernel_times waits for
 * the recorded launches, writes up to max_n durations in milliseconds
 * (host float array) in launch order, releases every recorded pair and
 * returns the number recorded (PKV_E_INVALID for a bad buffer, PKV_E_HIP if
 * an event failed).
 * ------------------------------------------------------------------------- */
pkv_status pkv_kernel_timing(int32_t enable);
int32_t pkv_kernel_times(float* ms_out, int32_t max_n);

/* ---------------------------------------------------------------------------
 * Measurement helper: a streaming 16-byte-per-lane read of n_bytes (a
 * multiple of 16) from d_src, reduced into d_sink (device, >= 16 bytes), to
 * measure the achievable HBM read rate in the same process.
 * ------------------------------------------------------------------------- */
pkv_status pkv_bw_probe(const void* d_src, size_t n_bytes, void* d_sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
