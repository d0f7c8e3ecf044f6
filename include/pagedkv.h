/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV cache and decode
 * attention library, libpagedkv.so.
 *
 * The library owns a pool of fixed-size physical KV blocks in device memory,
 * hands them to sequences through per-sequence block tables, scatters new K/V
 * into the pool (kv_append) and runs single-token decode attention through
 * the tables (paged_decode).  Pages cited by address and section:
 *   [cf1]  www.cf-1.com/news/5824798        KV memory analysis + PagedAttention
 *   [moo]  www.mooersco.com/news/1484987    practitioner guide
 *   [mlqm] www.mlqm.cn/news/394450          KV Cache explainer
 *   [lqnn] m.lqnn.cn/news/219451            capacity planning and strategy
 *   [xph]  inference.xph.ink kp-013         "KV Cache：原理与显存占比"
 *
 * Conventions for every entry point
 *   - Every function returns a pkv_status (0 = PKV_OK) unless stated, and
 *     never lets a C++ exception cross the ABI.  On failure
 *     pkv_last_error() returns a thread-local message.
 *   - "host" pointers are CPU memory, "device" pointers are HIP device memory
 *     of the GPU current when the pool was created.  The caller owns every
 *     pointer it passes; the library copies what it keeps.
 *   - Streams are hipStream_t handles passed as void*; NULL is the default
 *     stream.  kv_append and paged_decode are asynchronous on that stream:
 *     inputs must stay alive and unmodified until the stream has passed them.
 *   - A pool is not thread-safe: calls on one pool must be serialised by the
 *     caller.
 *   - Arguments are validated before any device work.  Device-side contents
 *     (slot values, table entries, context lengths) cannot be validated on the
 *     host; the kernels bound-check them instead and skip what is out of
 *     range (documented per call), so no input can make a kernel read or
 *     write outside the pool or the caller's buffers.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned, bad combination */
    PKV_ERR_NO_BLOCKS = 2,     /* pool exhausted; nothing was changed */
    PKV_ERR_OUT_OF_RANGE = 3,  /* a table would not fit the caller's width, length overflow */
    PKV_ERR_STATE = 4,         /* unknown or freed sequence, wrong pool kind for the call */
    PKV_ERR_UNSUPPORTED = 5,   /* a (dtype, head_dim, group) combination with no kernel */
    PKV_ERR_DEVICE = 6         /* a HIP runtime call failed (allocation, copy, launch) */
} pkv_status;

/* Storage / element types. */
typedef enum {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2,
    PKV_FP8_E4M3 = 3,          /* OCP 8-bit float E4M3 ("FN": max 448, NaN 0x7F/0xFF) */
    PKV_INT8_MINMAX = 4        /* 8-bit codes with a min-max range per (block, KV head) tile,
                                  [moo] §3.3; see kv_append */
} pkv_dtype;

typedef struct kv_pool kv_pool_t;

typedef struct {
    void* k_pool;              /* device; [num_blocks][kv_heads] tiles of block_bytes: the tile is
                                  [block_size][head_dim] elements.  INT8: a block holds the
                                  kv_heads tiles' codes ([kv_heads][block_size][head_dim]), then
                                  their kv_heads 16-byte headers {min, max, step, 0} as fp32 */
    void* v_pool;              /* device; same layout, separate buffer */
    float* k_scale;            /* device; [kv_heads] (FP8 pools only, else NULL) */
    float* v_scale;            /* device; [kv_heads] (FP8 pools only, else NULL) */
    uint64_t pool_bytes;       /* bytes of ONE of k_pool / v_pool */
    uint64_t block_bytes;      /* bytes of one (block, kv head) tile = block_size*head_dim*elem
                                  (+ 16 for the INT8 header); a block spans kv_heads of them */
    uint64_t total_bytes;      /* device bytes owned: 2*pool_bytes + scales + a 4 KiB zero tile
                                  (+ 8 bytes per slot of append tags for INT8 pools) */
    int32_t num_blocks, block_size, kv_heads, head_dim, dtype, elem_bytes;
    int32_t free_blocks;       /* refcount 0 */
    int32_t used_blocks;       /* refcount >= 1 */
    int32_t shared_blocks;     /* refcount >= 2 */
    int32_t live_seqs;
    int32_t host_only;         /* 1: metadata-only pool, no device memory */
    int32_t partition_tokens;  /* current paged_decode partition setting (0 = automatic) */
    int32_t cached_blocks;     /* blocks findable by content key (prefix cache) */
    int32_t evictable_blocks;  /* cached blocks nobody holds (reusable, evicted oldest first) */
} kv_pool_info_t;

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

/* KV size formula, [cf1] §1.2 and [xph] "公式与模型": bytes of K and V for
 * `tokens` cached tokens of each of `seqs` sequences:
 *   2 * layers * kv_heads * head_dim * elem_bytes * tokens * seqs.
 * Returns 0 on invalid input (any of the first four <= 0, tokens or seqs < 0),
 * as the budget script of [lqnn] §2 refuses such shapes. */
uint64_t kv_cache_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim,
                        int32_t elem_bytes, int64_t tokens, int64_t seqs);

/* ---------------------------------------------------------------------------
 * Pool
 * ------------------------------------------------------------------------ */

/* Create a pool: pre-allocate the K and V block pools once ([moo] §2.2
 * "pre-allocation"; [cf1] §3.1 "one unified pool of fixed-size blocks"), with
 * the per-block layout [moo] §3.1 gives for one layer and separate K and V
 * buffers: [num_blocks][kv_heads][block_size][head_dim], 256-byte aligned,
 * zero-filled.  FP8 pools also hold per-KV-head fp32 scales for K and V
 * ([lqnn] §4, per-attention-head scales), initialised to 1.
 *   block_size        must be 16 ([cf1] §3.1 default).
 *   head_dim          16, 64 or 128 (a 16-token tile must be >= 256 bytes).
 *   dtype             a pkv_dtype.
 *   initial_free_order host, nullable: a permutation of 0..num_blocks-1 giving
 *                     the initial order of the FIFO free list; NULL means
 *                     0, 1, ..., num_blocks-1.
 * Errors: INVALID_ARG (<= 0 sizes, not a permutation, null out),
 * UNSUPPORTED (block_size != 16, head_dim, dtype), DEVICE (allocation). */
int kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t kv_heads,
                   int32_t head_dim, int32_t dtype, const int32_t* initial_free_order,
                   kv_pool_t** out);

/* Same pool bookkeeping with no device memory: block tables, refcounts and
 * slot mappings only (capacity planning, host tests).  kv_append,
 * paged_decode and kv_pool_copy_to_host on it return PKV_ERR_STATE after
 * their argument checks.  Touches no HIP API. */
int kv_pool_create_host_only(int32_t num_blocks, int32_t block_size, int32_t kv_heads,
                             int32_t head_dim, int32_t dtype,
                             const int32_t* initial_free_order, kv_pool_t** out);

/* Free the pool, its device memory and every sequence.  NULL is a no-op.  The
 * caller must make sure no stream still uses the pool. */
int kv_pool_destroy(kv_pool_t* pool);

/* Describe the pool (pointers, sizes, layout, block counts). */
int kv_pool_info(const kv_pool_t* pool, kv_pool_info_t* out);

/* Set the static per-KV-head FP8 scales (host arrays of kv_heads floats).
 * Stored values are code = E4M3_rne_satfinite(x * (1/scale)) and read back as
 * decode(code) * scale ([lqnn] §4: the scale sets the dynamic range; outliers
 * beyond it saturate).  The library keeps inv = 1.0f/scale (one fp32
 * division) for kv_append.  Synchronous.
 * Errors: STATE (not an FP8 pool), INVALID_ARG (null, <= 0 or non-finite). */
int kv_pool_set_fp8_scales(kv_pool_t* pool, const float* k_scale, const float* v_scale);

/* ---------------------------------------------------------------------------
 * Sequences and block tables (host only; [cf1] §3.2-§3.3)
 *
 * Free list: FIFO, seeded by initial_free_order.  A sequence takes blocks
 * from the front when a new token position p has p % block_size == 0 (only
 * its last block is ever partly filled).  Releasing a sequence decrements the
 * refcount of each of its blocks in reverse logical order (deepest first);
 * blocks reaching 0 go to the back of the free list, or of the evictable list
 * when they hold a cached prefix block.  Slot of logical position p:
 *   table[p / block_size] * block_size + p % block_size.
 * ------------------------------------------------------------------------ */

/* New sequence with an empty table; ids are never reused. */
int kv_seq_create(kv_pool_t* pool, int32_t* seq_id);

/* Reserve n_tokens new positions at the end of `seq`, taking blocks on
 * demand, and write their slots to slot_mapping_out (host, n_tokens int32;
 * may be NULL when n_tokens == 0).  All or nothing: on NO_BLOCKS nothing
 * changed.  Errors: STATE (unknown seq), INVALID_ARG (n_tokens < 0),
 * NO_BLOCKS, OUT_OF_RANGE (length beyond INT32_MAX). */
int kv_seq_reserve(kv_pool_t* pool, int32_t seq, int32_t n_tokens, int32_t* slot_mapping_out);

/* Reserve for a whole batch in one call: for i in 0..n-1, in order, reserve
 * n_tokens[i] (n_tokens NULL: 1 each) positions for seqs[i] and write their
 * slots consecutively to slots_out (host, sum of the counts int32).  The decode
 * step of a batch is one such call with one token per sequence.  All or
 * nothing over the whole batch: on NO_BLOCKS (or any error) nothing changed.
 * A sequence may appear more than once.  Errors: as kv_seq_reserve, plus
 * INVALID_ARG (n < 0, NULL arrays). */
int kv_batch_reserve(kv_pool_t* pool, const int32_t* seqs, int32_t n, const int32_t* n_tokens,
                     int32_t* slots_out);

/* New sequence sharing the first n_shared_tokens of `parent` by reference:
 * the child's table points at the same ceil(n_shared/block_size) physical
 * blocks, each of whose refcount is incremented ([cf1] §3.3: beam-search
 * branches and parallel samples share the prefix blocks; [lqnn] §3).  Any
 * length in [0, parent length] is allowed.  When a holder of a shared, partly
 * filled last block reserves new positions, it first takes a fresh block and
 * owes the device a copy of the shared one (copy-on-write, [cf1] §3.3); the
 * copy runs on the stream of the next kv_append / paged_decode /
 * kv_apply_copies on this pool, before that call's own work.  The K/V of the
 * shared tokens must therefore have been appended before the fork.
 * Errors: STATE, INVALID_ARG. */
int kv_seq_fork(kv_pool_t* pool, int32_t parent, int32_t n_shared_tokens, int32_t* child);

/* ---------------------------------------------------------------------------
 * Prefix cache ([cf1] §3.3: a content hash per KV block lets a new request
 * whose prompt prefix matches reuse the cached physical blocks and skip their
 * prefill; [lqnn] §3: model, tokenizer, LoRA, RoPE, tenant and version must be
 * part of the cache identity, here the caller's namespace `ns`).
 *
 * A full block's key chains its predecessor's: key_i = kv_block_hash(key_{i-1},
 * ns, tokens of block i), key_{-1} = 0.  The pool also keeps each cached
 * block's 16 token ids and shares a block only on an exact token match, so a
 * hash collision can never serve wrong content.  A cached block whose last
 * holder is released is not freed but kept, evictable; blocks are allocated
 * from the free list first and then by evicting the least recently released
 * cached block.
 * ------------------------------------------------------------------------ */

/* Key of one 16-token block: SplitMix64's output function folded over parent,
 * ns and the 16 token ids (tokens NULL: the key of an empty block). */
uint64_t kv_block_hash(uint64_t parent, uint64_t ns, const int32_t* tokens);

/* Publish the first floor(n_tokens / 16) full blocks of `seq`, whose token ids
 * are tokens[0 .. n_tokens) (host), under namespace ns.  Blocks whose content
 * key is already cached, or that already carry a key, are skipped;
 * *n_registered (nullable) receives the number newly cached.  The K/V of those
 * tokens must be (or be about to be) appended by the caller.
 * Errors: STATE (unknown seq), OUT_OF_RANGE (n_tokens > sequence length). */
int kv_prefix_register(kv_pool_t* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                       uint64_t ns, int32_t* n_registered);

/* New sequence starting on the longest cached prefix of tokens[0 .. n_tokens)
 * (host) under ns, whole blocks only: its table points at those cached blocks
 * (refcount + 1 each; evictable ones are taken back) and its length is
 * *n_cached_tokens, a multiple of 16.  The caller reserves and appends the
 * rest.  Never allocates, so it cannot run out of blocks. */
int kv_seq_create_cached(kv_pool_t* pool, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                         int32_t* seq_id, int32_t* n_cached_tokens);

/* Forget every content key (e.g. on a model or scale change): evictable cached
 * blocks return to the free list now, held ones when released. */
int kv_prefix_evict_all(kv_pool_t* pool);

/* Copy-on-write block copies owed to the device, oldest first: src[i] ->
 * dst[i] (host arrays of capacity cap; *n receives the count).
 * Errors: OUT_OF_RANGE if cap is too small. */
int kv_pending_copies(const kv_pool_t* pool, int32_t* src, int32_t* dst, int32_t cap, int32_t* n);

/* Perform the owed copy-on-write block copies now, asynchronously on `stream`
 * (both pools, all KV heads of each block), and clear the list.  kv_append and
 * paged_decode do this themselves first; a metadata-only pool just clears the
 * list.  Errors: DEVICE. */
int kv_apply_copies(kv_pool_t* pool, void* stream);

/* Release a sequence (see above).  Errors: STATE (unknown or already freed). */
int kv_seq_free(kv_pool_t* pool, int32_t seq);

/* Current length (tokens) of a sequence.  Errors: STATE. */
int kv_seq_length(const kv_pool_t* pool, int32_t seq, int32_t* len);

/* Block tables and context lengths of n sequences, for upload by the caller:
 * tables_out (host, [n][max_blocks_per_seq] int32; unused entries -1) and
 * context_lens_out (host, [n] int32).  Errors: STATE (unknown seq),
 * OUT_OF_RANGE (a table wider than max_blocks_per_seq), INVALID_ARG. */
int kv_block_tables(const kv_pool_t* pool, const int32_t* seqs, int32_t n,
                    int32_t max_blocks_per_seq, int32_t* tables_out,
                    int32_t* context_lens_out);

/* Refcount of a physical block (inspection).  Errors: INVALID_ARG. */
int kv_block_refcount(const kv_pool_t* pool, int32_t block, int32_t* out);

/* Copy the free list, front first, into out (host, capacity cap);
 * *n receives its length.  Errors: OUT_OF_RANGE if cap is too small. */
int kv_free_list(const kv_pool_t* pool, int32_t* out, int32_t cap, int32_t* n);

/* ---------------------------------------------------------------------------
 * Device work
 * ------------------------------------------------------------------------ */

/* Scatter new keys and values into the pool ([cf1] §1.1 and [mlqm] 四: only
 * the new token's K/V are computed and appended).  For token t and KV head g,
 *   pool[slot / bs][g][slot % bs][:] = k_new[t][g][:]   (same for V)
 * where slot = slot_mapping[t].
 *   slot_mapping  device, [T] int32.  A slot < 0 or >= num_blocks*block_size
 *                 skips that token.  Duplicate slots race (undefined which
 *                 token wins).
 *   k_new, v_new  device, [T][kv_heads][head_dim] of src_dtype, 16-byte
 *                 aligned.  src_dtype must equal the pool dtype, or be BF16
 *                 or F32 for an FP8 pool, which quantises in the kernel:
 *                 code = E4M3_rne_satfinite(x * inv_scale[g]), NaN -> 0x7F;
 *                 or BF16, F16 or F32 for an INT8 pool (below).
 * T == 0 is a no-op.
 *
 * INT8 pools ([moo] §3.3, per-block min-max): src_dtype is BF16, F16 or F32.
 * Each (block, KV head) tile keeps, for K and for V separately, a range
 * (min, max) and codes q = round_half_even((x - min) / (max - min) * 255),
 * every step in fp32 (max == min gives 0); a code stands for
 * min + q * (max - min) / 255.  The range is the min and max of every value
 * written into the tile since its row 0 was last written: a call that writes
 * row 0 of a tile starts it afresh (its other rows no longer count); any
 * other call widens the range to take its values and, if the range moved,
 * re-encodes the tile's other rows from their fp32 values min + q * step
 * (step = (max - min) / 255).  All rows one call writes into a tile are taken
 * together.  Inputs must be finite.  Two kernels run: one tags each written
 * slot with the call, one encodes each touched tile; the tags are the
 * library's, so calls on one pool must not overlap on the device.
 *
 * Errors: INVALID_ARG, UNSUPPORTED (dtype pairing), STATE (host-only pool),
 * DEVICE (launch). */
int kv_append(kv_pool_t* pool, const int32_t* slot_mapping, int32_t T,
              const void* k_new, const void* v_new, int32_t src_dtype, void* stream);

/* Single-token decode attention through block tables ([mlqm] 二 and 四:
 * softmax(Q K^T * scale) V for the newest query over every cached token;
 * [cf1] §3.1 block table; [mlqm] 六 GQA).  For sequence b, query head h,
 * G = H_q / kv_heads, g = h / G, n = context_lens[b]:
 *   z_j = scale * <q[b][h], K_b[j][g]>,   j = 0..n-1 (logical order; the
 *         newest token, appended before the call, is j = n-1)
 *   out[b][h] = sum_j softmax(z)_j * V_b[j][g]
 * where K_b[j] lives in block block_tables[b][j / 16], row j % 16.  For an FP8
 * pool the stored values are decode(code) * k_scale[g] (resp. v_scale[g]); for
 * an INT8 pool, min + code * (max - min) / 255 of the token's tile.
 *   q             device [B][H_q][head_dim] of q_dtype (= pool dtype; BF16
 *                 or F16 for an FP8 or INT8 pool), 16-byte aligned.
 *   block_tables  device [B][max_blocks_per_seq] int32.  Entries outside
 *                 [0, num_blocks) make their 16 tokens count as absent.
 *   context_lens  device [B] int32, each clamped to
 *                 [0, min(max_context_len, 16*max_blocks_per_seq)]; rows with
 *                 length 0 get out = 0.
 *   max_context_len host upper bound of context_lens (sizes the grid).
 *   out           device [B][H_q][head_dim] of q_dtype, 16-byte aligned.
 *   workspace     device scratch of at least paged_decode_workspace_bytes()
 *                 for these B, H_q, max_context_len (NULL allowed if 0).
 * Work is split into partitions of the context; each partition keeps a running
 * max and sum (online softmax) and a second kernel merges partitions.  When a
 * context spans several partitions a small first kernel lists the live
 * (sequence, partition) items in the workspace, longest first, and the
 * partition kernel works through that list; the workspace also holds the
 * partials.  Calls that share one workspace must not overlap on the device.
 * Errors: INVALID_ARG, UNSUPPORTED (no kernel for dtype/head_dim/group: the
 * library refuses rather than fall back), STATE (host-only pool), DEVICE. */
int paged_decode(kv_pool_t* pool, const void* q, int32_t q_dtype, int32_t B, int32_t H_q,
                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t max_context_len, float scale,
                 void* out, void* workspace, size_t workspace_bytes, void* stream);

/* paged_decode without a workspace argument, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid hipMalloc.  Same arguments, kernels,
 * results (bit for bit) and errors as paged_decode, except that the work list
 * and partial results go to a fixed scratch array the library holds in each
 * device's memory until the process ends (PKV_NOALLOC_SCRATCH_BYTES per
 * device).  The call allocates nothing: no hipMalloc, hipFree or allocating
 * library routine.  It must be made with the pool's device current.
 *   Limit: paged_decode_workspace_bytes(pool, B, H_q, max_context_len) must
 *   not exceed PKV_NOALLOC_SCRATCH_BYTES (32 MiB: for example 64 sequences of
 *   up to 8192 tokens with 32 query heads of 128 dims need 8.5 MB); larger
 *   calls return PKV_ERR_OUT_OF_RANGE before anything is launched.
 *   Every call on one device shares that device's scratch, which keeps the
 *   last call's contents (the first kernel of a call resets what must start
 *   at zero): calls that overlap on one device race and must be ordered, for
 *   example on one stream.
 * Errors: those of paged_decode; OUT_OF_RANGE (scratch too small); INVALID_ARG
 * (the current device is not the pool's); DEVICE (the scratch's address could
 * not be looked up). */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int paged_decode_noalloc(kv_pool_t* pool, const void* q, int32_t q_dtype, int32_t B, int32_t H_q,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, float scale,
                         void* out, void* stream);

/* Workspace bytes paged_decode needs for these sizes with the pool's current
 * partition setting (0 if one partition covers max_context_len). */
size_t paged_decode_workspace_bytes(const kv_pool_t* pool, int32_t B, int32_t H_q,
                                    int32_t max_context_len);

/* Partition size (tokens) paged_decode uses: 0 = automatic, else a multiple
 * of 64 in [64, 1048576].  Affects only rounding order, never the result
 * beyond floating-point reassociation.  Errors: INVALID_ARG. */
int paged_decode_set_partition(kv_pool_t* pool, int32_t partition_tokens);

/* Partition size paged_decode would use for these sizes (resolves 0). */
int32_t paged_decode_partition_tokens(const kv_pool_t* pool, int32_t B, int32_t H_q,
                                      int32_t max_context_len);

/* ---------------------------------------------------------------------------
 * Swap ([cf1] §2.2: demand paging; blocks not in use may live in host memory
 * and come back when needed).  A whole sequence at a time.
 * ------------------------------------------------------------------------ */

/* Bytes a swapped copy of the sequence takes: ceil(len / block_size) blocks x
 * 2 x kv_heads x block_bytes.  Layout of the copy: for each logical block in
 * order, its K tiles of all KV heads, then its V tiles
 * ([kv_heads][block_size][head_dim] each, the pool's storage type).
 * Errors: INVALID_ARG, STATE. */
int kv_seq_swap_bytes(const kv_pool_t* pool, int32_t seq, size_t* bytes);

/* Copy the sequence's blocks to host_dst (host memory of at least
 * kv_seq_swap_bytes; pinned memory copies fastest) and release them as
 * kv_seq_free would (shared blocks stay with their other holders, cached
 * prefix blocks become evictable).  Owed copy-on-write copies run first.
 * The sequence keeps its id and length but cannot grow, fork, be registered
 * or appear in kv_block_tables until swapped in; kv_seq_free works either
 * way.  Synchronous: returns when host_dst holds the data (work queued
 * earlier on `stream` is waited for).  A metadata-only pool moves no data
 * (the buffer is ignored and may be NULL).  Errors: INVALID_ARG (buffer too small, NULL),
 * STATE (unknown or already swapped), DEVICE. */
int kv_seq_swap_out(kv_pool_t* pool, int32_t seq, void* host_dst, size_t bytes, void* stream);

/* Bring a swapped sequence back: ceil(len / block_size) fresh blocks, all or
 * nothing, in logical order (each the sequence's own; sharing and prefix-
 * cache keys it had are not restored), filled from host_src (the layout
 * kv_seq_swap_out wrote).  Synchronous.  Errors: INVALID_ARG, NO_BLOCKS
 * (nothing changed), STATE (not swapped out), DEVICE (the blocks are given
 * back and the sequence stays out). */
int kv_seq_swap_in(kv_pool_t* pool, int32_t seq, const void* host_src, size_t bytes, void* stream);

/* Multi-query attention through block tables: a chunk of prompt tokens per
 * sequence attending to the cached context and to itself (the prefill stage of
 * [mlqm] 三, and chunked prefill of [mlqm] 七, over the paged cache of [cf1]
 * §3.1).  Sequence s holds n_s = context_lens[s] tokens, the chunk's own K/V
 * already appended (kv_append), and brings q_len_s = q_start[s+1] - q_start[s]
 * query tokens: its last q_len_s positions.  Query token i of s, at position
 * p = n_s - q_len_s + i, attends to the positions
 *   causal != 0:  0 .. p         (a one-token chunk is the decode step)
 *   causal == 0:  0 .. n_s - 1   (every token sees the whole context)
 *   out[t][h] = sum_j softmax_j(scale * <q[t][h], K_s[j][g]>) * V_s[j][g],
 * t = q_start[s] + i, g = h / G.  FP8 pools: stored values are
 * decode(code) * scale of their KV head.
 *   q          device [total_q][H_q][head_dim] of q_dtype (BF16 or F16; the
 *              pool dtype, or either for an FP8 pool), 16-byte aligned.
 *   q_start    device [n_seqs + 1] int32, non-decreasing, q_start[0] = 0,
 *              q_start[n_seqs] = total_q, q_len_s <= n_s.
 *   block_tables, max_blocks_per_seq, context_lens: as for paged_decode;
 *              context_lens[s] is clamped to 16 * max_blocks_per_seq.
 *   max_q_len  host upper bound of q_len_s (sizes the grid).
 *   out        device [total_q][H_q][head_dim] of q_dtype, 16-byte aligned.
 * Supported: pool dtype F16, BF16 or FP8_E4M3, head_dim 64 or 128, any group
 * size.  Q.K^T and P.V run on the matrix cores.  Asynchronous on stream; no
 * workspace.  Device contents are not validated (q_start out of order or
 * q_len_s > n_s is undefined).  Errors: INVALID_ARG, UNSUPPORTED (F32 pool,
 * other head_dim, INT8 pool), STATE (host-only pool), DEVICE. */
int paged_prefill(kv_pool_t* pool, const void* q, int32_t q_dtype, int32_t n_seqs, int32_t H_q,
                  const int32_t* q_start, int32_t total_q, int32_t max_q_len,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, float scale, int32_t causal,
                  void* out, void* stream);

/* Synchronous copy of the whole K and V pools to host buffers of pool_bytes
 * each (inspection and tests).  Either pointer may be NULL.
 * Errors: STATE (host-only pool), DEVICE. */
int kv_pool_copy_to_host(const kv_pool_t* pool, void* k_dst, void* v_dst);

/* ---------------------------------------------------------------------------
 * Measurement
 * ------------------------------------------------------------------------ */

/* Per-kernel timing: while enabled, each call's kernels record a HIP event
 * pair on their launch stream as they start and end (hipExtLaunchKernel; the
 * pair spans a call's first kernel to its last).  pkv_profile_read waits for
 * the recorded events, fills up to cap entries of `out` with the launches
 * and summed device milliseconds per kernel name since the last read, and
 * resets the counters.  At most 65536 launches per kernel are kept between
 * reads; launches not timed (beyond that, or when an event is missing) are
 * counted in `dropped` and are not in total_ms, so the mean duration is
 * total_ms / (launches - dropped). */
typedef struct {
    char name[48];
    int64_t launches;
    int64_t dropped;
    double total_ms;
} pkv_kernel_stat_t;

int pkv_profile_enable(kv_pool_t* pool, int32_t on);
int pkv_profile_read(kv_pool_t* pool, pkv_kernel_stat_t* out, int32_t cap, int32_t* n);

/* Plain device-to-device copy of `bytes` (a multiple of 16, both pointers
 * 16-byte aligned) with 16-byte loads and stores: the reference kernel
 * against which HBM traffic counters are scaled.  Asynchronous on stream.
 * Errors: INVALID_ARG, DEVICE. */
int pkv_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Read-only probe over `bytes` of device memory at `src` (a multiple of 16,
 * 16-byte aligned): 16-byte loads, every wave instruction over 1 KiB, 512
 * workgroups each with four (address order) or eight (gathered) 4 KiB loads
 * in flight, with the nontemporal hint
 * when `nontemporal` is 1 and plain loads when 0.  It measures the HBM read
 * rate the decode kernels' loads can reach.
 *   order == NULL: the whole buffer in address order (n_order and
 *     chunk_bytes are ignored).
 *   order != NULL: a device array of n_order int32 chunk indices, owned by
 *     the caller; the buffer is cut into chunks of chunk_bytes (4096 times a
 *     power of two, dividing bytes) and the chunks are read in list order,
 *     as the paged kernels read tiles through a block table.  Entries outside
 *     [0, bytes / chunk_bytes) are skipped.
 * The launch XORs the XOR of all 32-bit words it read into *sink (a device
 * uint32, 4-byte aligned, owned by the caller; zero it first to read the
 * checksum).  Asynchronous on stream; nothing to read launches nothing (src
 * may then be NULL).
 * Errors: INVALID_ARG, DEVICE. */
int pkv_read_probe(const void* src, size_t bytes, int32_t nontemporal, const int32_t* order, int64_t n_order,
                   int32_t chunk_bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
