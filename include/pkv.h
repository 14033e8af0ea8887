/* pkv.h -- C ABI of libpkv: paged KV-cache decode attention on MI355X (gfx950).
 *
 * What the library computes (page title, section):
 *  - "无 vLLM 环境下的 Paged-KV 与连续批处理调度" §1.2: the KV cache is cut into
 *    fixed-size blocks (16 tokens by default) handed out from one global pool;
 *    a sequence of length l holds ceil(l / block_size) blocks and wastes less
 *    than one block. §2: the KV-bytes formula 2*L*H*d*s*B*bytes.
 *  - "vLLM核心概念：PagedAttention、Continuous Batching、KV Cache等原理" §3.1: a
 *    decode step attends the new token's query to every cached key/value;
 *    §3.2: a per-sequence block table maps logical blocks to any physical
 *    block, and sequences may share blocks, copied on the first divergent
 *    write (copy-on-write).
 *  - "连续批处理与KV缓存" §4.2: free blocks sit in one queue; allocation takes
 *    from the front and freeing returns to the back, O(1) per block;
 *    allocate fails when the queue is short, append reports "wait".
 *  - "轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" §三: symmetric
 *    INT8 with one scale per (block, KV head): scale = max|x|/127 (1.0 for an
 *    all-zero head), code = clamp(round(x/scale), -127, 127), x = code*scale.
 *
 * Conventions for every call:
 *  - Status: PKV_OK (0) or a negative pkv_status. Argument and shape errors
 *    are found on the host before anything is changed or launched; the
 *    message is available from pkv_last_error() (thread-local).
 *  - Allocator calls are host-only, all-or-nothing and O(1) per block.
 *  - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *    void*; NULL = the null stream). Their pointer arguments are device
 *    pointers on the pool's device unless marked "host".
 *  - A pool is not thread-safe: one host thread (or a lock) per pool.
 *  - Layout of the cache is private; pkv_read_blocks exports blocks in a
 *    canonical order for checks.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* bad argument or shape; nothing changed */
  PKV_ERR_OOM = -2,          /* allocate: not enough free blocks; nothing changed */
  PKV_ERR_NO_FREE_BLOCK = -3,/* append: pool empty, caller must wait or evict; nothing changed */
  PKV_ERR_UNKNOWN_SEQ = -4,  /* a sequence id that the pool does not hold */
  PKV_ERR_SEQ_EXISTS = -5,   /* allocate/fork onto an id already in use */
  PKV_ERR_DEVICE = -6,       /* a HIP call failed (message has the HIP error) */
  PKV_ERR_UNSUPPORTED = -7   /* valid but not implemented (e.g. head_dim 96) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_I8 = 3 } pkv_dtype;

typedef struct pkv_pool pkv_pool;

typedef struct {
  int32_t num_layers;    /* L >= 1: each layer has its own K and V slice of every block */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t block_size;    /* bs: 16, 32 or 64 tokens per block */
  int32_t num_blocks;    /* N >= 1 blocks in the pool (shared by all layers' slices) */
  pkv_dtype kv_dtype;    /* PKV_F16 or PKV_I8 */
  const int32_t* initial_free_order; /* host, optional: permutation of [0, N) giving the
                                        initial queue front to back; NULL = 0..N-1.
                                        Copied at create time. */
  void* device_arena;    /* optional caller-owned device memory of at least
                            pkv_pool_required_bytes(); the pool never frees it.
                            NULL = the library allocates (hipMalloc) and frees. */
  size_t arena_bytes;    /* size of device_arena */
  int32_t host_only;     /* 1 = allocator only, no device memory or HIP calls
                            (device entry points then return PKV_ERR_UNSUPPORTED) */
  const int32_t* layer_kv_dtype; /* host, optional: num_layers entries of PKV_F16 / PKV_I8,
                            the element type of each layer ("轻量级推理引擎实战" §3.2:
                            FP16 for the accuracy-sensitive first and last layers,
                            INT8 in between); NULL = kv_dtype for every layer.
                            Copied at create time. The automatic decode plan and
                            the workspace size follow kv_dtype for every layer. */
  int32_t seal_on_full;  /* 1 = lazy quantization of the INT8 layers ("轻量级推理引擎实战"
                            §三, third design note): a block stays in FP16 (staging
                            tiles, as much memory again as FP16 codes) while it is a
                            sequence's partly filled last block, and is quantized once,
                            all rows together, by the append that writes its last row
                            (see pkv_append_kv). Decode reads the FP16 rows of a
                            sequence's partly filled last block and INT8 elsewhere;
                            pkv_decode_step stages and seals the same way.
                            0 = quantize on append. */
} pkv_pool_config;

typedef struct {
  int64_t free_blocks;   /* blocks in the free queue */
  int64_t used_blocks;   /* blocks with reference count > 0 */
  int64_t shared_blocks; /* blocks with reference count > 1 */
  int64_t cow_copies;    /* copy-on-write copies made since creation */
  int64_t num_seqs;      /* live sequences */
  int64_t total_blocks;  /* N */
} pkv_stats;

/* Device bytes a pool with this configuration needs (codes for all layers,
 * K and V, plus for INT8 the fp32 scales and the int32 largest |code| of
 * each (block, head)), rounded up to 256 bytes. */
size_t pkv_pool_required_bytes(const pkv_pool_config* cfg);

/* Create a pool. Validates the configuration (including that
 * initial_free_order is a permutation). On success *out owns host state and,
 * unless host_only or device_arena is given, device memory on the current
 * HIP device. */
pkv_status pkv_pool_create(const pkv_pool_config* cfg, pkv_pool** out);

/* Destroy a pool and free what it owns. NULL is a no-op. The caller makes
 * sure no device work that uses the pool is still in flight. */
void pkv_pool_destroy(pkv_pool* pool);

/* ---------------- host allocator ("连续批处理与KV缓存" §4.2) ---------------- */

/* New sequence `seq` of n_tokens >= 0 tokens: ceil(n_tokens/bs) blocks from
 * the front of the free queue, in order. slots_out (host, n_tokens entries,
 * may be NULL) receives slot = block*bs + (t % bs) for t = 0..n_tokens-1.
 * PKV_ERR_SEQ_EXISTS if seq is live; PKV_ERR_OOM if the queue is short. */
pkv_status pkv_seq_allocate(pkv_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out);

/* Reserve n_new[i] >= 0 new token positions at the end of each seqs[i]
 * (distinct, live ids), processed in argument order and increasing
 * position. A position that starts a new logical block pops the queue
 * front; the first write into a partly filled block whose reference count
 * is above one pops a fresh block and copies the shared block's contents
 * (all layers, K and V, codes and scales) into it, enqueued on `stream`
 * (copy-on-write, "vLLM核心概念" §3.2). slots_out (host, sum(n_new) entries,
 * may be NULL) receives the slots in the same order. All-or-nothing:
 * PKV_ERR_NO_FREE_BLOCK if the queue cannot serve the whole call, or
 * PKV_ERR_DEVICE if a copy cannot be enqueued (the copies are enqueued
 * before anything changes). */
pkv_status pkv_seq_append_slots(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                                const int32_t* n_new, int64_t* slots_out, void* stream);

/* Make `child` share every block of `parent` (reference counts + 1) with the
 * same length. PKV_ERR_UNKNOWN_SEQ / PKV_ERR_SEQ_EXISTS as named. */
pkv_status pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child);

/* Drop `seq`: each of its blocks loses one reference, in table order, and a
 * block reaching zero goes to the BACK of the free queue. An unknown id is a
 * no-op returning PKV_OK (the page's pop(request_id, [])). */
pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq);

/* Host export of block tables: table_out (host) [n][max_blocks] int32, row i
 * = physical blocks of seqs[i] in logical order, padded with -1; lens_out
 * (host) [n] = lengths. PKV_ERR_INVALID_ARG if a sequence holds more than
 * max_blocks blocks. */
pkv_status pkv_seq_block_table(const pkv_pool* pool, const int64_t* seqs, int32_t n,
                               int32_t max_blocks, int32_t* table_out, int32_t* lens_out);

/* Length in tokens of a live sequence (host). */
pkv_status pkv_seq_length(const pkv_pool* pool, int64_t seq, int64_t* len_out);

/* A decode batch in the order that spreads its work evenly over the device:
 * seqs_out (host) [n] = seqs sorted by current length, longest first (equal
 * lengths keep their order; seqs_out may be seqs). Consecutive workgroups of
 * a decode launch go to different compute units, so when the whole grid is
 * resident at once (one partition per sequence) each compute unit then gets
 * sequences from every part of the length range instead of a random draw;
 * results do not depend on the order. PKV_ERR_UNKNOWN_SEQ for an unknown
 * id (seqs_out unchanged). */
pkv_status pkv_seq_order_longest_first(const pkv_pool* pool, const int64_t* seqs, int32_t n, int64_t* seqs_out);

pkv_status pkv_pool_stats(const pkv_pool* pool, pkv_stats* out);

/* Host copy of the free queue, front first (for checks). cap >= N. *n_out =
 * number of entries written. */
pkv_status pkv_pool_free_queue(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/* ------------------------------ device work ------------------------------ */

/* Store new tokens' K and V of one layer at their slots
 * ("轻量级推理引擎实战" §三 quantize_block, per (block, KV head)).
 * k, v: [n_tokens][num_kv_heads][head_dim] of in_dtype (F32, F16, BF16),
 * contiguous. slot_mapping: [n_tokens] int64 (device). Tokens that map to
 * one block must be adjacent in the token order with consecutive rows, the
 * first of them at row r meaning the block already holds rows [0, r) -- as
 * produced by pkv_seq_allocate / pkv_seq_append_slots. A slot outside
 * [0, num_blocks * block_size), e.g. -1 for a padding token, stores nothing;
 * it must not sit between two tokens of one block (that would split their
 * run). Slots are not otherwise checked on the device.
 *   F16 cache: each value is rounded to binary16, ties to even.
 *   I8 cache: for each touched (block, head, K|V) with new values X and r
 *   rows already present: if r == 0 the scale is max|X|/127 (1.0 when
 *   max|X| <= 1e-6) and X is encoded with it; else, with m_old =
 *   max|old code| * old scale, X is encoded with the old scale when
 *   max|X| <= m_old, otherwise the scale becomes max|X|/127 and the old
 *   codes are re-encoded from their dequantized values. Encoding divides by
 *   the scale (IEEE binary32) and rounds half to even.
 *   I8 layer of a seal_on_full pool: each value is rounded to binary16 and
 *   staged; when a block's last row is written, the block's bs rows (as
 *   binary16 values) are quantized together: scale max|x|/127 (1.0 when
 *   <= 1e-6), codes as above. */
pkv_status pkv_append_kv(pkv_pool* pool, int32_t layer, const void* k, const void* v,
                         pkv_dtype in_dtype, const int64_t* slot_mapping, int32_t n_tokens,
                         void* stream);

/* Every decode and prefill workspace starts with PKV_MERGE_COUNTER_BYTES of
 * int32 arrival counters (the merges done by the last workgroup to finish use
 * the first ones; a call leaves them at zero), whatever the call's sizes: so
 * one zero-filled workspace serves calls of any sizes in turn, none of
 * whose partials ever overwrite the counters another call reads. */
#define PKV_MERGE_COUNTER_BYTES 65536

/* Workspace bytes pkv_decode_attention needs for these sizes: the counter
 * prefix (one counter per (sequence, KV head) for a fused merge), then the
 * partition partials m, l and o/l in fp32. 0 when every sequence fits in
 * one partition. partition_tokens 0 = the automatic choice. */
size_t pkv_decode_workspace_bytes(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_tokens);

/* The partition size (tokens) pkv_decode_attention uses for these sizes when
 * partition_tokens is 0. */
int32_t pkv_decode_auto_partition(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len);

/* flags for pkv_decode_attention (0: automatic merge placement) */
#define PKV_DECODE_SEPARATE_MERGE 1 /* merge partitions in a second launch */
#define PKV_DECODE_FUSED_MERGE 2    /* merge partitions in the last workgroup of
                                       each (seq, KV head) to finish; at most
                                       PKV_MERGE_COUNTER_BYTES / 4 (seq, KV head)
                                       pairs, else PKV_ERR_UNSUPPORTED */
#define PKV_DECODE_VALU_CONTRACTION 4 /* pkv_decode_attention only, for comparing the two
                                       forms: the same launch with both contractions (q.k
                                       and p.v) as fp32 FMAs on the vector ALUs instead of
                                       the matrix cores. head_dim 128, 1 or 2 query heads
                                       per KV head, not seal_on_full layers; otherwise
                                       PKV_ERR_UNSUPPORTED. */

/* The launch plan pkv_decode_attention follows for these sizes and flags:
 * partition tokens, partitions per sequence, and 1 when partitions are
 * merged in the last workgroup of each (sequence, KV head), 0 when in a
 * second launch. Output pointers may be NULL. Host only, synchronous. */
pkv_status pkv_decode_plan(const pkv_pool* pool, int32_t num_seqs, int32_t max_context_len,
                           int32_t partition_tokens, int32_t flags, int32_t* partition_out,
                           int32_t* partitions_out, int32_t* fused_merge_out);

/* Single-token decode attention over one layer ("vLLM核心概念" §3.1):
 *   out[s][h][:] = sum_t softmax_t(softmax_scale * q[s][h] . K[s,t]) V[s,t]
 * over t < context_lens[s], where token t of sequence s lives in block
 * block_tables[s][t / bs], row t % bs, of KV head h / (num_q_heads /
 * num_kv_heads).
 *   q: [num_seqs][num_q_heads][head_dim] of q_dtype (F32, F16, BF16).
 *   block_tables: [num_seqs][max_blocks_per_seq] int32; entries past a
 *     sequence's last block are ignored. context_lens: [num_seqs] int32 with
 *     1 <= len <= max_blocks_per_seq*bs and len <= max_context_len (not
 *     checked on the device: the caller uploads what pkv_seq_block_table gave).
 *   out: [num_seqs][num_q_heads][head_dim] fp32.
 *   partition_tokens: context split (multiple of bs, at most 4096; 0 =
 *     automatic, which stays within 2048); each
 *     (sequence, KV head, partition) is one workgroup serving all query heads
 *     of the group; the partitions of a sequence are combined by a
 *     log-sum-exp merge, done by the last workgroup of each (sequence, KV
 *     head) to finish (PKV_DECODE_FUSED_MERGE) or by a second launch
 *     (PKV_DECODE_SEPARATE_MERGE). flags 0 picks the first when the whole
 *     grid fits on the device at once (and its counters fit the prefix), the
 *     second otherwise; both flags set is an error.
 *   workspace: at least pkv_decode_workspace_bytes(...) bytes (device). It
 *     must be zero-filled before its first use; every call leaves its
 *     counters at zero again, so one workspace serves any number of calls of
 *     any sizes on one stream (calls that overlap in time need separate
 *     workspaces).
 * Supported: head_dim 64/128, num_q_heads/num_kv_heads in {1,2,4}. */
pkv_status pkv_decode_attention(pkv_pool* pool, int32_t layer, const void* q, pkv_dtype q_dtype,
                                int32_t num_q_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, float softmax_scale,
                                int32_t partition_tokens, int32_t flags, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of one layer in a single launch: pkv_append_kv of each
 * sequence's new token, then pkv_decode_attention, with the same results
 * (cache codes and scales bit for bit, attention outputs as from
 * pkv_decode_attention over the updated cache). The new token of sequence s
 * is its last position, context_lens[s] - 1 (the context counts it, as in
 * "vLLM核心概念" §3.1: the new token's query is scored against the cache that
 * holds its own key); it is stored at block_tables[s][(len-1)/bs], row
 * (len-1) % bs.
 *   k_new, v_new: [num_seqs][num_kv_heads][head_dim] device rows in the same
 *     dtype as q (F32, F16 or BF16).
 *   Precondition: that block is not shared (pkv_seq_append_slots gave the
 *     position, copying a shared block first). A table entry outside the
 *     pool is not written.
 *   On an INT8 layer of a seal_on_full pool the new row is staged as
 *     binary16 and, when it fills its block, the block is sealed (codes,
 *     scales), both exactly as pkv_append_kv does; the decode then reads
 *     the block as the following pkv_decode_attention would.
 * All other arguments, the workspace and the flags are as for
 * pkv_decode_attention. */
pkv_status pkv_decode_step(pkv_pool* pool, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, pkv_dtype dtype, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           float softmax_scale, int32_t partition_tokens, int32_t flags, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* pkv_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launch, with the library's own scratch in place of a
 * caller's workspace; it calls no allocator. The scratch is one device array
 * of 16 MiB per GPU the library runs on (found and zero-filled when the
 * first pool is created on that device, held until the process ends); every
 * call leaves its arrival counters at zero again. All calls on one GPU share
 * it: calls that may overlap in time on one GPU (other streams, other
 * threads) race and must not be made.
 *   Arguments as pkv_decode_step, without workspace and workspace_bytes.
 *   PKV_ERR_INVALID_ARG (nothing launched) when these sizes need more than
 *   16 MiB of workspace (pkv_decode_workspace_bytes); PKV_ERR_DEVICE if the
 *   scratch of the pool's device was not set up. */
pkv_status pkv_decode_step_noalloc(pkv_pool* pool, int32_t layer, const void* q, const void* k_new,
                                   const void* v_new, pkv_dtype dtype, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                   float softmax_scale, int32_t partition_tokens, int32_t flags, float* out,
                                   void* stream);

/* Chunked prefill attention over one layer ("轻量级推理引擎实战" §一: prefill
 * processes a prompt's tokens in parallel, then decode adds one at a time).
 * For sequence s the last q_len = query_start[s+1] - query_start[s] of its
 * context_lens[s] cached tokens are queries (their K/V already appended with
 * pkv_append_kv); query i sits at position p = context_lens[s] - q_len + i
 * and attends causally to positions 0..p:
 *   out[qs+i][h] = sum_{t<=p} softmax_t(softmax_scale * q[qs+i][h] . K[s,t]) V[s,t]
 * with qs = query_start[s], K/V as in pkv_decode_attention. A whole-prompt
 * prefill is q_len = context_len; q_len = 1 is a decode step.
 *   q: [total][num_q_heads][head_dim] of q_dtype (F32, F16, BF16), rows packed
 *     sequence after sequence; out: same shape, fp32.
 *   query_start: [num_seqs+1] int32 (device), query_start[0] = 0, non-decreasing,
 *     1 <= q_len <= context_lens[s]; max_query_len >= every q_len (sizes the grid).
 *   block_tables, context_lens: as for pkv_decode_attention (device);
 *     max_context_len >= every context_lens[s] (plans the context split; a
 *     longer context is still computed in full, only less evenly split).
 *   piece_tokens: context split (0 = automatic, else a multiple of 64): each
 *     sequence's context is cut into pieces of this many tokens, each (group
 *     of query tiles, piece) one workgroup; the last workgroup of a tile
 *     group to finish merges its pieces' partial softmax sums per query
 *     (log-sum-exp, as the decode partitions). The automatic split cuts only
 *     when the query tiles alone would leave compute units idle.
 *     pkv_prefill_plan gives the split.
 *   workspace: device memory of at least the bytes pkv_prefill_plan gives
 *     (16-byte aligned): the counter prefix (PKV_MERGE_COUNTER_BYTES; one
 *     counter per (sequence, KV head, group of query tiles), at most
 *     PKV_MERGE_COUNTER_BYTES / 4, else PKV_ERR_UNSUPPORTED), then the
 *     partials; may be NULL when that is 0 (one piece). It must be
 *     zero-filled before its first use; every call leaves its counters at
 *     zero again, so one workspace serves any number of calls on one stream,
 *     decode calls included (calls that overlap in time need separate
 *     workspaces).
 * The K/V operands go through fp16 matrix-core products (INT8 codes convert
 * exactly), probabilities as fp16 hi + lo parts, fp32 accumulation.
 * Supported: head_dim 64/128, num_q_heads/num_kv_heads in {1,2,4}, F16 and
 * INT8 layers (not seal_on_full). */
pkv_status pkv_prefill_attention(pkv_pool* pool, int32_t layer, const void* q, pkv_dtype q_dtype,
                                 int32_t num_q_heads, const int32_t* query_start, int32_t max_query_len,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                 float softmax_scale, int32_t piece_tokens, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The launch plan pkv_prefill_attention follows for these sizes: the piece
 * size in tokens, the number of pieces per sequence, the workspace bytes it
 * needs (0 for one piece) and the wavefronts per workgroup (4; 8 when the
 * query tiles fill the larger workgroups and either the automatic split cuts
 * the context or four-wavefront workgroups would take two or more rounds of
 * the device: the larger workgroups share each staged step of the context
 * among twice the tiles). Output pointers may be NULL. Host only,
 * synchronous; the same argument checks as pkv_prefill_attention. */
pkv_status pkv_prefill_plan(const pkv_pool* pool, pkv_dtype q_dtype, int32_t num_q_heads, int32_t num_seqs,
                            int32_t max_query_len, int32_t max_context_len, int32_t piece_tokens,
                            int32_t* piece_tokens_out, int32_t* pieces_out, size_t* workspace_bytes_out,
                            int32_t* waves_out);

/* Synchronous host export of blocks of one layer in canonical order:
 * codes_out (host) [n][2 (K,V)][Hkv][bs][d] (int8 codes, or binary16 bits as
 * uint16 for an F16 layer); scales_out (host, may be NULL; written for an
 * INT8 layer only) [n][2][Hkv] fp32. */
pkv_status pkv_read_blocks(const pkv_pool* pool, int32_t layer, const int32_t* blocks, int32_t n,
                           void* codes_out, float* scales_out);

/* ------------------- continuous-batching step scheduler -------------------
 * The per-step micro-decisions of "无 vLLM 环境下的 Paged-KV 与连续批处理调度"
 * §3.1 (admit while page blocks remain, step the mixed batch, evict on EOS
 * (event kind 2) or on the length limit (kind 3) and reclaim the blocks at
 * once), in the order "vLLM核心概念" §3.3 gives (retire finished requests and
 * free their blocks, keep the others, admit from the waiting queue while free
 * blocks allow, decode every active request), over the pool's allocator
 * ("连续批处理与KV缓存" §4.2: append_block reports "wait" when the queue is
 * empty; §4.4: on running out of memory, pause new requests until blocks come
 * back). Requests are admitted first come, first served. Host only: the
 * scheduler plans a step; the caller writes the admitted prompts' K/V
 * (pkv_append_kv at prefill_slots) and runs the decode (pkv_decode_step over
 * the batch) on the stream given to pkv_sched_step, which also carries any
 * copy-on-write copies. Request ids are pool sequence ids: the caller keeps
 * its own sequences (shared prefixes) on other ids. Not thread-safe. */
typedef struct pkv_sched pkv_sched;

typedef struct {
  int32_t max_batch;      /* most requests decoded per step (>= 1; "--max-num-seqs") */
  int32_t max_model_len;  /* most tokens a request may hold, prompt included (>= 2);
                             a request that reaches it ends with PKV_EV_MAX_LENGTH */
  int32_t reserve_blocks; /* admission needs this many free blocks beyond those of the
                             prompt (>= 0; 1 leaves room for the first decode token) */
  int32_t batch_order;    /* order of a plan's decode rows: PKV_BATCH_ADMISSION or
                             PKV_BATCH_LONGEST_FIRST (as pkv_seq_order_longest_first,
                             equal lengths in admission order); the step's decisions and
                             allocations are the same either way */
} pkv_sched_config;

#define PKV_BATCH_ADMISSION 0
#define PKV_BATCH_LONGEST_FIRST 1

/* event kinds (2 and 3 as in "无 vLLM 环境下的 Paged-KV 与连续批处理调度" §3.1) */
#define PKV_EV_ADMIT 1      /* admitted: its prompt is in this step's prefill list */
#define PKV_EV_EOS 2        /* finished: the caller reported end of sequence */
#define PKV_EV_MAX_LENGTH 3 /* finished: max_new_tokens generated or max_model_len reached */
#define PKV_EV_PREEMPT 4    /* every running request was waiting for a block: the most
                               recently admitted one gave its blocks back and returned to
                               the front of the queue, to be written again in full */
#define PKV_EV_WAIT 5       /* no free block for its next token: not decoded this step */

typedef struct {
  int64_t request;
  int32_t kind;
  int32_t pad_;
} pkv_event;

/* A step's plan. The arrays are host memory owned by the scheduler, valid
 * until the next pkv_sched_step or pkv_sched_destroy. */
typedef struct {
  int32_t num_seqs;             /* requests decoded this step, in the configured batch order */
  int32_t max_blocks;           /* width of block_tables rows: ceil(max_model_len / bs) */
  int32_t max_context_len;      /* max of context_lens (0 when num_seqs is 0) */
  int32_t num_prefill;          /* requests admitted this step */
  int32_t prefill_total;        /* sum of prefill_tokens */
  int32_t num_events;
  const int64_t* seqs;          /* [num_seqs] request ids */
  const int64_t* slots;         /* [num_seqs] slot of each one's new token (position len - 1) */
  const int32_t* block_tables;  /* [num_seqs][max_blocks], padded with -1 */
  const int32_t* context_lens;  /* [num_seqs], counting the new token */
  const int64_t* prefill_seqs;  /* [num_prefill] */
  const int32_t* prefill_first; /* [num_prefill] first position to write (the shared
                                   prefix length, 0 without one) */
  const int32_t* prefill_tokens;/* [num_prefill] tokens to write from there */
  const int64_t* prefill_slots; /* [prefill_total] their slots, request after request */
  const pkv_event* events;      /* [num_events] in the order they happened */
} pkv_step_plan;

typedef struct {
  int64_t waiting, running;     /* requests in the queue / admitted and not finished */
  int64_t admitted, finished_eos, finished_max_length, preempted;  /* totals */
  int64_t generated;            /* tokens decoded so far */
  int64_t used_blocks, total_blocks;  /* the pool's, as in "12000 used / 15000 total" */
  int32_t paused;               /* admissions paused: a decode token found no free block */
  int32_t pad_;
} pkv_sched_stats;

pkv_status pkv_sched_create(pkv_pool* pool, const pkv_sched_config* cfg, pkv_sched** out);

/* Destroy the scheduler; the blocks of its requests go back to the pool. */
void pkv_sched_destroy(pkv_sched* sched);

/* Queue a request: prompt_len >= 1 prompt tokens, then at most max_new_tokens
 * >= 1 decoded ones. prefix_seq >= 0 names a live pool sequence of length
 * p <= prompt_len whose tokens are the prompt's first p (shared blocks,
 * forked at admission; the caller keeps it unchanged while requests may
 * use it); -1 = none. PKV_ERR_SEQ_EXISTS if the id is queued, running or a
 * pool sequence; PKV_ERR_INVALID_ARG if prompt_len >= max_model_len or if
 * min(prompt_len + max_new_tokens, max_model_len) tokens need more blocks
 * than the pool has (such a request could never finish). */
pkv_status pkv_sched_submit(pkv_sched* sched, int64_t request, int32_t prompt_len,
                            int32_t max_new_tokens, int64_t prefix_seq);

/* Plan one step. eos[0..n_eos) are requests of the previous step's batch
 * whose decoded token ended the sequence (the caller's sampling).
 *  1. Retire, in admission order: a request in eos (PKV_EV_EOS), or one that
 *     has decoded max_new_tokens tokens or holds max_model_len tokens
 *     (PKV_EV_MAX_LENGTH), frees its blocks; freed blocks lift a pause.
 *  2. Admit, unless paused, first come first served: while the batch has
 *     room and the queue front's prompt needs at most free - reserve_blocks
 *     new blocks, allocate it (or fork its prefix and reserve the rest) and
 *     list it for prefill (PKV_EV_ADMIT). The first request that does not fit
 *     stops admission.
 *  3. Decode: in admission order, each running request takes one new token
 *     position; one that needs a block the queue cannot give waits
 *     (PKV_EV_WAIT) and pauses admissions. If every running request waits,
 *     the most recently admitted one is preempted (PKV_EV_PREEMPT) and the
 *     others try again.
 * The requests that got a position form the batch; each counts one decoded
 * token. Argument errors (an eos id not in the previous batch) change nothing. */
pkv_status pkv_sched_step(pkv_sched* sched, const int64_t* eos, int32_t n_eos, pkv_step_plan* plan,
                          void* stream);

pkv_status pkv_sched_get_stats(const pkv_sched* sched, pkv_sched_stats* out);

/* Synchronous host export of the FP16 staging tiles of a seal-on-full INT8
 * layer (pool created with seal_on_full): f16_out (host) [n][2 (K,V)][Hkv]
 * [bs][d] binary16 bits in canonical order. Rows a block holds while it is
 * partly filled are meaningful; after it is sealed they are stale.
 * PKV_ERR_UNSUPPORTED for a layer without staging tiles. */
pkv_status pkv_read_tail_blocks(const pkv_pool* pool, int32_t layer, const int32_t* blocks, int32_t n,
                                uint16_t* f16_out);

/* Measurement helper: a plain streaming read of `bytes` (a positive multiple
 * of 16) of device memory at `buf` (16-byte aligned) with `workgroups` (1 ..
 * 65535) workgroups of 256 threads, each thread taking 16-byte pieces
 * workgroups*256 apart with four loads in flight; every thread stores one
 * word to sink (device, workgroups * 256 uint32), so the reads cannot be
 * dropped. It moves the same kind of 4 KB runs as the decode kernels and
 * nothing else: its time for the bytes a decode launch reads is the
 * practical floor of that launch on this GPU ("离开 N 卡后的真实世界" §3.1:
 * decode is bound by memory bandwidth). Asynchronous on `stream`. */
pkv_status pkv_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/* The KV-bytes formula 2*L*H*d*s*B*bytes ("无 vLLM 环境下的 Paged-KV" §2). */
uint64_t pkv_kv_bytes(uint64_t layers, uint64_t heads, uint64_t head_dim, uint64_t tokens,
                      uint64_t seqs, uint64_t bytes);

/* Message for the last non-OK status on this thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
