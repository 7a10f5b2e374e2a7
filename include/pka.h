/*
 * pka.h - paged KV attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operations follow three pages on paged attention:
 *   [MLR]  MiniLLM Runtime: "Core class relationships" (logical token ->
 *          logical block + offset -> block table -> physical KV address) and
 *          "CUDA PagedAttention scope" (one decode query; QK, softmax and
 *          weighted-value accumulation read straight from paged storage).
 *   [ME]   mini_engine: "Custom CUDA kernels" (KV-cache write with padded
 *          slots skipped; paged prefill with online softmax over ragged
 *          chunks that attend to earlier cached chunks; paged decode v1, one
 *          workgroup per (sequence, KV head) with the query heads of a GQA
 *          group sharing every K/V load; decode v2, split-K over 256-token
 *          partitions merged by a reduce that uses each partition's saved max
 *          and exp-sum; a dispatcher choosing between them; split attention
 *          writing decode and prefill rows into one output tensor).
 *   [MS]   miniserve: "Engine" flowchart (new K/V rows go to
 *          slot = block_id * block_size + offset before attention; prefill
 *          chunks use a bottom-right causal mask).
 *
 * Data layout (all tensors contiguous, row-major, in device memory that the
 * caller owns; the library never allocates, frees or synchronises):
 *   k_cache, v_cache   [num_blocks][block_size][num_kv_heads][head_dim]
 *                      element type fp16 or bf16; slot s is row s of the
 *                      flattened [num_blocks * block_size][num_kv_heads][head_dim]
 *                      view, i.e. block s / block_size, offset s % block_size.
 *   block_tables       int32 [num_seqs][max_blocks_per_seq]; entry [s][b] is
 *                      the physical block holding logical tokens
 *                      b*block_size .. b*block_size+block_size-1 of sequence s.
 *                      Entries at or past ceil(context_len / block_size) are
 *                      never read.
 *   context_lens       int32 [num_seqs]: tokens sequence s attends to,
 *                      including the current decode token or the whole
 *                      current prefill chunk (their K/V must already be in the
 *                      cache: write first, then attend).
 *   q, out (decode)    [num_seqs][num_q_heads][head_dim], element type of the cache.
 *   q, out (prefill)   [num_q_tokens][num_q_heads][head_dim]; the rows of
 *                      sequence s are query_start_loc[s] .. query_start_loc[s+1]-1.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * scale multiplies q.k before the (natural-base) softmax.
 * Arithmetic: fp32 accumulation; outputs rounded to nearest even.
 *
 * Supported shapes (mini_engine, "Roadmap": generalising beyond one head
 * shape): block_size 8, 16 or 32; head_dim 64, 128 or 256;
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}; fp16 or bf16.  Anything else
 * returns PKA_ERR_UNSUPPORTED.
 *
 * Errors: every host-checkable problem (null pointer, bad size, unsupported
 * shape, pointer not 16-byte aligned, workspace too small) returns a non-zero
 * status before anything is launched.  A failed launch returns PKA_ERR_HIP.
 * Device-data preconditions are documented and NOT checked:
 * 0 <= block id < num_blocks for every entry that is read,
 * 1 <= context_len <= max_blocks_per_seq * block_size,
 * context_len <= max_context_len, query length <= context_len, and
 * non-negative slots are distinct.  num_seqs == 0 (or num_tokens == 0) is a
 * no-op returning PKA_OK.
 *
 * Streams: every call enqueues its kernels on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without waiting.
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKA_F16 = 0, PKA_BF16 = 1 } pka_dtype;

typedef enum {
  PKA_OK = 0,
  PKA_ERR_NULL = 1,        /* a required pointer is NULL */
  PKA_ERR_SHAPE = 2,       /* a size is negative or sizes disagree */
  PKA_ERR_UNSUPPORTED = 3, /* shape or dtype not built into the library */
  PKA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  PKA_ERR_WORKSPACE = 5,   /* split-K workspace missing or too small */
  PKA_ERR_HIP = 6,         /* the HIP runtime reported an error */
  PKA_ERR_SCRATCH = 7      /* pka_paged_attn_decode_noalloc: more than its scratch holds */
} pka_status;

/* Shape of one layer's paged KV pool (k_cache and v_cache alike). */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pka_dtype */
} pka_cache_desc;

/* Split-K partition length in tokens ([ME] decode v2). */
#define PKA_PARTITION_SIZE 256

/* Human-readable name of a status code (static string). */
const char* pka_status_str(int32_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pka_version(void);

/*
 * KV-cache write ([ME] KV-cache write; [MS] index_copy_ into the pool).
 * For every i < num_tokens with slot_mapping[i] >= 0, copies key[i] into
 * k_cache slot slot_mapping[i] and value[i] into v_cache at the same slot;
 * rows with a negative slot are padding and are skipped.  A pure byte copy:
 * the result is bit-exact and no other byte of the pool changes.
 *   key, value    [num_tokens][num_kv_heads][head_dim], cache element type
 *   slot_mapping  int64 [num_tokens]
 */
int32_t pka_kv_cache_write(const void* key, const void* value, const int64_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           pka_cache_desc cache, void* stream);

/*
 * Rotary table for pka_fused_rope_kv_write (mini_engine: "Roadmap", fused
 * RoPE folded into the QKV split / KV-cache write).  Fills
 *   table[p][i] = (cos a, sin a), a = p * theta^(-2 i / head_dim),
 * for p < max_position, i < head_dim / 2, as fp32 pairs computed in double
 * precision on the device.  table: device memory of
 * pka_rope_table_bytes(max_position, head_dim) bytes, 16-byte aligned, owned
 * by the caller; fill it once per (theta, head_dim).  theta must be > 1 and
 * head_dim a multiple of 16 (PKA_ERR_SHAPE otherwise).
 */
int32_t pka_rope_table(float* table, int32_t max_position, int32_t head_dim, double theta, void* stream);
size_t pka_rope_table_bytes(int32_t max_position, int32_t head_dim);

/*
 * Rotary embedding fused into the KV-cache write (mini_engine: "Roadmap";
 * [MS] fused qkv projection, RoPE, then index_copy_ into the pool).  Reads
 * each token's fused projection row
 *   qkv[t] = [q heads (num_q_heads x head_dim) | k heads | v heads
 *             (num_kv_heads x head_dim each)], element stride qkv_row_stride,
 * rotates q and k by positions[t] with the rotate-half pairing (element
 * i < D/2 pairs with i + D/2; the pair turns by the table's angle), writes the
 * rotated q to q_out [num_tokens][num_q_heads][head_dim] (contiguous), and for
 * slot_mapping[t] >= 0 stores the rotated k and the unchanged v bits at that
 * slot of k_cache / v_cache.  Negative slots are padding: their q is still
 * rotated, nothing is written to the pool.  Rotation in fp32, one rounding
 * (to nearest even) to the cache type.
 *   positions     int64 [num_tokens], 0 <= positions[t] < max_position
 *                 (device precondition, unchecked)
 *   rope_table    as filled by pka_rope_table for this head_dim
 * PKA_ERR_SHAPE if qkv_row_stride is below the row length or breaks 16-byte
 * alignment of the rows.
 */
int32_t pka_fused_rope_kv_write(const void* qkv, int64_t qkv_row_stride, const int64_t* positions,
                                const int64_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                                const float* rope_table, int32_t max_position, void* q_out, void* k_cache,
                                void* v_cache, pka_cache_desc cache, void* stream);

/*
 * Paged decode, single pass ([MLR] CUDA PagedAttention; [ME] decode v1).
 * One query row per sequence; out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 * over the first context_lens[s] tokens of sequence s, K_s and V_s read in
 * place through block_tables.  No workspace.
 */
int32_t pka_paged_attn_decode_v1(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 float scale, void* out, pka_cache_desc cache, void* stream);

/*
 * Split-K decode, partition pass ([ME] decode v2).  Partition p of sequence s
 * covers logical tokens [p * partition_size, min((p + 1) * partition_size,
 * context_lens[s])).  For each (s, h, p) with p < ceil(context_lens[s] /
 * partition_size) it writes
 *   max_logits[(s * num_q_heads + h) * max_num_partitions + p] = m_p
 *       = max over the partition of scale * q . k_t
 *   exp_sums[...same index...] = l_p = sum over the partition of exp(scale * q . k_t - m_p)
 *   tmp_out[((s * num_q_heads + h) * max_num_partitions + p) * head_dim + d]
 *       = sum exp(scale * q . k_t - m_p) v_t[d] / l_p            (fp32)
 * Slots of partitions past a sequence's end are left untouched.
 * partition_size must be PKA_PARTITION_SIZE;
 * max_num_partitions >= ceil(max context_len / partition_size).
 */
int32_t pka_paged_attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                     float scale, int32_t partition_size, int32_t max_num_partitions,
                                     float* tmp_out, float* max_logits, float* exp_sums,
                                     pka_cache_desc cache, void* stream);

/*
 * Split-K reduce ([ME] decode v2, "small reduce kernel").  For each (s, h),
 * over the P = ceil(context_lens[s] / partition_size) partitions:
 *   M = max_p m_p,  w_p = l_p * exp(m_p - M),
 *   out[s][h][d] = sum_p w_p * tmp_out[..p..][d] / sum_p w_p,
 * rounded to `dtype`.  Buffers as written by pka_paged_attn_decode_splitk.
 */
int32_t pka_paged_attn_splitk_reduce(const float* tmp_out, const float* max_logits,
                                     const float* exp_sums, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                     int32_t partition_size, int32_t max_num_partitions,
                                     void* out, int32_t dtype, void* stream);

/*
 * Bytes of workspace the dispatched decode needs when it takes the split-K
 * path: a 64 KiB header of arrival counters, then tmp_out, max_logits and
 * exp_sums for max_num_partitions = ceil(max_context_len / PKA_PARTITION_SIZE),
 * each region 256-byte aligned.  Pure host function.
 */
size_t pka_splitk_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len);

/*
 * Decode dispatcher ([ME] "Custom CUDA kernels": v2 is chosen when the batch
 * alone would leave the GPU idle, i.e. few sequences or long contexts).
 * Returns 1 (single pass) or 2 (split-K) for num_seqs * num_kv_heads
 * workgroups on num_cus compute units with contexts up to max_context_len.
 * Pure host function.
 */
int32_t pka_decode_choose_variant(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                  int32_t num_cus);

/*
 * Paged decode with dispatch: runs v1, or split-K with its partition merge,
 * as pka_decode_choose_variant picks for this device.  max_context_len is a
 * host upper bound on context_lens.  The split-K path carves its buffers from
 * `workspace` (device memory, at least pka_splitk_workspace_bytes bytes,
 * 256-byte aligned); the v1 path ignores it.  PKA_ERR_WORKSPACE if split-K is
 * chosen and the workspace is missing or too small.
 *
 * Split-K runs as ONE launch when num_seqs * num_kv_heads <= 16384: each
 * (sequence, KV head) has an arrival counter in the workspace's first 64 KiB;
 * a partition workgroup stores its state (same format as
 * pka_paged_attn_decode_splitk), counts itself, and the one that arrives last
 * merges the sequence's partitions into `out` (the rule of
 * pka_paged_attn_splitk_reduce).  Larger batches run the partition pass and
 * the reduce as two launches.
 * Workspace contract: the first 64 KiB must be zero before the first call
 * that uses the workspace (e.g. hipMemset once after allocating it); every
 * call leaves them zero again, also under HIP-graph replay, so a workspace is
 * reused without clearing.  The rest is scratch.  Calls that share a
 * workspace must not run concurrently.
 */
int32_t pka_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, void* out, pka_cache_desc cache,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step with the KV-cache write folded in ([MS] "Engine" flowchart:
 * the new token's K/V is written at slot = block_id * block_size + offset,
 * then attention reads it; [ME] decode v1/v2).  For every sequence s with
 * t = context_lens[s] - 1 >= 0:
 *   the row key[s] / value[s] ([num_seqs][num_kv_heads][head_dim], the
 *   cache dtype) is written, bit for bit, to position t of s, i.e. slot
 *   block_tables[s][t / block_size] * block_size + t % block_size of
 *   k_cache / v_cache,
 *   and out[s] is the decode of pka_paged_attn_decode over positions
 *   0 .. t, position t taking those rows.
 * The result equals pka_kv_cache_write with slot_mapping[s] = that slot
 * followed by pka_paged_attn_decode, in one launch (two with split-K); the
 * kernels take the new rows from registers and never read the slot back, so
 * its previous contents do not matter.  Same dispatch, workspace and errors
 * as pka_paged_attn_decode; key, value: device pointers, 16-byte aligned
 * (PKA_ERR_NULL / PKA_ERR_ALIGN).  Preconditions (unchecked): position t's
 * block belongs to s alone (not a shared prefix block), and no other
 * sequence of the batch has that slot.
 */
int32_t pka_paged_attn_decode_append(const void* q, const void* key, const void* value,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                     void* out, pka_cache_desc cache, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Allocation-free paged decode, for callers that cannot allocate device
 * memory (code under HIP-graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same operation, arguments, dispatch and errors as
 * pka_paged_attn_decode without the workspace: the split-K path uses an array
 * inside the library instead, PKA_NOALLOC_SCRATCH_BYTES (32 MiB) per device,
 * held by each device the library runs on until the process ends.  Returns
 * PKA_ERR_SCRATCH, before launching anything, when the split-K path is chosen
 * and pka_splitk_workspace_bytes(...) exceeds it (at head size 128 it holds
 * about 64,000 (sequence, query head, partition) rows, e.g. 4 sequences of
 * 256,000 tokens with 16 query heads).  Allocates nothing (no hipMalloc, no allocating library
 * call); the first call on a device looks up the array's device address.  All
 * calls on one device share the array: calls that overlap in time on one
 * device (several streams or threads) race and must be serialised by the
 * caller.  The array's arrival counters start at zero and every call leaves
 * them at zero.
 */
#define PKA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int32_t pka_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, float scale, void* out, pka_cache_desc cache,
                                      void* stream);

/*
 * Paged prefill ([ME] paged prefill attention; [MS] bottom-right causal
 * mask).  Ragged chunks packed in q: sequence s contributes rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 (q_len_s rows) that occupy
 * its last q_len_s context positions; with c_s = context_lens[s] - q_len_s,
 * row i (0-based within the chunk) attends to logical tokens 0 .. c_s + i.
 * K and V of the chunk itself must already be in the cache.
 * max_query_len and max_context_len are host upper bounds on q_len_s and
 * context_lens[s].  MFMA (bf16/fp16 inputs, fp32 accumulation); the softmax
 * weights are rounded to the input type before the PV product.
 *   query_start_loc  int32 [num_seqs + 1], query_start_loc[0] = 0,
 *                    query_start_loc[num_seqs] = num_q_tokens
 * When the batch has too few query tiles (128 q-rows of one chunk and one KV
 * head) to fill the GPU, each tile's key range is split over several
 * workgroups (splits of at least 256 keys, enough of them for about four
 * work items per compute unit); their partial states go to `workspace`
 * (device memory, at least
 * pka_prefill_workspace_bytes(...) bytes, 256-byte aligned; contents need no
 * initialisation and are scratch after the call).  When that size is 0 the
 * workspace may be NULL.  PKA_ERR_WORKSPACE if it is needed and too small.
 * scale must be positive and finite (PKA_ERR_UNSUPPORTED otherwise): the
 * kernel tracks each row's running maximum of the unscaled scores.
 */
int32_t pka_paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* query_start_loc, int32_t num_seqs,
                               int32_t num_q_tokens, int32_t max_query_len, int32_t max_context_len,
                               int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, void* out,
                               pka_cache_desc cache, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes pka_paged_attn_prefill needs for these sizes (0 when no
 * query tile can see more keys than one split holds).  Host function; the
 * split choice uses the compute-unit count of the current device (256 when
 * there is none), so size the workspace with the device the launch uses. */
size_t pka_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len);

/* Keys per split that pka_paged_attn_prefill uses for these sizes on the
 * current device (a multiple of 64; a query tile whose visible keys number
 * more than this is split), or -1 for invalid sizes.  Host function, for
 * callers and tests that want to know where the split boundaries fall. */
int32_t pka_prefill_split_keys(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len);

/* Number of compute units of the current device (cached per device after the
 * first call), or a negative value if the HIP runtime fails. */
int32_t pka_device_cu_count(void);

/*
 * Host-side paged block manager (MiniLLM Runtime: "Features" - block
 * allocation, release, reuse, reference counting, prefix-cache lookup with
 * shared ownership; mini_engine "Features": a block gets its hash the moment
 * it is full; miniserve "Architecture": KVCacheManager with chained hashes,
 * refcounts and an LRU free list, and its request-state diagram).  Pure host
 * code, no GPU calls; one manager per KV pool, not thread-safe.
 *
 * Pages are reference counted; free pages form an LRU list (new pages from
 * its front, pages reaching refcount 0 to its tail in block-table order).  A
 * page that fills is registered under the chained hash of its token prefix
 * and keeps that registration while free, until it is taken for new
 * content.  Hits are confirmed against the stored tokens and parent hash.
 *
 * Request flow: add_request(prompt) -> admit(first chunk) -> [allocate(n) ->
 * run the kernels on slot_mapping / block_table -> commit(n) ->
 * append_token(sampled)]* -> free_request.  Return conventions: status codes
 * (pka_status) for commands; counts or 1/0 (done / no room) for queries, with
 * a negated pka_status on error.
 */
typedef struct pka_block_manager pka_block_manager;
pka_block_manager* pka_bm_create(int32_t num_blocks, int32_t block_size); /* NULL on bad sizes / no memory */
void pka_bm_destroy(pka_block_manager* m);
int32_t pka_bm_num_free(const pka_block_manager* m);
int32_t pka_bm_refcount(const pka_block_manager* m, int32_t block);
/* Register a request and its prompt token ids (copied). */
int32_t pka_bm_add_request(pka_block_manager* m, int64_t req_id, const int32_t* tokens, int32_t num_tokens);
int32_t pka_bm_append_token(pka_block_manager* m, int64_t req_id, int32_t token);
/* Pages of the longest cached whole-block prefix, always leaving >= 1 token to
 * compute; writes up to max_blocks ids, returns their number. */
int32_t pka_bm_find_cached_prefix(const pka_block_manager* m, int64_t req_id, int32_t* blocks, int32_t max_blocks);
/* Prefix lookup + room for first_chunk more tokens, all or nothing: 1 and
 * *num_cached_tokens set, or 0 when the pool cannot hold it (no change). */
int32_t pka_bm_admit(pka_block_manager* m, int64_t req_id, int32_t first_chunk, int32_t* num_cached_tokens);
/* Room for num_new_tokens past the computed ones: 1, or 0 (no change). */
int32_t pka_bm_allocate(pka_block_manager* m, int64_t req_id, int32_t num_new_tokens);
/* num_tokens more tokens now have K/V in the pool; filled pages get registered. */
int32_t pka_bm_commit(pka_block_manager* m, int64_t req_id, int32_t num_tokens);
/* Drop the request's pages (refcount - 1); keep_request != 0 keeps its tokens
 * with nothing computed (preemption), else forgets it. */
int32_t pka_bm_free_request(pka_block_manager* m, int64_t req_id, int32_t keep_request);
/* The request's block table (page ids in logical order); returns its length. */
int32_t pka_bm_block_table(const pka_block_manager* m, int64_t req_id, int32_t* out, int32_t max_blocks);
/* slot = page * block_size + offset for logical positions start .. start+n-1. */
int32_t pka_bm_slot_mapping(const pka_block_manager* m, int64_t req_id, int32_t start, int32_t num_tokens,
                            int64_t* out);
int32_t pka_bm_num_computed(const pka_block_manager* m, int64_t req_id);
/* One decode step for num_reqs running requests in one call: append
 * tokens[i] to request req_ids[i], make room for it, write its slot to
 * slots[i] and count it computed (ok[i] = 1), or leave the request unchanged
 * apart from the appended token when the pool is full (ok[i] = 0, slots[i] =
 * -1, a padded row for the KV write).  Returns the number of rows placed. */
int32_t pka_bm_decode_step(pka_block_manager* m, int32_t num_reqs, const int64_t* req_ids, const int32_t* tokens,
                           int64_t* slots, int32_t* ok);

#ifdef __cplusplus
}
#endif

#endif /* PKA_H */
