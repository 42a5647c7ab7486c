/*
 * pkv.h -- attention over a paged KV cache on AMD MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Plain pointers and sizes only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer (memory from hipMalloc or a
 *   framework allocator on the current device) and must be 16-byte aligned.
 *   The caller owns every buffer; the library allocates nothing and keeps
 *   no per-call state.
 * - Element types: K/V/q/out are bfloat16 stored as 16-bit words; every
 *   index array is int32.  All tensors are dense and row-major in the shape
 *   given.
 * - KV pool layout (miniVLLM "Engine Architecture", allocate_kv_cache: one
 *   tensor per layer and per K/V of shape [num_blocks, block_size,
 *   num_kv_heads, head_dim]): k_cache and v_cache are each
 *   [num_pages, page_size, num_kv_heads, head_dim].  The "slot" of a token is
 *   its row in the flat [num_pages * page_size, num_kv_heads, head_dim] view:
 *   slot = page * page_size + offset_in_page.
 * - Page table (mini-sglang "Engine Class", Key Attributes: page_table;
 *   miniVLLM prepare_prefill / prepare_decode: block_tables): int32
 *   [num_seqs, page_table_stride]; entry [r, j] is the physical page holding
 *   logical positions j*page_size .. (j+1)*page_size-1 of request r.  Entries
 *   past a request's last page are never read.
 * - GQA (miniVLLM "LLMEngine", Config parameters: num_heads, num_kv_heads):
 *   query head h reads K/V head h / (num_q_heads / num_kv_heads).
 * - stream: a hipStream_t (NULL = the legacy default stream).  Work is
 *   enqueued asynchronously; no entry point synchronises the host.
 * - Errors: a non-zero status is returned BEFORE anything is enqueued when
 *   an argument the host can check is wrong; PKV_EHIP reports a launch
 *   failure.  Device-resident values (page ids, slots, lengths) are not
 *   checked on the host: out-of-range values are clamped or skipped inside
 *   the kernels; where rows are fetched by range-checked buffer loads, a
 *   page id outside the pool reads zeros or (ids of 2^24 and more, whose
 *   offset wraps) other rows of the same pool.  No access leaves the buffers
 *   described here, and the affected outputs are unspecified.
 * - Thread safety: calls may be made from any host thread; calls that share
 *   an output or workspace buffer must be ordered by the caller.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL 1        /* null pointer, bad size, misaligned pointer,  */
                            /* inconsistent shapes                          */
#define PKV_EUNSUPPORTED 2  /* legal but not built: head_dim, page_size or  */
                            /* query-heads-per-KV-head outside the kernels  */
#define PKV_ENOSPACE 3      /* workspace smaller than required              */
#define PKV_EHIP 4          /* the HIP runtime failed to launch a kernel    */

/* Human-readable text for a status code (static storage; never NULL). */
const char* pkv_strerror(int status);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

/*
 * pkv_store_kv -- scatter this step's new K/V rows into the pool.
 *
 * For t in [0, num_tokens): row out_loc[t] of the flat K pool receives
 * k_new[t] and row out_loc[t] of the flat V pool receives v_new[t]; nothing
 * else in the pools changes.  This is the write that "out_loc" names in
 * mini-sglang "Engine Class" (forward_batch) and "slot_mapping" names in
 * miniVLLM "Engine Architecture" (prepare_prefill / prepare_decode); prefill
 * writes the initial KV cache and decode appends to it (zero-to-sglang Ch.1,
 * section 3.2).  The copy is bit-exact.
 *
 *   k_new, v_new : [num_tokens, num_kv_heads, head_dim] bf16, read only
 *   out_loc      : [num_tokens] int32 slots; must be distinct (several
 *                  tokens writing one slot leave one of them, unspecified);
 *                  a slot outside [0, num_slots) is skipped
 *   k_cache,
 *   v_cache      : pools, num_slots = num_pages * page_size rows of
 *                  num_kv_heads * head_dim values; written in place
 *   head_dim     : any multiple of 8 (rows are moved in 16-byte pieces)
 *
 * num_tokens == 0 is a no-op returning PKV_OK.
 */
int pkv_store_kv(const void* k_new, const void* v_new, const int32_t* out_loc,
                 int64_t num_tokens, void* k_cache, void* v_cache,
                 int64_t num_slots, int32_t num_kv_heads, int32_t head_dim,
                 void* stream);

/*
 * pkv_decode_workspace_bytes -- size of the workspace pkv_paged_attn_decode
 * needs for these arguments (0 when every request fits one split).  Pass the
 * same split_tokens (0 = automatic) as to the decode call.  Invalid shapes,
 * and shapes whose split partials would exceed 2^46 bytes, also give 0; the
 * decode call rejects the latter with PKV_EINVAL.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t split_tokens);

/*
 * pkv_decode_split_tokens -- the split length (tokens per split) the host
 * picks for these arguments, which sizes the launch and the workspace;
 * split_tokens != 0 is returned as the call would use it.  With
 * split_tokens = 0 and a batch that needs only a few rounds of the GPU's
 * resident wavefronts (at most 256 requests), the call may use a longer
 * split chosen on the device from the actual lengths, so that all work
 * units fit one round.  0 on invalid arguments.
 */
int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                int32_t max_seq_len, int32_t split_tokens);

/*
 * pkv_paged_attn_decode -- one query token per request attends to all of
 * its context through the page table.
 *
 * Decode feeds exactly one new token per sequence; context_lens counts
 * every token processed so far and block_tables give the KV history
 * (miniVLLM "Engine Architecture", prepare_decode).  seq_lens[r] therefore
 * INCLUDES the current token, whose K/V row must already be in the pool
 * (store first with pkv_store_kv).  For every query head h:
 *
 *   out[r, h, :] = softmax_j( softmax_scale * <q[r,h], K[r, j, h/g]> ) V[r, j, h/g]
 *
 * over j = 0 .. seq_lens[r]-1, with K[r, j, kvh] the row of slot
 * page_table[r, j / page_size] * page_size + j % page_size.  Long contexts
 * are cut into splits of split_tokens tokens that run in parallel; a second
 * kernel on the same stream merges the splits (flash-decoding).  With the
 * automatic split, a batch of at most 256 requests and 8 KV heads that
 * needs several rounds of units is instead shared evenly by one round of
 * workgroups (pieces cut at 16-token boundaries), when the workspace holds
 * the pieces' partials (pkv_decode_workspace_bytes counts them); the
 * result is the same up to rounding.
 *
 *   q            : [num_seqs, num_q_heads, head_dim] bf16
 *   k_cache,
 *   v_cache      : [num_pages, page_size, num_kv_heads, head_dim] bf16
 *   page_table   : [num_seqs, page_table_stride] int32
 *   seq_lens     : [num_seqs] int32, 1 <= seq_lens[r] <= max_seq_len;
 *                  a request with seq_lens[r] <= 0 gets an all-zero output
 *   max_seq_len  : host upper bound of seq_lens (sizes the launch);
 *                  page_table_stride * page_size >= max_seq_len
 *   head_dim     : 64 or 128
 *   page_size    : 16, 32, 64, 128 or 256
 *   num_q_heads / num_kv_heads : 1, 2, 4 or 8
 *   softmax_scale: finite and > 0 (typically 1/sqrt(head_dim))
 *   split_tokens : 0 = automatic (see pkv_decode_split_tokens), else a
 *                  multiple of 16 in [16, 65536]
 *   out          : [num_seqs, num_q_heads, head_dim] bf16 (round to nearest even)
 *   workspace    : device scratch of at least pkv_decode_workspace_bytes(...)
 *                  bytes, 256-byte aligned, for the per-split partial results
 *                  (running max, sum and un-normalised output in fp32); its
 *                  contents on entry do not matter.  Calls sharing one
 *                  workspace must be ordered (e.g. on one stream).  May be
 *                  NULL when the required size is 0.
 */
int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          int32_t page_size, int64_t num_pages,
                          const int32_t* page_table, int32_t page_table_stride,
                          const int32_t* seq_lens, int32_t num_seqs,
                          int32_t max_seq_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim,
                          float softmax_scale, int32_t split_tokens, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_decode_step -- one decode step of the batch in one call: the new
 * token's K/V rows are written to the pool (as pkv_store_kv) and every
 * request's query attends to its whole context (as pkv_paged_attn_decode).
 *
 * The engine's decode step first writes each sequence's new K/V row to the
 * slot out_loc assigns it and then runs attention over all tokens so far
 * (mini-sglang "Engine Class", forward_batch with out_loc; miniVLLM "Engine
 * Architecture", prepare_decode: slot_mapping of the one new token per
 * sequence).  Here the attention reads the new token's rows straight from
 * k_new / v_new while the same kernel writes them to the pool, so the step
 * is one launch (plus the split merge) instead of two.
 *
 * Arguments are those of pkv_paged_attn_decode plus:
 *   k_new, v_new : [num_seqs, num_kv_heads, head_dim] bf16, the rows of the
 *                  token at position seq_lens[r] - 1 of request r
 *   out_loc      : [num_seqs] int32, the slot of that token: it must be the
 *                  slot the page table gives position seq_lens[r] - 1, and no
 *                  other request of the call may read it.  Slots outside
 *                  [0, num_pages * page_size) are not written; a request with
 *                  seq_lens[r] <= 0 has no new token and its out_loc entry is
 *                  not used.
 *   k_cache,
 *   v_cache      : written at the out_loc slots (caller-owned, as above).
 *
 * Result: bit-identical to pkv_store_kv followed by pkv_paged_attn_decode on
 * the same stream.  Errors as pkv_paged_attn_decode; k_new, v_new or out_loc
 * NULL (with num_seqs > 0) or k_new / v_new not 16-byte aligned -> PKV_EINVAL.
 */
int pkv_decode_step(const void* q, const void* k_new, const void* v_new,
                    const int32_t* out_loc, void* k_cache, void* v_cache,
                    int32_t page_size, int64_t num_pages, const int32_t* page_table,
                    int32_t page_table_stride, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                    int32_t split_tokens, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pkv_decode_step_noalloc -- pkv_decode_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing: the
 * per-split partial results go to a fixed scratch array of the library
 * (pkv_decode_step_noalloc_max_bytes() bytes on each GPU, held from the
 * first call on that GPU until the process ends) instead of a caller
 * workspace.
 *
 * Arguments, result and errors are those of pkv_decode_step without
 * workspace and workspace_bytes.  A call whose arguments need more than
 * the scratch holds (pkv_decode_workspace_bytes(...) above the maximum)
 * returns PKV_ENOSPACE before anything is enqueued; PKV_EHIP if the
 * scratch array's device address cannot be found.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's partials (nothing
 * in it needs to start at zero): calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race.
 */
int pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                            const int32_t* out_loc, void* k_cache, void* v_cache,
                            int32_t page_size, int64_t num_pages, const int32_t* page_table,
                            int32_t page_table_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                            int32_t split_tokens, void* out, void* stream);

/* Bytes of the scratch array pkv_decode_step_noalloc uses on each GPU. */
size_t pkv_decode_step_noalloc_max_bytes(void);

/*
 * pkv_paged_attn_decode_shared -- decode (or the decode step, with the new
 * token's store) for a batch whose requests share cached prefixes, reading
 * each shared prefix once for all requests that share it.
 *
 * With prefix caching, requests that start with the same tokens point their
 * first page-table entries at the same physical pages (miniVLLM "Engine
 * Architecture", prepare_prefill: block tables for prefix reuse;
 * zero-to-sglang Ch.1, section 4 roadmap: RadixAttention).  The result is
 * that of pkv_paged_attn_decode (pkv_decode_step when k_new, v_new and
 * out_loc are given), up to rounding.  The work is split in two passes on
 * `stream`: for every group, the queries of all its members (all query
 * heads of a KV head) against the group's shared prefix as one MFMA
 * product per 128-key split of the prefix; then every request's remaining
 * tokens as in pkv_paged_attn_decode; the partial results of both are
 * merged by the split-merge kernel.
 *
 *   cu_groups    : [num_groups + 1] int32, cu_groups[0] = 0, non-decreasing,
 *                  cu_groups[num_groups] = num_seqs: group g is requests
 *                  cu_groups[g] .. cu_groups[g+1]-1 (a group of one request,
 *                  or with shared length 0, shares nothing)
 *   shared_lens  : [num_seqs] int32, tokens at the start of request r's
 *                  context that it shares with its group; used rounded down
 *                  to a multiple of 16.  Preconditions (not checked): every
 *                  member of a group has the same shared length and the same
 *                  page-table entries for it (the pass reads the pages through
 *                  the group's first member), and 0 <= shared_lens[r] <=
 *                  seq_lens[r] (< seq_lens[r] with the store: the new token
 *                  lies after the shared prefix).
 *   num_groups   : 1 .. num_seqs
 *   max_group_size, max_shared_len : host upper bounds (size the launch);
 *                  max_shared_len <= max_seq_len
 *   k_new, v_new, out_loc : as pkv_decode_step, or all NULL for plain decode
 *   workspace    : at least pkv_paged_attn_decode_shared_workspace_bytes(...)
 *                  bytes, 256-byte aligned (contents on entry do not matter)
 *   all others   : as pkv_decode_step
 *
 * Errors as pkv_decode_step; bad group arguments -> PKV_EINVAL.
 */
int pkv_paged_attn_decode_shared(const void* q, const void* k_new, const void* v_new,
                                 const int32_t* out_loc, void* k_cache, void* v_cache,
                                 int32_t page_size, int64_t num_pages,
                                 const int32_t* page_table, int32_t page_table_stride,
                                 const int32_t* seq_lens, int32_t num_seqs,
                                 int32_t max_seq_len, const int32_t* cu_groups,
                                 const int32_t* shared_lens, int32_t num_groups,
                                 int32_t max_group_size, int32_t max_shared_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 float softmax_scale, int32_t split_tokens, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

size_t pkv_paged_attn_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_seq_len, int32_t max_shared_len,
                                                    int32_t split_tokens);

/*
 * Decode-step graphs, one per batch-size bucket.
 *
 * The engines capture the decode step in graphs for a set of batch sizes
 * (e.g. 1, 2, 4, 8, 16, 32, ...), largest first, and at every step replay
 * the smallest graph that holds the batch: the batch is copied into the
 * first rows of fixed buffers and the rows past it are padded with a dummy
 * request (miniVLLM "Engine Architecture", CUDA graph capture and run_model;
 * mini-sglang "Engine Class", CUDA graph batch sizes and the dummy request
 * kept at an extra page-table row).
 *
 * pkv_decode_graphs_create captures, for each bucket b, one call of
 * pkv_decode_step (or of pkv_paged_attn_decode when k_new, v_new and
 * out_loc are all NULL) with num_seqs = b on the given fixed buffers, which
 * must be sized for the largest bucket (q [B_max, Hq, d], k_new / v_new
 * [B_max, Hkv, d], out_loc and seq_lens [B_max], page_table
 * [B_max, page_table_stride], out [B_max, Hq, d]).  The buffers stay owned
 * by the caller and must outlive the graphs; their contents are read when a
 * graph is replayed, not at capture.  Every bucket uses one workspace: the
 * caller's (at least pkv_decode_graphs_workspace_bytes(...) bytes, 256-byte
 * aligned) or, when workspace is NULL, the fixed scratch of
 * pkv_decode_step_noalloc.  The automatic split is used (split_tokens = 0).
 * The graphs belong to the device current at creation.
 *
 *   buckets      : num_buckets (1 .. 64) distinct positive batch sizes, any
 *                  order (pkv_decode_graphs_workspace_bytes returns 0 for
 *                  any other list)
 *   graphs       : receives the handle (NULL on error)
 *   all others   : as pkv_decode_step, for the largest bucket
 *
 * Returns PKV_EINVAL / PKV_EUNSUPPORTED as pkv_decode_step would for the
 * largest bucket, PKV_ENOSPACE if the workspace (or the fixed scratch) is
 * too small, PKV_EHIP if capture or instantiation fails; nothing is left
 * allocated on error.
 *
 * pkv_decode_graphs_replay enqueues on `stream` the graph of the smallest
 * bucket >= num_seqs (the bucket is written to *bucket_used when non-NULL).
 * Before it, rows num_seqs .. bucket-1 of seq_lens must hold padding
 * (seq_lens <= 0: the dummy request, which reads and writes nothing and
 * gets a zero output row).  num_seqs == 0 enqueues nothing; num_seqs above
 * the largest bucket, or a call on another device -> PKV_EINVAL.  Replays
 * sharing a workspace (or the fixed scratch) must be ordered.
 */
typedef struct pkv_decode_graphs pkv_decode_graphs;

size_t pkv_decode_graphs_workspace_bytes(const int32_t* buckets, int32_t num_buckets,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len);

int pkv_decode_graphs_create(const int32_t* buckets, int32_t num_buckets, const void* q,
                             const void* k_new, const void* v_new, const int32_t* out_loc,
                             void* k_cache, void* v_cache, int32_t page_size,
                             int64_t num_pages, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* seq_lens,
                             int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float softmax_scale, void* out,
                             void* workspace, size_t workspace_bytes,
                             pkv_decode_graphs** graphs);

int pkv_decode_graphs_replay(pkv_decode_graphs* graphs, int32_t num_seqs, void* stream,
                             int32_t* bucket_used);

/* Releases the graphs (NULL is a no-op); the caller's buffers are untouched. */
void pkv_decode_graphs_destroy(pkv_decode_graphs* graphs);

/*
 * pkv_decode_multi_workspace_bytes -- size of the workspace
 * pkv_paged_attn_decode_multi needs (0 when every request fits one split,
 * and on invalid arguments).  Pass the same split_tokens as to the call.
 */
size_t pkv_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_seq_len,
                                        int32_t split_tokens);

/*
 * pkv_paged_attn_decode_multi -- q_len query tokens per request, each
 * attending causally to the context up to its own position.
 *
 * This is the decode step of speculative decoding's verification, where a
 * request feeds a few draft tokens at once instead of one (zero-to-sglang
 * Part II Ch.1, section 4, roadmap: speculative decoding; the causal rule
 * with cached tokens is that of prefill, miniVLLM "Engine Architecture",
 * prepare_prefill).  seq_lens[r] = n counts every token including the q_len
 * new ones, whose K/V rows must already be in the pool (pkv_store_kv with
 * q_len rows per request).  Query token t of request r sits at position
 * n - q_len + t and, for every query head h,
 *
 *   out[r, t, h, :] = softmax_j( softmax_scale * <q[r,t,h], K[r, j, h/g]> ) V[r, j, h/g]
 *
 * over j = 0 .. n - q_len + t.  With q_len = 1 this is pkv_paged_attn_decode.
 * A token with no visible key (position < 0, when n < q_len) and every
 * token of a request with n <= 0 get an all-zero output row.
 *
 *   q            : [num_seqs, q_len, num_q_heads, head_dim] bf16
 *   q_len        : 1 .. 16.  A block of the kernel takes up to 16 / g query
 *                  tokens of one KV head; longer drafts run in several
 *                  blocks per KV head, each reading the context again
 *                  (mostly from L2).  Longer query runs are prefill's shape.
 *   out          : [num_seqs, q_len, num_q_heads, head_dim] bf16
 *   workspace    : at least pkv_decode_multi_workspace_bytes(...) bytes,
 *                  256-byte aligned (contents on entry do not matter).
 *   all others   : as pkv_paged_attn_decode.
 *
 * Errors as pkv_paged_attn_decode; q_len outside 1 .. 16 -> PKV_EINVAL.
 */
int pkv_paged_attn_decode_multi(const void* q, int32_t q_len, const void* k_cache,
                                const void* v_cache, int32_t page_size, int64_t num_pages,
                                const int32_t* page_table, int32_t page_table_stride,
                                const int32_t* seq_lens, int32_t num_seqs,
                                int32_t max_seq_len, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                float softmax_scale, int32_t split_tokens, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn_prefill -- causal attention of a flat ragged batch of new
 * tokens over their cached prefix and themselves.
 *
 * Prefill feeds only the tokens after each request's cached prefix, laid
 * out flat with cumulative offsets cu_seqlens_q, e.g. [0, 5, 8, 12]
 * (miniVLLM "Engine Architecture", prepare_prefill); the extend length is
 * the sequence length minus the cached length (zero-to-sglang Ch.1,
 * section 3.3).  New token i of request r sits at absolute position
 * prefix_lens[r] + i and sees keys 0 .. prefix_lens[r] + i of its request:
 *
 *   out[t, h, :] = softmax_{j <= P_r+i}( softmax_scale * <q[t,h], K[r,j,h/g]> ) V[r, j, h/g]
 *
 * with t = cu_seqlens_q[r] + i.  Keys are read through the page table, so
 * the new tokens' K/V rows must already be in the pool (pkv_store_kv first).
 *
 *   q            : [num_tokens, num_q_heads, head_dim] bf16
 *   cu_seqlens_q : [num_seqs + 1] int32, non-decreasing, cu[0] = 0,
 *                  cu[num_seqs] = num_tokens; request r owns rows
 *                  cu[r] .. cu[r+1]-1 (an empty request is allowed)
 *   prefix_lens  : [num_seqs] int32 >= 0, cached tokens per request
 *   max_q_len    : host upper bound of cu[r+1]-cu[r] (sizes the launch)
 *   max_seq_len  : host upper bound of prefix_lens[r] + (cu[r+1]-cu[r]);
 *                  page_table_stride * page_size >= max_seq_len
 *   head_dim     : 64 or 128
 *   page_size    : 16, 32, 64, 128 or 256
 *   num_q_heads / num_kv_heads : 1, 2, 4 or 8
 *   softmax_scale: finite and > 0
 *   out          : [num_tokens, num_q_heads, head_dim] bf16; rows outside
 *                  every request are not written
 *   workspace    : device memory, 16-byte aligned, at least
 *                  pkv_prefill_workspace_bytes() bytes, caller-owned.  It
 *                  holds the counter that hands work items to the resident
 *                  blocks: it must be zero before its first use (e.g.
 *                  allocated zeroed), and every call puts it back to zero
 *                  before its kernel ends, so it is reused without clearing.
 *                  Calls sharing one workspace must be ordered (one stream);
 *                  concurrent calls need separate workspaces.
 *
 * Returns PKV_ENOSPACE if workspace_bytes is too small.  num_tokens == 0 is a
 * no-op returning PKV_OK (the workspace is not touched).
 */
int pkv_paged_attn_prefill(const void* q, const int32_t* cu_seqlens_q,
                           const int32_t* prefix_lens, int32_t num_seqs,
                           int32_t num_tokens, int32_t max_q_len,
                           int32_t max_seq_len, const void* k_cache,
                           const void* v_cache, int32_t page_size,
                           int64_t num_pages, const int32_t* page_table,
                           int32_t page_table_stride, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           float softmax_scale, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of workspace pkv_paged_attn_prefill needs (a small constant). */
size_t pkv_prefill_workspace_bytes(void);

/*
 * pkv_prefill_metadata -- build a prefill batch's cu_seqlens_q and
 * slot_mapping (out_loc) on the device from lengths and the page table.
 *
 * The prefill batch holds only the tokens after each sequence's cached
 * prefix; cu_seqlens_q accumulates their counts, e.g. [0, 5, 8, 12], and
 * slot_mapping gives every new token the cache slot it is written to
 * (miniVLLM "Engine Architecture", ModelRunner / prepare_prefill).  New token
 * i of request r is at position prefix_lens[r] + i; its slot is
 * page_table[r, t / page_size] * page_size + t % page_size with that t.
 *
 *   seq_lens     : [num_seqs] int32, tokens of each sequence including the
 *                  new ones
 *   prefix_lens  : [num_seqs] int32, cached tokens (the new count is
 *                  max(seq_lens[r] - max(prefix_lens[r], 0), 0))
 *   page_table   : [num_seqs, page_table_stride] int32
 *   page_size    : > 0 (any value)
 *   max_tokens   : capacity of out_loc; tokens at flat index >= max_tokens
 *                  are not written
 *   cu_seqlens_q : [num_seqs + 1] int32, written
 *   out_loc      : [max_tokens] int32, written for flat indices below the
 *                  total; a position outside the page-table row gets -1
 *                  (pkv_store_kv skips it)
 *
 * Host-checkable errors: null pointers, num_seqs < 0, max_tokens < 0,
 * page_table_stride <= 0 or page_size <= 0 -> PKV_EINVAL.  num_seqs == 0 is
 * a no-op.
 */
int pkv_prefill_metadata(const int32_t* seq_lens, const int32_t* prefix_lens,
                         int32_t num_seqs, const int32_t* page_table,
                         int32_t page_table_stride, int32_t page_size,
                         int32_t max_tokens, int32_t* cu_seqlens_q,
                         int32_t* out_loc, void* stream);

/*
 * pkv_decode_metadata -- the decode step's slot_mapping on the device: each
 * sequence contributes its most recent token, at position seq_lens[r] - 1
 * (context_lens counts every token so far), and out_loc[r] is that token's
 * slot (miniVLLM "Engine Architecture", prepare_decode).  A sequence with
 * seq_lens[r] <= 0 (a padding row) or whose position falls outside its
 * page-table row gets -1.
 *
 * Errors as pkv_prefill_metadata.
 */
int pkv_decode_metadata(const int32_t* seq_lens, int32_t num_seqs,
                        const int32_t* page_table, int32_t page_table_stride,
                        int32_t page_size, int32_t* out_loc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
