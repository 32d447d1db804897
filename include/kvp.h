/*
 * kvp.h -- paged KV cache and paged decode attention for AMD MI355X (gfx950).
 *
 * The method ("KV-Cache Optimization Techniques", section "PagedAttention",
 * eq. 1; "Understanding KV-Cache Optimization in Modern LLM Serving", section
 * "PagedAttention Solution"): the K/V rows of every sequence live in
 * fixed-size physical pages of P tokens; a per-sequence block table maps the
 * sequence's logical block i (tokens i*P .. i*P+P-1) to a physical page id.
 * Decode attention gathers the pages in logical order and computes
 *     out_j = softmax(scale * q_j . [K_page1; ...; K_pagen]^T) [V_page1; ...; V_pagen]
 * for every query head j of the one new query token of each sequence.
 *
 * ---------------------------------------------------------------------------
 * Symbols
 *   P      page size in tokens (16 or 32)
 *   H_kv   KV heads, H_q query heads, g = H_q / H_kv query heads per KV head
 *   D      head dimension (64 or 128)
 *   B      sequences in a call
 * Query head j reads KV head j / g: consecutive query heads share a KV head
 * ("KV-Cache Optimization Techniques", section "Multi-Query and Grouped-Query
 * Caching", eq. 7; MQA is H_kv = 1).
 *
 * ---------------------------------------------------------------------------
 * Memory layout (one layer).  All arrays are dense, row-major, no padding.
 *   K pool, element type T (bfloat16 bits, or int8 code):
 *       K[page][h][t][d]      at element ((page*H_kv + h)*P + t)*D + d
 *   V pool, element type T, stored transposed inside each (page, head) tile:
 *       V[page][h][t][d]      at element ((page*H_kv + h)*D + d)*P + t
 *   INT8 metadata, one (scale, zero) float16 pair per token per KV head, the
 *   same layout for K and for V:
 *       scale of row (page,h,t)  at float16 element ((page*H_kv + h)*P + t)*2 + 0
 *       zero  of row (page,h,t)  at float16 element ((page*H_kv + h)*P + t)*2 + 1
 *     and the stored value of element d of that row is
 *       float(scale) * code[d] + float(zero)
 *   A pool of num_pages pages spans num_pages*H_kv*P*D elements per K or V
 *   array (kvp_pool_bytes).  One page id names the same page in every layer's
 *   pool, so one block table serves all layers.
 *   q, out:         [B][H_q][D] bfloat16 bits.
 *   block_tables:   [B][max_blocks] int32; entry (b, i) is the page holding
 *                   tokens i*P .. i*P+P-1 of sequence b.  Entries at
 *                   i >= ceil(ctx_b / P) are never read.
 *   context_lens:   [B] int32, tokens each sequence attends over.
 * Token position pos of sequence b sits in page block_tables[b][pos / P] at
 * in-page row pos % P.  Rows of a page beyond a sequence's length, and pages
 * no table names, are never read by decode and may hold anything (NaN too).
 *
 * INT8 rows ("KV-Cache Optimization Techniques", section "KV-Cache
 * Quantization", eq. 3, per-token calibration): each (token, KV head) row x of
 * D bfloat16 values is stored as
 *     mn = min x, mx = max x                          (float32, exact)
 *     z  = f16( (mx + mn) * 0.5f )                    (float32 ops, RNE to f16)
 *     s  = f16( (mx - mn) / 254.0f ); s = 1.0 if s == 0
 *     code[d] = clamp( rint_even( (x[d] - float(z)) / float(s) ), -128, 127 )
 * with every float32 operation IEEE round-to-nearest-even.  Inputs need
 * |x| <= 65504 so that z is finite in float16.
 *
 * INT4 rows (the same section: FP16 -> INT4 is a 4x smaller cache): the
 * INT8 contract with 14 steps and codes clamped to [-8, 7],
 *     z = f16((mx + mn) * 0.5f),  s = f16((mx - mn) / 14.0f) (1 if 0),
 *     code[d] = clamp(rint_even((x[d] - float(z)) / float(s)), -8, 7),
 * stored two channels per byte as code + 8, channel 2j in the low nibble of
 * byte j.  K:  byte ((page*H_kv + h)*P + t)*(D/2) + d/2
 *        V:  byte ((page*H_kv + h)*(D/2) + d/2)*P + t
 * (every byte belongs to one token, so appends never share a byte).
 *
 * FP8 rows: OCP e4m3 ("e4m3fn": 4 exponent bits with bias 7, 3 mantissa
 * bits, largest finite 448, no infinities) with one float16 scale per row:
 *     s = f16(max|x| / 448.0f) (1 if 0),  code[d] = e4m3(x[d] / float(s)),
 * x / s in float32, e4m3() rounding to nearest with ties to the even code and
 * saturating to +-448; stored value float(s) * e4m3_value(code).  Codes use
 * the INT8 layout (one byte per element); the metadata pair is (scale, 0).
 *
 * ---------------------------------------------------------------------------
 * Ownership.  The caller owns every device buffer (pools, metadata, q, out,
 * tables, lengths, workspace) and keeps it alive until the work queued on the
 * stream has finished.  The library owns the host pool object: the page
 * free-list and per-page reference counts.  The library never allocates or
 * frees device memory.
 *
 * Errors.  Every call returns kvp_status.  A host call that fails leaves all
 * state unchanged.  Device work is queued asynchronously on the given stream
 * (NULL = the default stream); a failed launch returns KVP_E_HIP.  Device data
 * the host cannot see is handled without faulting: a page id outside
 * [0, num_pages) makes the tokens of that block count as absent (decode) or
 * the row is not written (append); context_lens are clamped to
 * [0, min(max_context_len, max_blocks*P)].  Such inputs are caller errors
 * with no other guarantee about the result.
 *
 * Threads.  A pool object is not thread safe; the caller serializes calls on
 * one pool.  Device calls on one stream run in order.
 */
#ifndef KVP_H
#define KVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; NULL means the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t* kvp_stream_t;

typedef enum {
  KVP_OK = 0,
  KVP_E_INVAL = 1,        /* bad argument, or a state violation (double free ...) */
  KVP_E_NOPAGES = 2,      /* not enough free pages; nothing was allocated */
  KVP_E_UNSUPPORTED = 3,  /* shape or dtype with no kernel (P, D, g, dtype) */
  KVP_E_HIP = 4,          /* a HIP runtime call failed */
  KVP_E_SCRATCH = 5       /* needs more scratch than KVP_DECODE_SCRATCH_BYTES (noalloc call) */
} kvp_status;

typedef enum { KVP_BF16 = 0, KVP_INT8 = 1, KVP_INT4 = 2, KVP_FP8 = 3 } kvp_kv_dtype;

typedef struct {
  int32_t num_pages;     /* pages in the pool, > 0 */
  int32_t page_size;     /* P: 16 or 32 */
  int32_t num_kv_heads;  /* H_kv, > 0 */
  int32_t head_dim;      /* D: 64 or 128 */
  kvp_kv_dtype dtype;     /* KVP_BF16, KVP_INT8, KVP_INT4 or KVP_FP8 */
} kvp_pool_desc;

typedef struct kvp_pool kvp_pool; /* opaque; host memory owned by the library */

/* Text for a status code (static storage). */
const char* kvp_status_string(kvp_status s);

/* ---- Pool and page allocation (host only; "KV-Cache Optimization
 * Techniques", section "PagedAttention": pages allocated on demand and freed
 * when the request completes; section "Prefix Caching": pages shared by
 * requests with a common prefix). -------------------------------------- */

/* Bytes of one layer's K (or V) array, and of its metadata array (0 for
 * bfloat16; INT8, INT4 and FP8 pools have one).  Either output pointer may be
 * NULL. */
kvp_status kvp_pool_bytes(const kvp_pool_desc* desc, size_t* kv_bytes, size_t* meta_bytes);

/* Create a pool object: every page free, reference count 0.  *out receives a
 * new object the caller releases with kvp_pool_destroy. */
kvp_status kvp_pool_create(const kvp_pool_desc* desc, kvp_pool** out);
void kvp_pool_destroy(kvp_pool* pool);                 /* NULL is a no-op */
kvp_status kvp_pool_get_desc(const kvp_pool* pool, kvp_pool_desc* out);
int32_t kvp_pool_free_count(const kvp_pool* pool);     /* -1 if pool is NULL */
/* Reference count of one page (0 = free), or -1 if the id is out of range. */
int32_t kvp_pool_refcount(const kvp_pool* pool, int32_t page);

/* Take n pages from the free-list (last freed, first taken) and write their
 * ids to out_ids[0..n-1]; each gets reference count 1.  All or nothing:
 * KVP_E_NOPAGES if fewer than n are free. */
kvp_status kvp_pages_alloc(kvp_pool* pool, int32_t n, int32_t* out_ids);
/* Add one reference to each listed page (sharing it with one more sequence).
 * Every page must be in use (count >= 1); KVP_E_INVAL otherwise. */
kvp_status kvp_pages_ref(kvp_pool* pool, int32_t n, const int32_t* ids);
/* Drop one reference from each listed page; a page whose count reaches 0
 * returns to the free-list.  A listed page must hold at least as many
 * references as times it is listed; KVP_E_INVAL otherwise. */
kvp_status kvp_pages_free(kvp_pool* pool, int32_t n, const int32_t* ids);

/* Block-table row helpers (host memory).  kvp_seq_grow makes row cover
 * new_len tokens: blocks ceil(cur_len/P) .. ceil(new_len/P)-1 get freshly
 * allocated pages; earlier entries are kept.  All or nothing. */
kvp_status kvp_seq_grow(kvp_pool* pool, int32_t* row, int32_t max_blocks,
                        int32_t cur_len, int32_t new_len);
/* Point blocks 0..n_blocks-1 of dst_row at the pages of src_row and add a
 * reference to each (a shared prefix of whole pages). */
kvp_status kvp_seq_share(kvp_pool* pool, const int32_t* src_row, int32_t* dst_row,
                         int32_t n_blocks);
/* Drop the references of blocks 0..n_blocks-1 of row and set them to -1
 * (the request completed). */
kvp_status kvp_seq_release(kvp_pool* pool, int32_t* row, int32_t n_blocks);

/* Drop the pages of a sequence of ctx_len tokens that hold only tokens a
 * sink + window decode (kvp_paged_attention_decode_window) never reads:
 * blocks ceil(sink_tokens/P) .. floor((ctx_len - window_tokens)/P) - 1.  Their
 * references are released and their entries set to -1; entries that are
 * already -1 are skipped.  Nothing happens when sink_tokens + window_tokens >=
 * ctx_len.  window_tokens must be > 0.  All or nothing. */
kvp_status kvp_seq_evict_window(kvp_pool* pool, int32_t* row, int32_t max_blocks, int32_t ctx_len,
                                int32_t sink_tokens, int32_t window_tokens);

/* ---- Prefix cache (host) ------------------------------------------------------
 * "KV-Cache Optimization Techniques", section "Prefix Caching": requests that
 * share a prefix reuse its KV-cache; the token sequence is hashed, cached
 * prefixes form a radix tree for longest-prefix matching, and shared pages
 * are copied on write.  The cache is a radix tree over whole pages: one node
 * per block of P token ids, keyed by a 64-bit hash chained over the whole
 * prefix, holding the page with that block's K/V and one reference to it.
 * Token ids of every matched block are compared, so a hash collision can
 * only shorten a match.  The pool must outlive the cache; the cache is not
 * thread safe (serialize with the pool). */
typedef struct kvp_prefix_cache kvp_prefix_cache;  /* opaque, host memory */

kvp_status kvp_prefix_cache_create(kvp_pool* pool, kvp_prefix_cache** out);
/* Drops the cache's reference on every cached page (pages no sequence holds
 * return to the free list).  NULL is a no-op. */
void kvp_prefix_cache_destroy(kvp_prefix_cache* cache);
/* Pages the cache holds a reference to, or -1 for NULL. */
int32_t kvp_prefix_cache_pages(const kvp_prefix_cache* cache);
/* Longest cached prefix of tokens[0..n_tokens) in whole blocks, at most
 * max_pages blocks: *n_blocks_out = k and pages_out[0..k) are its pages in
 * block order, each with one reference added for the caller (the pages go
 * into the new sequence's block table; release them with kvp_pages_free or
 * kvp_seq_release).  Matched nodes become most recently used. */
kvp_status kvp_prefix_match(kvp_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                            int32_t* pages_out, int32_t max_pages, int32_t* n_blocks_out);
/* Cache the full blocks of a sequence whose K/V are in pages[0..n_tokens/P):
 * blocks already cached keep their page; each newly cached block's page
 * (which must be in use) gets one reference held by the cache.  All or
 * nothing; a hash collision with different tokens stops caching there. */
kvp_status kvp_prefix_insert(kvp_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                             const int32_t* pages);
/* Evict least-recently-used leaf blocks whose page only the cache holds,
 * until n_pages pages went back to the free list or none is left; parents
 * left without children become candidates in turn.  *n_freed (may be NULL)
 * receives the count. */
kvp_status kvp_prefix_evict(kvp_prefix_cache* cache, int32_t n_pages, int32_t* n_freed);

/* Make the blocks a sequence will write to private before appending tokens
 * cur_len .. new_len-1: missing blocks get fresh pages; if the partly filled
 * last block (the one holding position cur_len) is also held elsewhere
 * (reference count > 1), the row gets a fresh page for it, one reference to
 * the shared page is dropped, and the pair (old page, new page) is written to
 * copy_src[0], copy_dst[0] with *n_copies = 1 (0 otherwise): copy it on the
 * device with kvp_copy_pages before appending.  All or nothing
 * (KVP_E_NOPAGES if the free list is short). */
kvp_status kvp_seq_prepare_append(kvp_pool* pool, int32_t* row, int32_t max_blocks,
                                  int32_t cur_len, int32_t new_len, int32_t* copy_src,
                                  int32_t* copy_dst, int32_t* n_copies);

/* ---- Append (device) ------------------------------------------------------
 * For each of n_tokens new tokens i: sequence seq_idx[i], position pos[i];
 * write k_new[i][h][:] and v_new[i][h][:] (bfloat16 [n_tokens][H_kv][D]) into
 * row pos[i] % P of page block_tables[seq_idx[i]][pos[i] / P], for every KV
 * head h; INT8, INT4 and FP8 pools quantize each row as described above and
 * write its codes and (scale, zero).  k_meta/v_meta must be NULL for bfloat16
 * pools and non-NULL otherwise.
 * All pointers are device pointers.  Rows whose seq_idx is outside
 * [0, num_seqs), whose pos is outside [0, max_blocks*P) or whose page id is
 * outside [0, num_pages) are not written.  Two tokens naming the same row
 * race.  A page shared by several sequences must not be appended into. */
kvp_status kvp_kv_append(const kvp_pool* pool, void* k_pool, void* v_pool,
                         void* k_meta, void* v_meta,
                         const void* k_new, const void* v_new,
                         const int32_t* seq_idx, const int32_t* pos, int32_t n_tokens,
                         const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks,
                         kvp_stream_t stream);

/* Copy whole pages of one layer's pools (K, V and, for INT8, both metadata
 * arrays; every KV head): for i < n, page src_dst[2i] to page src_dst[2i+1].
 * src_dst is a device array of n int32 pairs; a pair naming a page outside
 * the pool, or the same page twice, is skipped.  Pairs must not overlap (no
 * page both written and read by the call). */
kvp_status kvp_copy_pages(const kvp_pool* pool, void* k_pool, void* v_pool, void* k_meta,
                          void* v_meta, const int32_t* src_dst, int32_t n, kvp_stream_t stream);

/* ---- Decode plan (host, pure) -----------------------------------------------
 * Work is split into B * H_kv * num_splits workgroups: each covers one
 * (sequence, KV head) pair and one range of pages_per_split logical blocks,
 * handled by waves_per_group wavefronts that each stream a share of the pages
 * and merge their softmax partials in LDS.  With num_splits > 1 the partials
 * go to the workspace and a second kernel merges them by log-sum-exp.
 * num_splits_req <= 0 picks a split count from max_context_len and num_cus.
 */
typedef struct {
  int32_t num_splits;
  int32_t pages_per_split;
  int32_t waves_per_group;
  int32_t use_mfma;          /* 1: matrix-core kernel (g >= 4); 0: vector ALU kernel */
  size_t workspace_bytes;    /* device workspace decode needs (0 when num_splits == 1) */
} kvp_decode_plan_t;

kvp_status kvp_decode_plan(const kvp_pool_desc* desc, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_context_len, int32_t num_splits_req, int32_t num_cus,
                           kvp_decode_plan_t* out);

/* Workspace bytes kvp_paged_attention_decode needs on the current device. */
kvp_status kvp_decode_workspace_bytes(const kvp_pool* pool, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      int32_t num_splits_req, size_t* bytes);

/* ---- Decode (device) --------------------------------------------------------
 * out[b][j][:] = attention of q[b][j][:] over tokens 0 .. ctx_b-1 of sequence
 * b (ctx_b = context_lens[b]) through KV head j/g, as eq. 1 above, scores
 * multiplied by `scale` (normally 1/sqrt(D)).  Scores, softmax and the
 * weighted sum are accumulated in float32; out is rounded to bfloat16 (RNE).
 * Matrix-core operands (g >= 4): for bfloat16 pools q and K are used as
 * stored and the softmax weights p are rounded to bfloat16 before P.V.  For
 * INT8, INT4 and FP8 pools the codes convert to float16 exactly, q is rounded
 * to float16 (so |q| <= 65504 is a precondition, and elements below 2^-14
 * keep fewer bits), and each weight times the token's V scale, p * s, is
 * rounded to float16 before P.V.  The weights carry a power of two chosen
 * from the largest V scale seen so far in the sequence (raised, with the
 * running sums rescaled exactly, when a page brings a larger one), so these
 * operands stay below 2^15 and above float16's subnormals for V scales from
 * about 2^-85 to the largest float16 (tested with V rows 1e-4 and 3e4 times
 * unit draws); only products p * s below about 2^-28 times the largest V
 * scale lose bits.  INT4 K codes enter as code + 1032 (exact in float16) and
 * 1032 times the sum of q's float16 values starts each score's float32
 * accumulation at the negated offset, so the accumulator holds values of
 * about 1032 |sum of q| and its roundings are relative to that (for unit q,
 * about 1e-3 absolute on raw dot products of ~50, below the float16
 * rounding of q and p * s).  The vector-ALU path (g < 4) computes in float32
 * throughout.
 * ctx_b == 0 gives out = 0.  max_context_len is a host-side upper bound of
 * context_lens (1 .. max_blocks*P), used to plan the split.  workspace must
 * be a device buffer of at least kvp_decode_workspace_bytes (may be NULL when
 * that is 0).  All array pointers are device pointers.  Output rows depend
 * only on the pages' contents in logical order, so relabelling physical pages
 * leaves the result bit-identical. */
kvp_status kvp_paged_attention_decode(const kvp_pool* pool, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const void* k_meta, const void* v_meta,
                                      const int32_t* block_tables, int32_t max_blocks,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      float scale, void* out, int32_t num_splits_req,
                                      void* workspace, size_t workspace_bytes,
                                      kvp_stream_t stream);

/* ---- Decode that allocates nothing (device) ---------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * attention, plan and kernels as kvp_paged_attention_decode, with the split
 * partials in a fixed device buffer the library holds on each GPU it runs on
 * (KVP_DECODE_SCRATCH_BYTES, until the process ends) instead of a workspace
 * argument.  The caller still passes every input and output.  The call makes
 * no device allocation; a plan whose workspace (kvp_decode_workspace_bytes)
 * exceeds the buffer returns KVP_E_SCRATCH and queues nothing.  All calls on
 * one GPU share its buffer: calls that can overlap on one GPU (different
 * streams, or several threads) race and must be serialized by the caller.
 * The first call on a device looks up the buffer's address there (KVP_E_HIP
 * if that fails). */
#define KVP_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
kvp_status kvp_paged_attention_decode_noalloc(const kvp_pool* pool, const void* q,
                                              const void* k_pool, const void* v_pool,
                                              const void* k_meta, const void* v_meta,
                                              const int32_t* block_tables, int32_t max_blocks,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len,
                                              float scale, void* out, int32_t num_splits_req,
                                              kvp_stream_t stream);

/* ---- Decode over attention sinks and a recent window (device) --------------
 * "KV-Cache Optimization Techniques", section "Token Eviction Strategies",
 * eq. 5 (StreamingLLM): keep the first s tokens ("attention sinks") and the
 * last w tokens; section "Sliding Window Cache", eq. 6: the window alone
 * (s = 0).  For a sequence of n = context_lens[b] tokens with
 * sink_tokens + window_tokens < n, the query attends only to tokens t < s and
 * t >= n - w; otherwise to all n tokens.  window_tokens == 0 means no window
 * (the same result as kvp_paged_attention_decode).  Pages that hold only
 * dropped tokens are never read, so their table entries may be -1 (see
 * kvp_seq_evict_window).  Everything else is as kvp_paged_attention_decode;
 * the workspace is sized by kvp_decode_window_workspace_bytes. */
kvp_status kvp_decode_window_workspace_bytes(const kvp_pool* pool, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t max_context_len,
                                             int32_t sink_tokens, int32_t window_tokens,
                                             int32_t num_splits_req, size_t* bytes);
kvp_status kvp_paged_attention_decode_window(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, int32_t sink_tokens, int32_t window_tokens, void* out, int32_t num_splits_req,
    void* workspace, size_t workspace_bytes, kvp_stream_t stream);

/* ---- Balanced decode for ragged batches (host schedule + device) ----------
 * "KV-Cache Optimization Techniques", section "PagedAttention": the work of
 * a decode step is the (sequence, KV head, page) triples.  With ragged
 * lengths, splitting each sequence the same way leaves the compute units
 * that hold short sequences idle while the long ones finish.  Here the
 * caller, who knows the lengths on the host, builds a schedule that gives
 * every bin an equal share of the streamed blocks.  A bin is one wavefront's
 * stream on the matrix-core path (g >= 4) and one workgroup on the vector
 * path (g < 4):
 *   - the (sequence, KV head) pairs are laid end to end, KV head fastest,
 *     each contributing its streamed blocks (all ceil(n/P), or with sinks and
 *     a window, eq. 5 of section "Token Eviction Strategies", the sink blocks
 *     and the window's blocks);
 *   - bin k of num_bins covers blocks [k*T/num_bins, (k+1)*T/num_bins) of
 *     that list (T = all blocks); num_bins = min(max_bins, ceil(T/8)), at
 *     least 1 (kvp_decode_schedule_bins gives the count that fills the
 *     device);
 *   - the pieces of pairs a bin covers are its items, processed in order; on
 *     the matrix-core path the items of a wavefront's stream share its
 *     register ring, so the next item's pages load while the current one
 *     finishes, and no barrier separates items; a pair inside one bin writes
 *     its output directly, a pair cut by bin boundaries writes a float32
 *     partial per piece and is merged by log-sum-exp afterwards (a second
 *     kernel, launched only if needed).
 * With equal lengths whose pairs divide evenly into bins, every pair lands in
 * one bin and no merge runs. */
typedef struct {
  int32_t num_bins;       /* workgroups of the split kernel */
  int32_t num_items;      /* pieces over all bins */
  int32_t num_merge;      /* pairs cut across bins (merge entries) */
  int32_t num_slots;      /* partials those pairs write */
  int32_t items_offset;   /* word offset of the item records in the schedule */
  int32_t merge_offset;   /* word offset of the merge records */
  int32_t sink_tokens;    /* the selection the schedule was built for */
  int32_t window_tokens;
  int32_t sched_words;    /* int32 words of the schedule that are used */
  size_t workspace_bytes; /* device workspace the partials need (0: none) */
} kvp_schedule_info;

/* Upper bounds, for any lengths, of the schedule size (bytes of int32 words)
 * and of the workspace the scheduled decode needs, for num_seqs sequences,
 * num_q_heads query heads and at most max_bins bins (> 0). */
kvp_status kvp_decode_schedule_bounds(const kvp_pool* pool, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_bins,
                                      size_t* sched_bytes, size_t* workspace_bytes);

/* Bins that keep every compute unit of the current device busy along a
 * schedule for this pool and num_q_heads: four per compute unit (one
 * wavefront per SIMD), eight for INT8 and FP8 pools and twelve for INT4
 * pools on the matrix-core path with 4 <= g <= 16, whose stream kernel is
 * built for two (INT4: three) wavefronts per SIMD.  The
 * value to pass as max_bins below when there is no reason to pick another.
 * KVP_E_INVAL for a bad pool, head count or pointer; KVP_E_HIP when the
 * device cannot be queried. */
kvp_status kvp_decode_schedule_bins(const kvp_pool* pool, int32_t num_q_heads,
                                    int32_t* max_bins);

/* Build the schedule (host).  context_lens: host array of the B lengths the
 * device array will hold at decode time (0 <= n <= max_blocks*P, else
 * KVP_E_INVAL); sink_tokens/window_tokens as for the window decode (0, 0 for
 * the full decode); max_bins > 0; sched: host buffer of sched_bytes >= the
 * bound above.  Layout (int32 words):
 *   [0..7]   num_bins, num_items, num_merge, num_slots, items_offset,
 *            merge_offset, 0, 0;
 *   [8 .. 8+num_bins]  bin_start: bin k owns items bin_start[k] .. bin_start[k+1]-1;
 *   items_offset + 8*i: item i = sequence, KV head, first streamed block,
 *            end block (exclusive, counted in the sequence's streamed list),
 *            partial slot (-1: write the output), 0, 0, 0;
 *   merge_offset + 4*e: entry e = sequence, KV head, first slot, slot count.
 * The caller copies the first info->sched_words words to device memory. */
kvp_status kvp_decode_schedule(const kvp_pool* pool, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                               int32_t sink_tokens, int32_t window_tokens, int32_t max_bins,
                               int32_t* sched, size_t sched_bytes, kvp_schedule_info* info);

/* The decode (window decode when info->window_tokens > 0) along a schedule:
 * the same result as kvp_paged_attention_decode(_window) within float32
 * summation order.  sched: device copy of the schedule built for these
 * lengths (device context_lens must equal the host lengths it was built
 * from; blocks beyond a device length are masked, blocks the schedule does
 * not name are not read).  workspace: device buffer of at least
 * info->workspace_bytes (may be NULL when that is 0).  Other arguments as
 * for kvp_paged_attention_decode. */
kvp_status kvp_paged_attention_decode_scheduled(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, const int32_t* sched, const kvp_schedule_info* info, void* out,
    void* workspace, size_t workspace_bytes, kvp_stream_t stream);

/* ---- Several new tokens per sequence: chunked prefill, verification (device)
 * "KV-Cache Optimization Techniques", section "Cache-Aware Scheduling": long
 * prompts are processed in chunks against the cache.  Sequence b holds
 * n_b = context_lens[b] tokens, the last q_len_b = q_start[b+1] - q_start[b]
 * of which are its chunk, already written to its pages (kvp_kv_append).
 * Query row q_start[b] + i (0 <= i < q_len_b) sits at position
 * n_b - q_len_b + i and attends to positions 0 .. n_b - q_len_b + i (causal),
 * eq. 1 over those positions, query head j through KV head j / g:
 *   q, out        [N][H_q][D] bfloat16, N = q_start[B]; rows in position order;
 *   q_start       [B + 1] int32 device array, q_start[0] = 0, nondecreasing;
 *   max_q_len     host bound on every q_len_b (rows beyond it are not computed);
 *   max_context_len  host bound on context_lens, as for decode.
 * A row whose position would be negative (q_len_b > n_b) gives 0.  Scores,
 * softmax and sums are float32; out is rounded to bfloat16.  No workspace.
 * Reads every pool format (quantized pools as for decode, with the same
 * float16 operands). */
kvp_status kvp_paged_attention_prefill(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, void* out, kvp_stream_t stream);

/* ---- Multi-query attention along a longest-first order (host + device) ----
 * The same section ("Cache-Aware Scheduling"): the chunks of one batch see
 * caches of very different lengths, so the workgroups of the call above run
 * for very different times, and in grid order the longest can start last
 * and leave the device idle at the end.  A caller who knows the lengths on
 * the host can build an order that starts the costliest workgroups first:
 *   - the call's workgroups (units) are those of kvp_paged_attention_prefill
 *     for the same pool, num_seqs, num_q_heads, max_blocks, max_q_len and
 *     max_context_len; a unit's cost is the number of 64-key blocks its last
 *     query row sees, plus one; units with no query row are left out;
 *   - (sequence, KV head) items go to the eight XCDs (workgroup position
 *     i runs on XCD i mod 8), costliest item first, each to the XCD with the
 *     least cost so far, so that all units of an item share one L2; when
 *     that would leave one XCD more than 1.2 times the mean cost (fewer items
 *     than XCDs, or a few dominant ones), the units are shared out the same
 *     way instead, costliest first;
 *   - each XCD runs its units costliest first: entry 8r + x of the order is
 *     the r-th unit of XCD x, or -1 when XCD x has fewer than r + 1 units.
 * Results are bit-identical to the unordered call: each unit computes the
 * same rows the same way. */

/* Upper bound of the order's length (entries) for these arguments, any lengths. */
kvp_status kvp_prefill_schedule_bound(const kvp_pool* pool, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_blocks, int32_t max_q_len,
                                      int32_t max_context_len, int64_t* max_entries);
/* Build the order (host).  q_start: host copy of the B + 1 chunk offsets
 * (q_start[0] = 0, nondecreasing); context_lens: host copy of the B lengths
 * (>= 0); the other arguments as the call will get them (KVP_E_INVAL /
 * KVP_E_UNSUPPORTED as for that call).  *entries receives the order's length
 * (a multiple of 8); sched is a host buffer of capacity int32 entries, and
 * KVP_E_INVAL with *entries set is returned when that is too few. */
kvp_status kvp_prefill_schedule(const kvp_pool* pool, const int32_t* q_start,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_blocks, int32_t max_q_len,
                                int32_t max_context_len, int32_t* sched, int64_t capacity,
                                int64_t* entries);
/* kvp_paged_attention_prefill with its workgroups in a built order: sched is
 * a device copy of the entries entries (entries = 0 launches nothing).
 * Entries outside [0, units) are skipped; an order built for other lengths
 * or arguments still reads and writes only in bounds, but rows of units it
 * does not name are not written. */
kvp_status kvp_paged_attention_prefill_scheduled(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, const int32_t* sched,
    int64_t entries, void* out, kvp_stream_t stream);

/* ---- Decode in two phases (device) -----------------------------------------
 * The same attention as kvp_paged_attention_decode, with its two kernels
 * exposed separately: the split kernel writes one normalized partial per
 * (sequence, query head, split) and kvp_lse_merge combines them.  A caller
 * that spreads one sequence's pages over several devices gathers the partial
 * buffers and merges them the same way ("KV Cache Optimization" glossary:
 * splitting the cache across GPUs and gathering for attention).
 *
 * Partials buffer layout, for rows = num_seqs * H_q and S splits (row index
 * b*H_q + j, split s):
 *   o[row][s][D]  float32 at byte 0: sum_t p_t v_t / sum_t p_t over the split;
 *   ml[row][s][2] float32 at byte offset align256(rows*S*D*4):
 *       ml[..][0] = m, the largest score of the split in base-2 units
 *                   (score * scale * log2 e); -inf when the split is empty;
 *       ml[..][1] = l = sum_t 2^(score_t*log2e - m); 0 when the split is empty.
 * kvp_decode_partials_bytes gives the byte size and the split count S the
 * planner picks for these arguments (num_splits_req <= 0: automatic). */
kvp_status kvp_decode_partials_bytes(const kvp_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_context_len, int32_t num_splits_req,
                                     int32_t* num_splits, size_t* bytes);
/* Split kernel only; every partial of the layout above is written (empty
 * splits too).  *num_splits (may be NULL) receives S.  partials is a device
 * buffer of at least kvp_decode_partials_bytes bytes; KVP_E_INVAL otherwise. */
kvp_status kvp_paged_attention_decode_partials(
    const kvp_pool* pool, const void* q, const void* k_pool, const void* v_pool,
    const void* k_meta, const void* v_meta, const int32_t* block_tables, int32_t max_blocks,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    float scale, int32_t num_splits_req, void* partials, size_t partials_bytes,
    int32_t* num_splits, kvp_stream_t stream);
/* Log-sum-exp merge: out[row][:] = sum_s w_s o_s / sum_s w_s with
 * w_s = l_s 2^(m_s - max_s m_s), rounded to bfloat16; rows whose splits are
 * all empty give 0.  head_dim is 64 or 128; out is [rows][D] bfloat16. */
kvp_status kvp_lse_merge(const void* partials, int32_t rows, int32_t num_splits, int32_t head_dim,
                         void* out, kvp_stream_t stream);

/* ---- Measurement: streaming-read ceiling (device) ---------------------------
 * Decode reads every (page, KV head) tile of K and V once per step and is
 * bound by memory bandwidth ("KV Cache Optimization" glossary, section
 * "Memory-Bound Operation").  This probe reads the same pattern with no
 * arithmetic: for each of n_chunks entries of chunk_ids (device int32 array),
 * chunk chunk_ids[i] (chunk_bytes contiguous bytes at chunk_ids[i] *
 * chunk_bytes) of pool_a and of pool_b, both device buffers of at least
 * pool_bytes; with the decode kernels' loads (16 bytes per lane, non-temporal
 * hint), chunks_in_flight (1, 2, 4 or 8; not 8 with 8 KiB chunks) chunks per
 * wavefront in flight, num_waves wavefronts each taking a contiguous share of
 * the list (four per workgroup).  An id outside the buffers reads
 * chunk 0.  sink: device array of num_waves * 64 uint32 that receives a fold
 * of the bytes read (its value has no meaning).  chunk_bytes is 1024, 2048,
 * 4096 or 8192 (KVP_E_UNSUPPORTED otherwise).  Bytes read: 2 * n_chunks *
 * chunk_bytes. */
kvp_status kvp_probe_read_chunks(const void* pool_a, const void* pool_b, size_t pool_bytes,
                                 const int32_t* chunk_ids, int32_t n_chunks, int32_t chunk_bytes,
                                 int32_t chunks_in_flight, int32_t num_waves, uint32_t* sink,
                                 kvp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVP_H */
