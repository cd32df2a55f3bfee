/*
 * libattn: fused causal grouped-query attention for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer named "device" is GPU memory on the current HIP device;
 * "host" pointers are read during the call only.  The caller owns every buffer:
 * the library never allocates or frees memory and never copies a layout.  Every
 * call is asynchronous on the given stream (a hipStream_t passed as void*, NULL
 * for the default stream) and never synchronises.  On any status other than
 * ATTN_OK nothing has been launched and no output has been touched.
 *
 * Method.  Scaled dot-product attention softmax(scale * Q K^T + mask) V computed
 * without materialising the score matrix, as the fused full-attention path of
 * the page "Gemma4 FFPA attention backend support for accelerating Gemma4-family
 * training" (sections Integration and Debugging notes) does in place of the
 * unfused path that builds the S x S matrix.  The eligibility gate of that page
 * (section Integration: head_dim 512, 16-bit floats, no dropout, a given scale)
 * becomes the argument checks below; unsupported cases return
 * ATTN_ERR_UNSUPPORTED so that the caller can fall back, as the page does.
 *
 * Conventions shared by every call:
 *   - bf16 tensors: last (head_dim) dimension contiguous; other strides are in
 *     elements, non-negative multiples of 8; base pointers 16-byte aligned.
 *   - Grouped-query heads: query head h reads key/value head h / (Hq / Hkv)
 *     (the repeat-KV mapping of the first page's Debugging notes).
 *   - Mask: key j is visible from query i when both are inside the sequence
 *     (i, j < len), j <= i when causal, and j > i - window when window > 0.
 *   - A query row with no visible key yields O = 0 and LSE = 0, never NaN
 *     (page "flex_attention + paged KV + CUDA graphs vs vLLM", section "What
 *     broke correctness and had to be dropped").
 *   - Padded rows (positions at or past a sequence's length) of O, dQ and LSE,
 *     and padded keys of dK and dV, are written as exact zeros.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,  /* null pointer, bad shape, stride or alignment */
    ATTN_ERR_UNSUPPORTED = 2,  /* head_dim, window without causal, ... : caller falls back */
    ATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes query */
    ATTN_ERR_HIP = 4           /* a HIP runtime call failed; see attn_last_hip_error() */
} attn_status;

/* Element types.  Attention tensors (Q, K, V, O, dO, dQ, dK, dV, caches) are 16-bit:
 * bfloat16 or IEEE half, both admitted by the first page's gate (section Integration);
 * some outputs can also be kept in fp32. */
enum { ATTN_DTYPE_BF16 = 0, ATTN_DTYPE_F32 = 1, ATTN_DTYPE_F16 = 2 };

/* A bf16 tensor: device pointer plus element strides of the batch, sequence and
 * head dimensions (the head_dim dimension is contiguous).  For packed
 * (cu_seqlens) rows stride_b is ignored. */
typedef struct {
    void* ptr;
    int64_t stride_b;
    int64_t stride_s;
    int64_t stride_h;
} attn_tensor;

/* Sizes of one attention call.
 *   B      batch (number of sequences)
 *   S      sequence capacity: the padded length for dense and pad_mask inputs,
 *          the longest sequence for cu_seqlens inputs
 *   total  packed row count (cu_seqlens[B]); only read with cu_seqlens
 *   Hq     query heads; Hkv key/value heads; Hq % Hkv == 0
 *   D      head_dim: 256 or 512
 *   dtype  element type of every tensor of the call: ATTN_DTYPE_BF16 or
 *          ATTN_DTYPE_F16 (products accumulate in fp32 either way) */
typedef struct {
    int32_t B, S, total, Hq, Hkv, D, dtype;
} attn_shape;

/*
 * attn_fwd: O = softmax(scale * Q K^T + mask) V and the row log-sum-exp.
 *
 * Layouts: dense or pad_mask inputs are (B, S, H, D); with cu_seqlens they are
 * packed (total, H, D), sequence b owning rows cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *   q, o        Hq heads; k, v Hkv heads (o is written)
 *   lse         device fp32, written: (B, Hq, S) contiguous, or (Hq, total) for
 *               cu_seqlens; natural-log log-sum-exp of the scaled visible scores
 *   scale       multiplies Q K^T (must be finite and > 0)
 *   causal      0 or 1
 *   window      0 for none; W > 0 keeps keys j > i - W and requires causal
 *   softcap     0 for none; cap > 0 replaces every scaled score s by
 *               cap * tanh(s / cap) before the mask (the tanh soft-capping that
 *               the first page's gate sends to the eager path, section
 *               Integration); must be finite and >= 0
 *   cu_seqlens  device int32 (B+1), or NULL
 *   pad_mask    device uint8 (B, S), row-major, 1 = valid; each row must be a
 *               prefix of ones (right padding); or NULL.  At most one of
 *               cu_seqlens and pad_mask may be given.  Their contents are not
 *               checked (except in debug mode, see attn_debug); lengths are
 *               clamped to [0, S] so no access leaves the buffers.
 *   workspace   device scratch of at least attn_fwd_workspace_bytes(shape,
 *               varlen) bytes (0 for dense inputs), 256-byte aligned
 * The first page's Results section records that the forward's outputs are kept
 * for the backward rather than recomputed; attn_bwd takes O and LSE from here.
 */
attn_status attn_fwd(const attn_shape* shape,
                     attn_tensor q, attn_tensor k, attn_tensor v,
                     float scale, int causal, int window, float softcap,
                     const int32_t* cu_seqlens, const uint8_t* pad_mask,
                     attn_tensor o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd: gradients of sum(O * dO) with respect to Q, K and V.
 *
 * q, k, v, scale, causal, window, softcap, cu_seqlens, pad_mask and the layouts
 * are as in attn_fwd, and o and lse must be that call's outputs.  Under a softcap
 * the stored dS and the gradients include the cap's derivative 1 - tanh^2.  dq (Hq heads), dk
 * and dv (Hkv heads, summed over the Hq/Hkv query heads that share them) are
 * written in the same layouts as q, k and v.  The page "Root cause analysis:
 * Gemma4 sliding-window BF16 cuDNN SDPA NaN on H100" (Debug and validation
 * results) traces a failure where finite dO produced non-finite dQ/dK/dV; here
 * every gradient of finite inputs is finite.
 *   workspace  at least attn_bwd_workspace_bytes(shape, varlen, causal, window)
 *              bytes: row statistics (fp32 per query row and head) and dS =
 *              P * (dP - delta) in bf16 for every visible (query, key) pair, kept
 *              between the dK/dV pass and the dQ pass (in 32-key x 128-row blocks,
 *              about B * Hq * S * S bytes for causal attention, less with a window or
 *              with cu_seqlens rows; see the workspace queries below)
 */
attn_status attn_bwd(const attn_shape* shape,
                     attn_tensor q, attn_tensor k, attn_tensor v,
                     attn_tensor o, const float* lse, attn_tensor dout,
                     float scale, int causal, int window, float softcap,
                     const int32_t* cu_seqlens, const uint8_t* pad_mask,
                     attn_tensor dq, attn_tensor dk, attn_tensor dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Sizes of one chunk pair of a sequence split into chunks (ring context parallelism).
 *   B       batch
 *   Sq      query rows of the query chunk; Sk key/value rows of the key/value chunk
 *           (each below 2^28)
 *   Hq, Hkv, D, dtype as in attn_shape */
typedef struct {
    int32_t B, Sq, Sk, Hq, Hkv, D, dtype;
} attn_chunk_shape;

/*
 * attn_fwd_chunk: partial attention of one query chunk against one key/value chunk of
 * the same sequences.  The ring path of the page "Gemma4 FFPA attention backend support
 * for accelerating Gemma4-family training" (section Integration) runs the fused kernel on
 * full-attention chunks; a rank holds one query chunk, sees the key/value chunks one ring
 * step at a time, and combines the partial results with attn_lse_merge.
 *
 * Query row i of the chunk sits at sequence position q_pos0 + i and key row j at
 * k_pos0 + j (both >= 0); the mask compares positions: key visible when k_pos <= q_pos
 * (causal) and k_pos > q_pos - window (window > 0, requires causal).
 *   q      dense bf16 (B, Sq, Hq, D); k, v dense bf16 (B, Sk, Hkv, D)
 *   o      (B, Sq, Hq, D), written, element type o_dtype: ATTN_DTYPE_F32 for a partial
 *          that attn_lse_merge will combine (the row is then rounded to 16 bits once,
 *          at the last merge), or the inputs' dtype for a pair that is the row's only one
 *   lse    device fp32 (B, Hq, Sq) contiguous, written: natural-log log-sum-exp of the
 *          row's scaled visible scores in this chunk, or -inf for a row that sees no
 *          key of the chunk (its O is 0); -inf is the identity of attn_lse_merge
 * No workspace.  Other conventions as attn_fwd.
 */
attn_status attn_fwd_chunk(const attn_chunk_shape* shape,
                           attn_tensor q, attn_tensor k, attn_tensor v,
                           float scale, int causal, int window, float softcap,
                           int64_t q_pos0, int64_t k_pos0,
                           attn_tensor o, int o_dtype, float* lse, void* stream);

/*
 * attn_bwd_chunk: the gradient parts of one chunk pair.  o and lse are the query rows'
 * final results, merged over every key chunk the rows attend to (not this pair's
 * partial), and dout is the gradient of the loss with respect to that final O.  With
 * P = exp(scale Q K^T - lse) on the pair's visible entries (0 elsewhere) and
 * dS = P * (dO V^T - rowsum(dO * o)), it writes
 *   dq  (B, Sq, Hq, D):  scale dS K,
 *   dk, dv (B, Sk, Hkv, D):  scale dS^T Q and P^T dO, summed over each kv head's
 *       query heads.
 * Summed over the key chunks of a query chunk (dq) and over the query chunks of a key
 * chunk (dk, dv), the parts are the gradients of attention over the whole sequence.
 *   grad_dtype  ATTN_DTYPE_F32: dq, dk, dv are fp32 accumulators (zeroed by the caller
 *               before a chunk's first pair) and the pair's parts are added to them, so a
 *               ring step needs no separate sum; a pair with no visible (query, key) pair
 *               launches nothing.  The inputs' dtype: the parts are written in it, not
 *               accumulated; a row that sees no key of the pair gets dq = 0 and a key that
 *               no row of the pair sees gets dk = dv = 0.
 *   workspace  at least attn_bwd_chunk_workspace_bytes(shape, causal, window, q_pos0,
 *              k_pos0) bytes, 256-byte aligned (row statistics and dS blocks, as attn_bwd)
 * Other conventions as attn_bwd.
 */
attn_status attn_bwd_chunk(const attn_chunk_shape* shape,
                           attn_tensor q, attn_tensor k, attn_tensor v,
                           attn_tensor o, const float* lse, attn_tensor dout,
                           float scale, int causal, int window, float softcap,
                           int64_t q_pos0, int64_t k_pos0,
                           attn_tensor dq, attn_tensor dk, attn_tensor dv, int grad_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_lse_merge: combine two partial results of the same query rows over disjoint key
 * sets (the ring path's per-step results, first page, section Integration), in place:
 *   L = ln(e^lse + e^lse_part),  o = e^(lse - L) o + e^(lse_part - L) o_part,  lse = L.
 * A partial with LSE = -inf contributes nothing (its O is not read into the result);
 * two such partials give o = 0 and lse = -inf.
 *   o, o_part       fp32 (B, S, H, D) with attn_tensor strides (element strides,
 *                   multiples of 8, 16-byte aligned); o is updated; the two must not
 *                   overlap
 *   lse, lse_part   device fp32 (B, H, S) contiguous; lse is updated
 *   out             (B, S, H, D) of type out_dtype (ATTN_DTYPE_BF16 or ATTN_DTYPE_F16):
 *                   if out.ptr is not NULL, the merged o rounded to it (round to nearest
 *                   even) is also written there, for the last merge of a row
 *   D               128, 256 or 512
 */
attn_status attn_lse_merge(int32_t B, int32_t S, int32_t H, int32_t D,
                           attn_tensor o, float* lse,
                           attn_tensor o_part, const float* lse_part,
                           attn_tensor out, int out_dtype, void* stream);

/*
 * attn_fwd_chunk_merge: attn_fwd_chunk of one chunk pair with its partial merged straight
 * into a running result, in one pass (the same ring step as attn_fwd_chunk followed by
 * attn_lse_merge, first page, section Integration, without the fp32 partial going through
 * memory).  With (O_p, L_p) the pair's partial as attn_fwd_chunk defines it:
 *   lse' = ln(e^lse + e^L_p),  o' = e^(lse - lse') o + e^(L_p - lse') O_p.
 * The result equals attn_fwd_chunk (o_dtype ATTN_DTYPE_F32) then attn_lse_merge bit for
 * bit.  A running row with lse = -inf has weight 0 and its o is not read, so a ring may
 * start from lse = -inf everywhere and o uninitialised (the first pair's call then writes
 * its partial exactly).
 *   q, k, v, shape, scale, causal, window, softcap, q_pos0, k_pos0   as attn_fwd_chunk
 *   o     fp32 (B, Sq, Hq, D) with attn_tensor strides, read and written
 *   lse   device fp32 (B, Hq, Sq) contiguous, read and written
 *   out   (B, Sq, Hq, D) in the inputs' dtype: if out.ptr is not NULL, the merged o rounded
 *         to it (round to nearest even) is also written there, for the row's last pair; it
 *         must not overlap o
 * No workspace.  Each call is one kernel; calls on one stream merge in order.
 */
attn_status attn_fwd_chunk_merge(const attn_chunk_shape* shape,
                                 attn_tensor q, attn_tensor k, attn_tensor v,
                                 float scale, int causal, int window, float softcap,
                                 int64_t q_pos0, int64_t k_pos0,
                                 attn_tensor o, float* lse, attn_tensor out, void* stream);

/* Sizes of one paged decode call.
 *   B                 sequences, one query token each
 *   Hq, Hkv, D        heads and head_dim (D = 128)
 *   page_size         tokens per cache page (16)
 *   num_pages         pages in the cache pool
 *   max_pages_per_seq columns of block_table */
typedef struct {
    int32_t B, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq;
    int32_t dtype;  /* q, caches and o: ATTN_DTYPE_BF16 or ATTN_DTYPE_F16 */
} attn_decode_shape;

/*
 * paged_decode: one query token per sequence against a paged KV cache
 * (page "flex_attention + paged KV + CUDA graphs vs vLLM", Architecture notes:
 * a paged cache plus a page table mapping logical to physical pages; section
 * "What each option did": the per-block page-table indirection that a random
 * page placement makes necessary).
 *
 *   q            device 16-bit (shape->dtype) (B, Hq, D); element strides q_stride_b,
 *                q_stride_h
 *   k_cache,     device 16-bit (num_pages, page_size, Hkv, D); attn_tensor strides
 *   v_cache      are (page, slot, head) in elements; a slot stride of 2^26 elements
 *                or more returns ATTN_ERR_UNSUPPORTED
 *   block_table  device int32 (B, max_pages_per_seq), row-major: logical page p of
 *                sequence b lives in physical page block_table[b][p].  Entries a
 *                sequence does not use are never read.  An entry outside
 *                [0, num_pages) is clamped into range (no out-of-bounds read).
 *   ctx_lens     device int32 (B): tokens in each sequence's cache, including the
 *                current one; the query sits at position ctx_lens[b]-1 and sees
 *                every token t < ctx_lens[b].  Clamped to
 *                [0, max_pages_per_seq * page_size]; 0 gives O = 0.
 *   softcap      as for attn_fwd (0: none)
 *   o            device 16-bit (B, Hq, D), written; strides o_stride_b, o_stride_h
 *   workspace    at least paged_decode_workspace_bytes(shape) bytes; used only when the
 *                call splits contexts into chunks (below), and always checked
 * Two schedules, same results within rounding: when B * Hkv >= 256 and
 * max_pages_per_seq * page_size <= 8192, one kernel gives each (sequence, kv head) one
 * workgroup that covers the whole context and writes o; otherwise a first kernel scores
 * 512-token chunks into the workspace and a second merges them into o.  A row's result is
 * deterministic for a given shape, but the same row in calls of different B (or table width)
 * may differ in its last bits.
 */
attn_status paged_decode(const attn_decode_shape* shape,
                         const void* q, int64_t q_stride_b, int64_t q_stride_h,
                         attn_tensor k_cache, attn_tensor v_cache,
                         const int32_t* block_table, const int32_t* ctx_lens,
                         float scale, float softcap,
                         void* o, int64_t o_stride_b, int64_t o_stride_h,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_noalloc: paged_decode for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  It takes no
 * workspace: the chunk partials (when the call splits contexts into chunks, see paged_decode)
 * live in a fixed device array inside the library, of
 * paged_decode_noalloc_max_bytes() bytes (16 MiB) on every GPU it runs on, held until the
 * process ends.  The call allocates nothing and frees nothing.
 *   Arguments, layouts, results and errors are those of paged_decode without workspace and
 *   workspace_bytes; the results equal paged_decode's bit for bit.  A shape whose
 *   paged_decode_workspace_bytes(shape) exceeds the fixed array returns ATTN_ERR_WORKSPACE
 *   before anything is launched.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   (other streams, other threads, other processes do not share it) race and give wrong
 *   results.  Calls on one stream run one after the other and do not.
 * The first call on each device looks the array's address up (hipGetSymbolAddress), which may
 * load the library's code object on that device; it launches nothing extra.
 */
attn_status paged_decode_noalloc(const attn_decode_shape* shape,
                                 const void* q, int64_t q_stride_b, int64_t q_stride_h,
                                 attn_tensor k_cache, attn_tensor v_cache,
                                 const int32_t* block_table, const int32_t* ctx_lens,
                                 float scale, float softcap,
                                 void* o, int64_t o_stride_b, int64_t o_stride_h, void* stream);

/* Size in bytes of paged_decode_noalloc's fixed device array. */
size_t paged_decode_noalloc_max_bytes(void);

/*
 * paged_decode_contiguous: paged_decode for caches whose every sequence holds consecutive pages
 * (the BLOCKS_ARE_CONTIGUOUS setting of the page "flex_attention + paged KV + CUDA graphs vs
 * vLLM", section "What each option did": safe there because a fresh batch reserves its pages in
 * order, and faster because no per-block page-table lookup is made).  Instead of a block table
 * it takes
 *   first_page   device int32 (B): logical page p of sequence b is physical page
 *                first_page[b] + p.  Ids outside [0, num_pages) are clamped into range.
 * shape->max_pages_per_seq still bounds ctx_lens (clamped to max_pages_per_seq * page_size)
 * and sizes the workspace (paged_decode_workspace_bytes).  Other arguments, layouts and
 * results as paged_decode; the result equals paged_decode's bit for bit when block_table[b][p]
 * = first_page[b] + p.  In debug mode (attn_debug) a sequence whose pages leave the pool
 * returns ATTN_ERR_INVALID_ARG.
 */
attn_status paged_decode_contiguous(const attn_decode_shape* shape,
                                    const void* q, int64_t q_stride_b, int64_t q_stride_h,
                                    attn_tensor k_cache, attn_tensor v_cache,
                                    const int32_t* first_page, const int32_t* ctx_lens,
                                    float scale, float softcap,
                                    void* o, int64_t o_stride_b, int64_t o_stride_h,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_append: write the n_tokens newest tokens of each sequence into its cache pages:
 * token i of sequence b (k_new/v_new row (b, i)) goes to logical position
 * ctx_lens[b] - n_tokens + i, i.e. ctx_lens counts the appended tokens, as it does for
 * paged_decode (which takes the current token's K/V from the cache).  Positions below 0 are
 * skipped, as are positions whose table entry is outside [0, num_pages).
 *   shape       B, Hkv, D (128, 256 or 512), page_size, num_pages, max_pages_per_seq and
 *               dtype as for paged_decode (Hq is not used)
 *   k_new,      device (B, n_tokens, Hkv, D) with attn_tensor strides (batch, token, head)
 *   v_new
 *   k_cache,    device (num_pages, page_size, Hkv, D), strides (page, slot, head); written
 *   v_cache
 *   block_table, ctx_lens  as for paged_decode (ctx_lens clamped the same way)
 * Sequences whose positions map to the same page slot race; a table that gives each
 * sequence its own pages (as a page pool does) has none.
 */
attn_status paged_kv_append(const attn_decode_shape* shape, int32_t n_tokens,
                            attn_tensor k_new, attn_tensor v_new,
                            attn_tensor k_cache, attn_tensor v_cache,
                            const int32_t* block_table, const int32_t* ctx_lens, void* stream);

/*
 * paged_kv_gather: the first n_tokens logical tokens of each sequence's cache, contiguous:
 * row (b, t) of k_out/v_out is token t of sequence b for t < ctx_lens[b], zeros for
 * t >= ctx_lens[b] or a table entry outside [0, num_pages).  With attn_fwd_chunk over the
 * gathered keys (k_pos0 = 0) this is the paged prefill of a chunk of new queries.
 *   k_out, v_out  device (B, n_tokens, Hkv, D) with attn_tensor strides; written
 * Other arguments as for paged_kv_append.
 */
attn_status paged_kv_gather(const attn_decode_shape* shape, int32_t n_tokens,
                            attn_tensor k_cache, attn_tensor v_cache,
                            const int32_t* block_table, const int32_t* ctx_lens,
                            attn_tensor k_out, attn_tensor v_out, void* stream);

/*
 * Decode-step graphs per batch bucket: one captured HIP graph of a decode step (optionally the
 * append of the current token's K/V, then paged_decode) for each batch size of a bucket list,
 * all over the same fixed buffers and one shared workspace, so that a serving loop replays a
 * graph instead of launching kernels (page "flex_attention + paged KV + CUDA graphs vs vLLM",
 * Architecture notes: one graph per bucket in [1, 2, 4, 8, ..., max_bs]; section "What each
 * option did": graph capture took that decode from about 420 to 4279 tokens/s).
 *
 * paged_decode_graphs_create
 *   shape        sizes of the largest bucket: shape->B is the buffers' row count
 *   buckets      host int32 (n_buckets): increasing batch sizes in [1, shape->B]
 *   q, k_cache, v_cache, block_table, ctx_lens, scale, softcap, o and strides
 *                as for paged_decode; the graphs keep these device addresses
 *   k_new, v_new device (B, 1, Hkv, D) with attn_tensor strides: the current token's K and V,
 *                appended by each replay before its decode (as paged_kv_append with n_tokens
 *                = 1); k_new.ptr = v_new.ptr = NULL for a graph of the decode alone
 *   workspace    at least paged_decode_workspace_bytes(shape) bytes, shared by every graph
 *   stream       a created stream (not NULL) to capture on; nothing runs during creation
 *   out          receives the graph set (free it with paged_decode_graphs_destroy)
 * The graph of bucket n processes rows 0 .. n-1 of the buffers.  In debug mode the metadata is
 * checked once, here.  Creating graphs allocates host and device memory (hipGraphInstantiate).
 *
 * paged_decode_graphs_launch: replays, on `stream`, the graph of the smallest bucket >= B
 * (0 <= B <= largest bucket; B = 0 launches nothing) and stores that bucket in *bucket if
 * bucket is not NULL.  Rows B .. bucket-1 are processed too: a caller gives them ctx_lens 0
 * (their O is then 0 and nothing is appended for them) or ignores them.  A replay equals the
 * eager step on the bucket's rows bit for bit.  The replay reads
 * whatever the buffers hold when it runs.  Replays of one graph set share its workspace:
 * overlapping replays (other streams) race.
 */
typedef struct attn_decode_graphs attn_decode_graphs;

attn_status paged_decode_graphs_create(const attn_decode_shape* shape,
                                       const int32_t* buckets, int32_t n_buckets,
                                       const void* q, int64_t q_stride_b, int64_t q_stride_h,
                                       attn_tensor k_new, attn_tensor v_new,
                                       attn_tensor k_cache, attn_tensor v_cache,
                                       const int32_t* block_table, const int32_t* ctx_lens,
                                       float scale, float softcap,
                                       void* o, int64_t o_stride_b, int64_t o_stride_h,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       attn_decode_graphs** out);
attn_status paged_decode_graphs_launch(const attn_decode_graphs* graphs, int32_t B, void* stream,
                                       int32_t* bucket);
void paged_decode_graphs_destroy(attn_decode_graphs* graphs);

/* Sizes of one paged prefill call.
 *   B                 sequences
 *   max_q             most new query rows of one sequence
 *   total_q           packed query rows, cu_q[B]
 *   Hq, Hkv, D        heads and head_dim (256 or 512)
 *   dtype             q, caches and o: ATTN_DTYPE_BF16 or ATTN_DTYPE_F16
 *   page_size         tokens per cache page (16)
 *   num_pages         pages in the cache pool
 *   max_pages_per_seq columns of block_table */
typedef struct {
    int32_t B, max_q, total_q, Hq, Hkv, D, dtype;
    int32_t page_size, num_pages, max_pages_per_seq;
} attn_paged_shape;

/*
 * attn_fwd_paged: causal attention of each sequence's new query tokens against that sequence's
 * whole paged K/V cache, the cache read through the block table inside the kernel (no gathered
 * copy).  A sequence with one new token is a decode row, so one call serves a serving step that
 * mixes prompt chunks and decode tokens: the interleaving of prefill and decode in one step that
 * the page "flex_attention + paged KV + CUDA graphs vs vLLM" (section "What's left on the
 * table", chunked prefill) names as the missing piece, over the paged cache and page table of
 * its Architecture notes.
 *   q            device 16-bit, packed (total_q, Hq, D): sequence b's new tokens are rows
 *                cu_q[b] .. cu_q[b+1]-1 (attn_tensor stride_b is ignored)
 *   k_cache,     device 16-bit (num_pages, page_size, Hkv, D), strides (page, slot, head) in
 *   v_cache      elements; they already hold the new tokens' K and V (paged_kv_append).  A slot
 *                stride of 2^26 elements or more returns ATTN_ERR_UNSUPPORTED.
 *   block_table  device int32 (B, max_pages_per_seq) as for paged_decode; entries outside
 *                [0, num_pages) are clamped, entries past a sequence's tokens are not read
 *   cu_q         device int32 (B+1): query row offsets, non-decreasing, cu_q[B] = total_q;
 *                n_b = cu_q[b+1] - cu_q[b] is clamped to [0, max_q]
 *   ctx_lens     device int32 (B): tokens in sequence b's cache, the n_b new ones included,
 *                clamped to [0, max_pages_per_seq * page_size].  Query row i of sequence b sits
 *                at position ctx_lens[b] - n_b + i and sees key t when t <= that position and,
 *                with window > 0, t > position - window.  A row at a negative position
 *                (ctx_lens[b] < n_b) sees no key.
 *   scale, softcap  as for attn_fwd; window 0 (none) or > 0
 *   o            device 16-bit, packed (total_q, Hq, D), written
 *   lse          device fp32 (Hq, total_q) contiguous, written
 * No workspace: one kernel launch, which reads cu_q, ctx_lens and the table itself.  Rows with no visible key get O = 0 and LSE = 0, as in attn_fwd.  Every other row's O and
 * LSE equal those of attn_fwd_chunk over the sequence's cached keys 0 .. ctx_lens[b]-1 laid out
 * densely, with q_pos0 = ctx_lens[b] - n_b and k_pos0 = 0.
 */
attn_status attn_fwd_paged(const attn_paged_shape* shape,
                           attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                           const int32_t* block_table, const int32_t* cu_q, const int32_t* ctx_lens,
                           float scale, int window, float softcap,
                           attn_tensor o, float* lse, void* stream);

/*
 * attn_fwd_paged_split: attn_fwd_paged for a serving step whose decode rows sit beside prompt
 * chunks (the mixed prefill / decode step of the page "flex_attention + paged KV + CUDA graphs
 * vs vLLM", section "What's left on the table").  A decode row (a sequence with one new token)
 * whose visible keys span more than 8 tiles of 32 keys is cut into at most 16 pieces of whole
 * tiles, each computed by its own workgroup into the workspace; a second kernel combines a
 * row's pieces, in piece order, by log-sum-exp weighting (the combination of partial results
 * over disjoint key sets, as attn_lse_merge) and writes its O and LSE.  Without the split, a
 * decode row's one workgroup walks the whole context for 1/16 of a prompt tile's work.  The
 * split applies while the batch's (sequence, kv head) units number fewer than the 256 compute
 * units and some sequence can have one new token; the tiles are then dealt by the sequences'
 * work (new rows x cached keys, ranked on the device), heaviest first, and the pieces after them.
 * Arguments as attn_fwd_paged, and
 *   workspace  device, at least attn_fwd_paged_workspace_bytes(shape) bytes, 256-byte aligned
 *              (fp32 O and LSE per piece, B * Hq * 16 * (D + 1) * 4 bytes, and the sequences'
 *              order by work, B * 4 bytes, rounded up); its contents on return are unspecified;
 *              missing or too small: ATTN_ERR_WORKSPACE
 * Rows that are not split get exactly attn_fwd_paged's O and LSE (bit for bit); a split row's
 * O is the fp32 combination of its pieces' normalised O rounded once to 16 bits, equal to
 * attn_fwd_paged's within rounding.  Two launches; calls on one stream that share a workspace
 * are ordered by the stream.
 */
attn_status attn_fwd_paged_split(const attn_paged_shape* shape,
                                 attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                                 const int32_t* block_table, const int32_t* cu_q, const int32_t* ctx_lens,
                                 float scale, int window, float softcap,
                                 attn_tensor o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace sizes in bytes.  varlen: 0 dense, 1 pad_mask, 2 cu_seqlens; causal and
 * window as in the call.  Return 0 for arguments that the matching call would reject.
 * Each call computes its own requirement and the caller owns the memory, so one
 * workspace grown to the largest query can serve every call issued on one stream (the
 * page "[Reland] Add dist GEMM attention and FFN backend", section "Symmetric memory",
 * sizes its shared workspace the same way: every op states its need, the buffer grows to
 * the maximum, and serialised calls may reuse the same bytes).
 * Backward: for cu_seqlens rows each sequence's dS blocks take room for its own length,
 * bounded from `total` and S (about Hq * total * S bytes for causal attention instead of
 * B * Hq * S^2); dense and pad_mask rows take B * Hq times the longest sequence's room.  A
 * backward whose workspace would pass 128 GiB is refused (0 here, ATTN_ERR_UNSUPPORTED
 * from the call): split such sequences into chunk pairs (attn_bwd_chunk), whose workspace
 * is bounded by the chunk sizes. */
size_t attn_fwd_workspace_bytes(const attn_shape* shape, int varlen);
size_t attn_bwd_workspace_bytes(const attn_shape* shape, int varlen, int causal, int window);
size_t paged_decode_workspace_bytes(const attn_decode_shape* shape);
/* For attn_fwd_paged_split; 0 for a shape that it would reject. */
size_t attn_fwd_paged_workspace_bytes(const attn_paged_shape* shape);
/* For attn_bwd_chunk; 0 for arguments that it would reject. */
size_t attn_bwd_chunk_workspace_bytes(const attn_chunk_shape* shape, int causal, int window,
                                      int64_t q_pos0, int64_t k_pos0);

/* Debug mode: calls that take device-resident metadata (cu_seqlens, pad_mask, block tables,
 * ctx_lens) first check it on their stream and synchronise; inconsistent metadata (a mask that
 * is not a prefix, offsets that decrease or do not end at `total`, a length above S, a page id
 * outside the pool, a context longer than the table) returns ATTN_ERR_INVALID_ARG before any
 * other launch.  Outside debug mode the metadata is not checked (lengths, offsets and page ids
 * are clamped so that nothing is accessed outside the buffers).  attn_debug(on) sets the mode
 * for the process and returns the previous one; its initial value is 1 when the environment
 * variable ATTN_DEBUG is set to anything but "0".  A check synchronises its stream, so debug
 * mode is for eager calls, not for calls recorded into a graph. */
int attn_debug(int on);

/* Static string for a status code.  The codes follow the eligibility gate of the page
 * "Gemma4 FFPA attention backend support for accelerating Gemma4-family training" (section
 * Integration): a case the fused path does not take is reported (ATTN_ERR_UNSUPPORTED) so
 * that the caller can fall back, rather than computed some other way. */
const char* attn_status_str(attn_status status);

/* The hipError_t (as int) of the last ATTN_ERR_HIP on this thread, 0 if none. */
int attn_last_hip_error(void);

/* Kernel timing for benchmarks.  After attn_profile(1), every call made on this thread
 * records a HIP event pair on its own stream around each kernel it launches; after
 * attn_profile(0) it stops.  attn_profile_read() waits for the recorded events and
 * fills up to max_entries records (one per kernel name, in first-launch order) with the
 * launch count and the summed milliseconds, then forgets them; it returns the number of
 * records, or -1 after a HIP error.  Events come from a pool of at most 4096 pairs per
 * thread; launches beyond that are not timed.  Not for use under graph capture. */
typedef struct {
    const char* kernel;   /* static string */
    int launches;
    double total_ms;
} attn_kernel_time;

int attn_profile(int on);
int attn_profile_read(attn_kernel_time* out, int max_entries);

/* Softmax-reference restarts, for tests.  At head_dim 512 the forward fixes each row's
 * softmax reference from the first keys it sees and, when a later score exceeds it by more
 * than the 16-bit probability range allows, restarts the workgroup's key loop with raised
 * references (exact in real arithmetic; see the forward kernel).  After
 * attn_count_restarts(p) with p a device int32, every forward kernel launched from this
 * thread (attn_fwd, attn_fwd_chunk, attn_fwd_chunk_merge) atomically adds 1 to *p per
 * restart of one of its workgroups; attn_count_restarts(NULL) stops it.  Returns 0.  The
 * counter is the caller's memory and must stay valid while such calls run. */
int attn_count_restarts(int32_t* device_counter);

/* Roofline probes for benchmarks (not on the attention path): one launch, asynchronous on
 * `stream`, of a kernel that shows what a plain kernel reaches on this device, to set beside
 * the published MI355X peaks (dense bf16 matrix 2.5 PFLOP/s and HBM 8 TB/s, which assume the
 * peak engine clock).  The caller times it (HIP events on the stream).
 *   kind 0  matrix rate: 4 workgroups of 4 waves per compute unit, each wave `reps` rounds of
 *           8 independent v_mfma_f32_32x32x16_bf16 (32768 flop each); writes 1024 bytes per
 *           workgroup to buf (bytes >= compute units * 4096)
 *   kind 1  streaming read of the first `bytes` of buf (a multiple of 32, >= 4096)
 *   kind 2  streaming copy of the first half of buf's `bytes` to the second half
 * Returns ATTN_ERR_INVALID_ARG for a null or misaligned buf, too few bytes or another kind. */
attn_status attn_peak_probe(int kind, void* buf, size_t bytes, int reps, void* stream);

/* Library version, "major.minor.patch". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
