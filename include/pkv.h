/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on MI355X (gfx950).
 *
 * The operation (page 2, "FlashAttention + PageAttention joint tuning",
 * section 2.1): out = softmax(Q K^T * scale) V for every query row, reduced
 * tile by tile with an online softmax (same page, section 2.2).  K and V live
 * in fixed-size physical pages; each sequence reaches its pages through a
 * block table whose entry i holds the physical page of logical tokens
 * [i*P, (i+1)*P) (page 2, section 3.2; page 3, section 3.2: the page of token
 * t is table[t / P]).  Query heads share KV heads in contiguous groups of
 * G = H_q / H_kv (page 4, section 2.2, GQA): query head h reads KV head h / G.
 *
 * Data layout, shared by every call (one layer per call):
 *   k_cache, v_cache : [num_pages][H_kv][P][D] of desc->dtype, separate buffers.
 *                      One (page, head) block is P*D contiguous elements.
 *   block_table      : int32 [batch][block_table_stride], device memory.
 *   context_lens     : int32 [batch], device memory.
 *   slot             : page * P + offset (int32).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers; "host" ones are CPU
 *     memory.  The caller owns every buffer.  The library allocates no device
 *     memory (the one static device array of the allocation-free decode step
 *     comes with the loaded library), keeps no pointer after returning, and
 *     never synchronises (outside the PKV_CHECK debug mode below).
 *   - stream: a hipStream_t passed as void*; NULL is the null stream.  All
 *     device work is enqueued on it asynchronously.
 *   - Base pointers of device buffers must be 16-byte aligned.
 *   - Return value: PKV_OK (0) or a negative pkv_status.  Argument checks run
 *     on the host before any HIP call; on error nothing is enqueued and
 *     pkv_last_error() gives a message (per calling thread).
 *   - Supported shapes: page_size 16; head_dim 64 or 128; dtype f32, f16,
 *     bf16; H_q a multiple of H_kv with G in {1, 2, 4, 8, 16} (decode at
 *     G = 16 needs head_dim 128 and f16 or bf16 queries); the prefill call
 *     needs f16 or bf16 and head_dim 128.  fp8 caches (PKV_FP8_E4M3,
 *     PKV_FP8_E5M2) are read by the *_ex decode calls with head_dim 128 and
 *     f16 or bf16 queries; kv_append and gather_kv copy their bytes, and
 *     kv_append_quant fills them from wider types.
 *   - Contents of device tables (page ids, lengths, slots) are preconditions
 *     the host cannot see.  Kernels keep every memory access inside the
 *     buffers described by the arguments even when a precondition is broken;
 *     a decode or prefill row whose table entries or length are out of range
 *     is written as NaN.  pkv_validate_tables() checks host copies.
 *   - Debugging: with the environment variable PKV_CHECK set (to anything but
 *     "" or "0"; read at every call), each call that reads device tables
 *     (slots, block table, lengths, q_indptr) first copies them to the host
 *     on its stream, which synchronises the stream, and returns
 *     PKV_ERR_INVALID with a "PKV_CHECK: ..." message instead of launching
 *     when one of the preconditions above is broken.  A windowed decode
 *     checks only the pages it reads.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_VERSION 4

/*
 * Element types.  The fp8 types are the OCP 8-bit floats (E4M3 without
 * infinities, largest finite 448; E5M2 with IEEE infinities and NaNs, largest
 * finite 57344); page 1, section 4.1 and page 4, section 3.2 name them as KV
 * cache types.  An fp8 pool carries one fp32 scale: element = scale * value.
 */
typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3,
  PKV_FP8_E5M2 = 4
} pkv_dtype;

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* bad pointer, size or descriptor field */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, D, P, G) */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  PKV_ERR_HIP = -4          /* a HIP launch failed; see pkv_last_error() */
} pkv_status;

/* Describes one layer's K and V page pools (both have this shape and type). */
typedef struct pkv_cache_desc {
  int32_t num_pages;    /* physical pages in each pool */
  int32_t page_size;    /* tokens per page, P */
  int32_t num_kv_heads; /* H_kv */
  int32_t head_dim;     /* D */
  int32_t dtype;        /* pkv_dtype of K and V (and of Q and the output,
                           except for fp8 caches: see pkv_decode_opts) */
} pkv_cache_desc;

/*
 * Options of the *_ex decode, prefill and mixed-batch calls.  NULL options
 * mean: q_dtype = the cache dtype, unit scales, no window.
 *   q_dtype  : pkv_dtype of q and out.  Must equal desc->dtype for f32, f16
 *              and bf16 caches; PKV_F16 or PKV_BF16 for fp8 caches.
 *   k_scale, v_scale : fp8 caches only (1 otherwise): a K (V) element is
 *              k_scale (v_scale) times the stored fp8 value.  Finite, > 0.
 *   window   : 0 = every key.  window > 0: the query, at position L - 1 of a
 *              context of L keys, sees the keys t >= L - window (the window
 *              most recent, itself included) and the first `sink` keys,
 *              nothing else (page 4, section 2.3: a local sliding window
 *              mixed with a few global tokens; that page's mask with
 *              window_size W and global_tokens n opens exactly these keys of
 *              the last row for window = W / 2 + 1, sink = n).  Pages that
 *              hold no visible key are never read, and their block-table
 *              entries are not looked at.
 *   sink     : >= 0; ignored when window == 0.
 */
/* The prefill and mixed-batch calls take q_dtype and the scales; their
 * window and sink must be 0. */
typedef struct pkv_decode_opts {
  int32_t q_dtype;
  float k_scale;
  float v_scale;
  int32_t window;
  int32_t sink;
} pkv_decode_opts;

/* Library version (PKV_VERSION). */
int pkv_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

/*
 * kv_append -- write new tokens' K/V into their page slots (page 2, section
 * 5.2: pages for the next step are allocated ahead; the new token's K/V is
 * then stored in place).  For each i < n_tokens with s = slot_mapping[i] >= 0
 * and every KV head g:
 *     k_cache[s / P][g][s % P][:] = k_new[i][g][:]   (same for V)
 * A bitwise copy.  slot < 0 skips the token; a slot >= num_pages * P is also
 * skipped.  Two tokens with the same slot race (unspecified result).
 *   k_cache, v_cache : device, updated in place.
 *   k_new, v_new     : device, [n_tokens][H_kv][D] of desc->dtype.
 *   slot_mapping     : device int32 [n_tokens].
 * n_tokens == 0 is a no-op.
 */
int pkv_kv_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                  const void* k_new, const void* v_new, const int32_t* slot_mapping,
                  int32_t n_tokens, void* stream);

/*
 * gather_kv -- copy logical tokens [0, len) of one sequence into contiguous
 * k_out, v_out [len][H_kv][D] (device), following table_row (device int32,
 * ceil(len/P) entries; page 3, section 3.2 address rule).  Bitwise.  Used to
 * check the indexing path; a page id out of range yields NaN rows for f16,
 * bf16 and f32 alike.
 */
int pkv_gather_kv(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                  const int32_t* table_row, int32_t len, void* k_out, void* v_out,
                  void* stream);

/*
 * decode_plan -- how the decode call splits each sequence's keys.  The keys
 * of a sequence are cut into blocks that are reduced one at a time (page 2,
 * "FlashAttention + PageAttention joint tuning", section 2.2: the tiling of
 * K and V, and the online-softmax recursion that joins the blocks); a split
 * is such a block run by its own workgroup, and the workspace holds each
 * split's partial result until the merge applies that recursion across the
 * splits.  (This call also answers "how many workspace bytes": it reports
 * them beside the split count.)
 * split_tokens > 0 (a multiple of P) fixes the keys per split; 0 lets the
 * library choose from batch, H_kv and max_context_len (a fixed rule aimed at
 * filling a 256-CU device, so the result does not depend on the device; a
 * max_context_len of at most 32 pages is not split).
 * Writes *n_split (splits per sequence; 1 means no workspace and no merge
 * pass) and *workspace_bytes (0 when n_split == 1).  Host-only; no HIP call.
 */
int pkv_decode_plan(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                    int32_t max_context_len, int32_t split_tokens, int32_t* n_split,
                    size_t* workspace_bytes);

/*
 * paged_attn_decode -- one query token per sequence against its paged K/V
 * (page 1, chapter 4.3: a batched decode over kv_cache, block_table
 * [batch, max_blocks] and context_lens [batch]).
 *   q, out       : device [batch][H_q][D] of desc->dtype.
 *   lse_out      : device float [batch][H_q], natural-log log-sum-exp of the
 *                  scaled scores; may be NULL.  Empty context: out row 0,
 *                  lse -inf.
 *   block_table  : device int32 [batch][block_table_stride].
 *   context_lens : device int32 [batch]; keys 0 .. len-1 are attended.
 *   max_context_len : host bound, >= every context_lens[b] and
 *                  <= block_table_stride * P; sizes the grid.
 *   scale        : multiplies Q.K (normally 1/sqrt(D)).
 *   split_tokens : as in pkv_decode_plan.
 *   workspace    : device, >= the workspace_bytes pkv_decode_plan reports for
 *                  the same arguments (may be NULL when that is 0).
 * With n_split > 1 the keys of a sequence are cut into splits of
 * split_tokens; each split yields a partial (o_k, lse_k) and a merge pass
 * combines them by their log-sum-exp (the online-softmax recursion of page 2,
 * section 2.2, applied across splits).
 */
int pkv_paged_attn_decode(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                          const void* q, int32_t batch, int32_t num_q_heads,
                          const int32_t* block_table, int32_t block_table_stride,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          int32_t split_tokens, void* out, float* lse_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_partials -- the first pass of paged_attn_decode alone:
 * writes, for every (b, h, split k), o_k = (sum_t w_t V_t) / (sum_t w_t) and
 * lse_k into the workspace, laid out as
 *     o_parts   float [batch * H_q][n_split][D]      at workspace
 *     lse_parts float [batch * H_q][n_split]         at workspace + o_bytes,
 * o_bytes = batch * H_q * n_split * D * 4 rounded up to 256.  An empty split
 * has o_k = 0 and lse_k = -inf.  Follow with pkv_merge_states() to finish.
 * Arguments as in paged_attn_decode; the workspace is required even when
 * n_split == 1 (size: pkv_decode_plan with that split, or the formula above).
 */
int pkv_paged_attn_decode_partials(const pkv_cache_desc* desc, const void* k_cache,
                                   const void* v_cache, const void* q, int32_t batch,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t block_table_stride, const int32_t* context_lens,
                                   int32_t max_context_len, float scale, int32_t split_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_plan_ex, paged_attn_decode_ex, paged_attn_decode_partials_ex -- the
 * three decode calls above with options (fp8 caches, a q type apart from the
 * cache type, a sliding window).  Same arguments and layouts otherwise; q and
 * out hold opts->q_dtype.  With a window the split plan counts only the pages
 * a window can reach (at most ceil(sink / P) + ceil(window / P) + 1 per
 * sequence), so the plan and the workspace must come from decode_plan_ex with
 * the same options.  opts may be NULL.  fp8 caches need head_dim 128.
 */
int pkv_decode_plan_ex(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                       int32_t max_context_len, int32_t split_tokens,
                       const pkv_decode_opts* opts, int32_t* n_split, size_t* workspace_bytes);

/*
 * decode_split_for_lens -- a split size for a batch whose lengths the caller
 * holds on the host, as a batching scheduler does (page 2, section 4.2:
 * continuous batching mixes requests of every length).  decode_plan's
 * automatic rule sizes every sequence by max_context_len, one or two
 * workgroups per CU; with unequal lengths those workgroups end at different
 * times and leave CUs idle.  This rule counts the pages the batch actually
 * visits (lens_host[b] keys of sequence b, window-aware under opts): when
 * every sequence visits as many pages it returns the automatic split;
 * otherwise a split that spreads them over about 1024 workgroups (four per
 * CU, balanced by the hardware), with at least 32 pages (512 keys) per
 * split.  The decode hands out every sequence's first split before any
 * second split, so the longest pieces of work start first.
 *   lens_host    : host int32 [batch], the lengths the decode will see
 *   opts         : as for decode_plan_ex (may be NULL)
 *   split_tokens : out, a multiple of P, to pass to decode_plan(_ex) and to
 *                  the decode calls
 * Host-only; no HIP call.  Errors: as decode_plan_ex, plus a negative length
 * or a NULL pointer (PKV_ERR_INVALID).
 */
int pkv_decode_split_for_lens(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                              const int32_t* lens_host, const pkv_decode_opts* opts,
                              int32_t* split_tokens);

int pkv_paged_attn_decode_ex(const pkv_cache_desc* desc, const void* k_cache,
                             const void* v_cache, const void* q, int32_t batch,
                             int32_t num_q_heads, const int32_t* block_table,
                             int32_t block_table_stride, const int32_t* context_lens,
                             int32_t max_context_len, float scale, int32_t split_tokens,
                             const pkv_decode_opts* opts, void* out, float* lse_out,
                             void* workspace, size_t workspace_bytes, void* stream);

int pkv_paged_attn_decode_partials_ex(const pkv_cache_desc* desc, const void* k_cache,
                                      const void* v_cache, const void* q, int32_t batch,
                                      int32_t num_q_heads, const int32_t* block_table,
                                      int32_t block_table_stride, const int32_t* context_lens,
                                      int32_t max_context_len, float scale,
                                      int32_t split_tokens, const pkv_decode_opts* opts,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_append, paged_attn_decode_append_partials -- a decode
 * step whose new tokens are stored by the decode launch itself.  The result
 * equals kv_append (kv_append_quant for fp8 caches) of each sequence's newest
 * token followed by paged_attn_decode_ex (paged_attn_decode_partials_ex),
 * bit for bit, with one kernel launch fewer.  A step of page 2, section 5.2
 * stores the new token's K/V in its page (allocated ahead) and then attends
 * it with the rest; that token sits at position L - 1 of its sequence,
 * L = context_lens[b], so only the decode workgroup whose split ends at that
 * page reads it.  That workgroup stores the row before it loads anything.
 * For each b with 1 <= L and every KV head g, with
 * s = block_table[b][(L - 1) / P] * P + (L - 1) % P:
 *     k_cache[s / P][g][s % P][:] = k_new[b][g][:]   (same for V)
 * (fp8 caches: each element divided by opts->k_scale (v_scale) in IEEE fp32
 * and rounded to the fp8 code, as kv_append_quant does).
 *   k_cache, v_cache : device, updated in place (the row at L - 1 only).
 *   k_new, v_new     : device [batch][H_kv][D] of opts->q_dtype (the cache
 *                      dtype, except for fp8 caches: f16 or bf16), 16-byte
 *                      aligned.
 * Other arguments, layouts and errors are as for paged_attn_decode_ex and
 * paged_attn_decode_partials_ex.  L = 0 stores nothing.  A length or page the
 * decode flags as invalid (NaN output rows) stores nothing for that sequence.
 * Two sequences whose newest tokens map to the same slot race, as two equal
 * slots do in kv_append.
 */
int pkv_paged_attn_decode_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                                 const void* k_new, const void* v_new, const void* q,
                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                 int32_t block_table_stride, const int32_t* context_lens,
                                 int32_t max_context_len, float scale, int32_t split_tokens,
                                 const pkv_decode_opts* opts, void* out, float* lse_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

int pkv_paged_attn_decode_append_partials(
    const pkv_cache_desc* desc, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const void* q, int32_t batch, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* context_lens,
    int32_t max_context_len, float scale, int32_t split_tokens, const pkv_decode_opts* opts,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_append_noalloc -- paged_attn_decode_append without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The split-KV partials go to a static device array of
 * pkv_noalloc_scratch_bytes() bytes (16 MiB), one per GPU, held until the
 * process ends; the call itself allocates and frees nothing.  Arguments,
 * layouts, results (bit for bit) and errors are those of
 * paged_attn_decode_append with the same split_tokens, plus
 * PKV_ERR_WORKSPACE when the split plan needs more than that array
 * (batch * H_q * n_split * (D + 1) * 4 bytes, the partials rounded up to 256
 * bytes; pass a larger split_tokens).  A plan with n_split == 1 needs none.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (on different streams, or from different threads) race and give
 * unspecified results; calls on one stream are ordered and safe.  The first
 * call on a device looks up the array's device address (no allocation).
 */
int pkv_paged_attn_decode_append_noalloc(const pkv_cache_desc* desc, void* k_cache,
                                         void* v_cache, const void* k_new, const void* v_new,
                                         const void* q, int32_t batch, int32_t num_q_heads,
                                         const int32_t* block_table, int32_t block_table_stride,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         float scale, int32_t split_tokens,
                                         const pkv_decode_opts* opts, void* out, float* lse_out,
                                         void* stream);

/* Bytes of the static scratch array of paged_attn_decode_append_noalloc. */
size_t pkv_noalloc_scratch_bytes(void);

/*
 * kv_append_quant -- kv_append into an fp8 cache from wider new tokens.
 * For each i with s = slot_mapping[i] >= 0 (and < num_pages * P), every KV
 * head g and element d:
 *     k_cache[s / P][g][s % P][d] = fp8(k_new[i][g][d] / k_scale)   (V alike)
 * where the quotient is taken in IEEE fp32 and fp8() rounds to the nearest
 * code, ties to the even code, clips values beyond the largest finite one to
 * it (infinities included) and maps NaN to the byte 0x7F.  The pages fix no
 * quantization rule; this is the plainest per-tensor one.
 *   desc->dtype      : PKV_FP8_E4M3 or PKV_FP8_E5M2.
 *   k_new, v_new     : device [n_tokens][H_kv][D] of src_dtype (f32, f16, bf16).
 *   k_scale, v_scale : finite, > 0.
 */
int pkv_kv_append_quant(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                        const void* k_new, const void* v_new, int32_t src_dtype, float k_scale,
                        float v_scale, const int32_t* slot_mapping, int32_t n_tokens,
                        void* stream);

/*
 * merge_states -- combine n_parts partial attention states per row.  Each
 * part is the softmax-weighted V sum of one block of keys with its
 * log-sum-exp; joining them is the online-softmax recursion of page 2,
 * "FlashAttention + PageAttention joint tuning", section 2.2 (the running
 * maximum and the rescaled sums), applied once across the blocks:
 *     M = max_k lse_k,  w_k = exp(lse_k - M),
 *     out = sum_k w_k o_k / sum_k w_k,  lse = M + log(sum_k w_k),
 * in ascending k order.  Parts with lse_k = -inf are skipped; all skipped
 * gives out 0 and lse -inf.
 *   o_parts   : device float [rows][n_parts][head_dim], 16-byte aligned;
 *               head_dim 64 or 128
 *   lse_parts : device float [rows][n_parts]
 *   out       : device [rows][head_dim] of out_dtype (f32, f16 or bf16)
 *   lse_out   : device float [rows] or NULL
 */
int pkv_merge_states(const float* o_parts, const float* lse_parts, int32_t rows,
                     int32_t n_parts, int32_t head_dim, int32_t out_dtype, void* out,
                     float* lse_out, void* stream);

/*
 * paged_attn_prefill_chunk -- a causal chunk of query rows against the paged
 * history plus the chunk itself (page 4, section 3.1: chunked prefill splits
 * a prompt into chunks that reuse the KV cache).  The caller appends the
 * chunk's K/V with pkv_kv_append first; kv_lens[b] counts history plus chunk.
 * Chunk row i of sequence b (C_b rows) sits at position kv_lens[b] - C_b + i
 * and attends to keys 0 .. that position (bottom-right aligned causal mask).
 *   q, out       : device, packed [total_q_rows][H_q][D] of desc->dtype;
 *                  total_q_rows = sum_b C_b.
 *   q_indptr     : device int32 [batch + 1]; rows of sequence b are
 *                  q_indptr[b] .. q_indptr[b+1]-1; q_indptr[0] = 0.  Rows
 *                  outside [0, total_q_rows) are never read or written.
 *   max_q_len    : host bound >= every C_b; sizes the grid.
 *   block_table, block_table_stride : as for decode.
 *   kv_lens      : device int32 [batch]; C_b <= kv_lens[b] <= stride * P.
 *   max_kv_len   : host bound >= every kv_lens[b], <= stride * P.
 *   lse_out      : device float [total_q_rows][H_q] or NULL.
 * QK^T and PV run on the matrix cores (MFMA, fp32 accumulation); the
 * probabilities enter the PV product rounded to the query type.  Needs f16
 * or bf16 pools with head_dim 128 or 64 (fp8 pools, head_dim 128: the _ex
 * form).
 */
int pkv_paged_attn_prefill_chunk(const pkv_cache_desc* desc, const void* k_cache,
                                 const void* v_cache, const void* q, const int32_t* q_indptr,
                                 int32_t batch, int32_t num_q_heads, int32_t total_q_rows,
                                 int32_t max_q_len, const int32_t* block_table,
                                 int32_t block_table_stride, const int32_t* kv_lens,
                                 int32_t max_kv_len, float scale, void* out, float* lse_out,
                                 void* stream);

/*
 * paged_attn_prefill_chunk_ex -- paged_attn_prefill_chunk with options, for
 * fp8 pools (page 4, section 3.1 prefills in chunks over an fp8_e5m2 cache;
 * page 1, section 4.1 names e4m3).  opts: q_dtype PKV_F16 or PKV_BF16 for
 * fp8 pools (q and out of that type), k_scale / v_scale as for decode;
 * window and sink must be 0 (PKV_ERR_INVALID otherwise).  The chunk's K/V go
 * in with pkv_kv_append_quant first.  Each fp8 page is widened exactly to
 * q_dtype inside the kernel; the K scale multiplies the softmax scale, the V
 * scale the output.  NULL opts: as paged_attn_prefill_chunk (fp8 pools then
 * fail with PKV_ERR_INVALID).
 */
int pkv_paged_attn_prefill_chunk_ex(const pkv_cache_desc* desc, const void* k_cache,
                                    const void* v_cache, const void* q,
                                    const int32_t* q_indptr, int32_t batch,
                                    int32_t num_q_heads, int32_t total_q_rows,
                                    int32_t max_q_len, const int32_t* block_table,
                                    int32_t block_table_stride, const int32_t* kv_lens,
                                    int32_t max_kv_len, float scale,
                                    const pkv_decode_opts* opts, void* out, float* lse_out,
                                    void* stream);

/*
 * paged_attn_mixed -- one call for a ragged batch that mixes decode rows and
 * prefill chunks, the batch a chunked-prefill scheduler forms under a token
 * budget (page 1, section 4.1: chunked prefill with a bound on the batched
 * tokens; page 2, section 4.2: continuous batching puts new requests next to
 * running ones).  It computes exactly what paged_attn_prefill_chunk computes
 * for the whole batch (row i of sequence b at position kv_lens[b] - C_b + i,
 * bottom-right causal), with the batch laid out decode-first: sequences
 * 0 .. num_decode-1 have one query row each, rows 0 .. num_decode-1
 * (q_indptr[b] = b for b <= num_decode, a precondition on device data), and
 * the remaining sequences carry chunks.  The decode rows go through the
 * split-KV decode kernel (workspace and merge as in paged_attn_decode, with
 * batch = num_decode and max_context_len = max_kv_len), the chunks through
 * the MFMA prefill kernel; both on `stream`, in that order.
 *   num_decode : 0 <= num_decode <= batch and <= total_q_rows.
 *   max_q_len  : host bound >= C_b of every chunk sequence (>= 1 if any).
 *   workspace  : >= the workspace_bytes of pkv_decode_plan(desc, num_decode,
 *                num_q_heads, max_kv_len, split_tokens); may be NULL when 0.
 * Other arguments as for paged_attn_prefill_chunk (f16 or bf16 pools, head_dim
 * 128 or 64; fp8 pools, head_dim 128: the _ex form).
 */
int pkv_paged_attn_mixed(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                         const void* q, const int32_t* q_indptr, int32_t batch,
                         int32_t num_decode, int32_t num_q_heads, int32_t total_q_rows,
                         int32_t max_q_len, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* kv_lens, int32_t max_kv_len,
                         float scale, int32_t split_tokens, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_mixed_ex -- paged_attn_mixed with options (fp8 pools): opts as
 * for paged_attn_prefill_chunk_ex, used for both the decode rows and the
 * chunks; the workspace is that of pkv_decode_plan_ex(desc, num_decode,
 * num_q_heads, max_kv_len, split_tokens, opts).
 */
int pkv_paged_attn_mixed_ex(const pkv_cache_desc* desc, const void* k_cache,
                            const void* v_cache, const void* q, const int32_t* q_indptr,
                            int32_t batch, int32_t num_decode, int32_t num_q_heads,
                            int32_t total_q_rows, int32_t max_q_len,
                            const int32_t* block_table, int32_t block_table_stride,
                            const int32_t* kv_lens, int32_t max_kv_len, float scale,
                            int32_t split_tokens, const pkv_decode_opts* opts, void* out,
                            float* lse_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * decode_shared_prefix_plan -- the partial count and workspace of
 * paged_attn_decode_shared_prefix for these sizes (host only, no HIP call).
 * *n_parts = key splits of the shared pages + splits of the own pages (the
 * latter as pkv_decode_plan_ex would pick them for max_suffix_len);
 * *workspace_bytes > 0 whenever batch > 0.
 */
int pkv_decode_shared_prefix_plan(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                  int32_t prefix_len, int32_t max_suffix_len,
                                  int32_t split_tokens, const pkv_decode_opts* opts,
                                  int32_t* n_parts, size_t* workspace_bytes);

/*
 * paged_attn_decode_shared_prefix -- decode for a batch whose sequences all
 * begin with the same physical pages (page 2, section 3.2: identical prompt
 * prefixes share physical pages; page 4, section 3.3: shared prefixes are
 * reused from the cache automatically).  The
 * result is that of paged_attn_decode_ex over, for sequence b, the table
 * prefix_table ++ block_table[b] and prefix_len + suffix_lens[b] keys; it is
 * computed as a cascade: the shared pages are read once for the whole batch
 * (every sequence's query rows against them on the matrix cores, split over
 * the keys), each sequence's own pages by the split-KV decode, and all
 * partial results are combined by the log-sum-exp merge (rounding differs
 * from the one-pass decode; the result is within the same tolerance).
 *   q, out        : device [batch][H_q][D] of the query type; 16-byte aligned.
 *   prefix_table  : device int32 [prefix_len / P], the shared pages in order;
 *                   may be NULL when prefix_len == 0.
 *   prefix_len    : >= 0, a multiple of P (shared pages are whole pages;
 *                   PKV_ERR_INVALID otherwise).
 *   block_table, block_table_stride : device int32 [batch][stride], the pages
 *                   of each sequence after the shared ones.
 *   suffix_lens   : device int32 [batch], keys of each sequence after the
 *                   shared ones (0 allowed); max_suffix_len a host bound, as
 *                   max_context_len of paged_attn_decode.
 *   opts          : as for paged_attn_decode_ex (query type, fp8 scales);
 *                   window and sink must be 0.  NULL: the cache type.
 *   workspace     : >= the workspace_bytes of decode_shared_prefix_plan,
 *                   16-byte aligned; holds fp32 partials [batch*H_q][n_parts]
 *                   [D] and their log-sum-exps.
 * Pools: f16 or bf16 with head_dim 128 or 64, fp8 (e4m3 / e5m2) with head_dim
 * 128; G as for decode.
 * Three launches on `stream`; no synchronisation.
 */
int pkv_paged_attn_decode_shared_prefix(
    const pkv_cache_desc* desc, const void* k_cache, const void* v_cache, const void* q,
    int32_t batch, int32_t num_q_heads, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* suffix_lens,
    int32_t max_suffix_len, float scale, int32_t split_tokens, const pkv_decode_opts* opts,
    void* out, float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * validate_tables -- host-side check of host copies of the tables (no HIP
 * call), the consistency checker that page 3, "Flash Attention and Paged KV
 * Cache in practice", section 6.2 recommends against scrambled attention
 * after page replacement (every page within its size, every page id valid):
 * every entry a sequence uses (the first ceil(lens[b]/P) of its row)
 * is in [0, num_pages); 0 <= lens[b] <= stride * P; every slot is < 0 or in
 * [0, num_pages * P) and no slot >= 0 repeats.  slots may be NULL (n = 0).
 * Returns PKV_OK or PKV_ERR_INVALID with the first offence in
 * pkv_last_error().
 */
int pkv_validate_tables(const pkv_cache_desc* desc, const int32_t* block_table_host,
                        int32_t block_table_stride, const int32_t* lens_host, int32_t batch,
                        const int32_t* slots_host, int32_t n_slots);

/*
 * Measurement aids -- not part of the attention path.  They give the
 * measured ceilings the rooflines of the kernels above are read against
 * (the nominal peaks being the chip's published figures).
 *
 * probe_read -- read every byte of buf once with 16-byte streaming loads.
 *   block_order == NULL: sequentially, grid workgroups of 256 threads
 *   stepping over the buffer.  Otherwise buf is bytes / block_bytes blocks
 *   (block_bytes a multiple of 4096) read whole in the order block_order
 *   (device int32 [bytes / block_bytes]) gives -- the decode's pattern of
 *   randomly placed 4 KiB (page, KV head) blocks when it is a permutation;
 *   ids outside the range are skipped.  Bytes read per launch: bytes.
 *   sink: device uint32 [1]; written only when the loaded data's XOR hits a
 *   fixed value, which keeps the loads live.  16-byte aligned buf; bytes a
 *   positive multiple of 16 (and of block_bytes).
 *
 * probe_mfma -- grid workgroups of 8 waves (two per SIMD), each wave running
 *   iters rounds of 4 independent v_mfma_f32_32x32x16_bf16 on operands read
 *   from `operands` (device, 256 x 16 bytes of bf16, e.g. random values; the
 *   matrix cores draw more power, and the clock drops further, on random
 *   data than on zeros).  vector_work 1 adds, per MFMA, the vector work the
 *   prefill kernel does per MFMA (an FMA, an exp2 and an add per score, a
 *   bf16 pair conversion every second MFMA).  Flops per launch:
 *   grid * 8 * iters * 4 * 32768.  clocks: device int64 [2], the shader-clock
 *   and the 100 MHz constant-clock cycles of wave 0 of workgroup 0 (their
 *   ratio times 100 MHz is the shader clock under this load).  sink as above.
 *
 * probe_prefill_loop -- the chunked-prefill kernel's tile loop on its own:
 *   grid workgroups of 8 waves, each wave running iters rounds of two 64-key
 *   tiles at bf16, head_dim 128, 32 query rows: per tile 16 QK MFMAs whose K
 *   operands are read from an LDS tile in that kernel's layout, then 16 PV
 *   MFMAs whose V^T operands come from transposing LDS reads (the tiles are
 *   filled once from `operands`, 256 x 16 bytes of bf16).  vector_work 1
 *   forms the weights of each tile's scores beside the next tile's QK MFMAs
 *   (an FMA, an exp2 and an add per score, a bf16 pair conversion per two),
 *   as that kernel does; 0 leaves them out.  No page copies, barriers, masks
 *   or rescaling.  Flops per launch: grid * 8 * iters * 2 * 32 * 32768.
 *   clocks and sink as for probe_mfma.
 */
int pkv_probe_read(const void* buf, size_t bytes, const int32_t* block_order,
                   int32_t block_bytes, int32_t grid, uint32_t* sink, void* stream);

int pkv_probe_mfma(const void* operands, int32_t iters, int32_t vector_work, int32_t grid,
                   uint32_t* sink, int64_t* clocks, void* stream);

int pkv_probe_prefill_loop(const void* operands, int32_t iters, int32_t vector_work,
                           int32_t grid, uint32_t* sink, int64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
