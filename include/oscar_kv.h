/*
 * liboscar_kv: the OSCAR INT2 KV-cache hot path on AMD Instinct MI355X (gfx950).
 *
 * The method (OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
 * Quantization) keeps a three-segment token pool per request and KV head: a BF16 sink of
 * 64 tokens, an INT2 history, and a BF16 recent window of 256 tokens (QbitAI article on
 * OSCAR, serving-path section). Tokens leaving the recent window are rotated by a fixed
 * per-layer, per-KV-head orthogonal R = U * Hadamard * bit-reversal (same article, section
 * on aiming the rotation at attention), clipped, quantised to 2 bits with a per-group
 * scale and zero point and packed four codes per byte. Decode processes the INT2 history
 * and the BF16 sink/recent separately and joins them with an online-softmax merge.
 *
 * Conventions for every entry point:
 *   - Plain C ABI. All tensor pointers are DEVICE pointers unless marked host. The caller
 *     owns every buffer; the library allocates nothing and keeps no state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and returns
 *     without synchronising. Calls on different streams may run concurrently when they
 *     write disjoint memory.
 *   - Arguments are validated on the host before any HIP call; a failed check returns a
 *     status and enqueues nothing. Device-resident values (page ids, lengths, slots) are
 *     trusted: out-of-range values are undefined behaviour.
 *   - bf16 and fp16 tensors are passed as raw 16-bit storage (`const void*`).
 *   - Vectors are rows; rotating is y = x R (R row-major [128][128]); un-rotating is y R^T.
 *   - Each failing call also records a message, readable with oscar_last_error() on the
 *     same host thread.
 *
 * Fixed shapes: head_dim = 128, page_tokens = 64, sink_tokens = 64,
 * recent_tokens = 256; n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}; query head h uses KV
 * head h / (n_q_heads / n_kv_heads). group_size is 128 (one scale and zero point per
 * vector) for every entry point except the *_grouped ones, which also take 64 and 32; the
 * size helpers, oscar_decode_bf16 and oscar_merge take any of the three.
 *
 * INT2 pool layout (4608 bytes per page per KV head, head h of physical page p at byte
 * (p * n_kv_heads + h) * 4608). Codes are packed 16 to a little-endian 32-bit word, the code
 * with index 4m + j of the word's 16 in byte j at bits 2m..2m+1.
 *   [   0, 2048)  K codes: the word of slot t, dims 16w..16w+15, at byte
 *                 32 (16 (w / 2) + t / 4) + 8 (t % 4) + 4 (w % 2).
 *   [2048, 4096)  V codes: the word of dim d, slots 16u..16u+15, at byte
 *                 2048 + 32 (16 u + d % 16) + 4 (d / 16).
 *   [4096, 4352)  K fp16 scale s and zero point z of slot t at 4096 + 4 t (s first).
 *   [4352, 4608)  V fp16 scale and zero point of slot t at 4352 + 4 t.
 * (The word order lets lane l = 16 G + n of the decode pass read its K and V words as two
 * contiguous 32-byte chunks at 32 l and 2048 + 32 l.)
 * A code q stands for q * s + z in the rotated basis. History entry j of a request lives in
 * slot j % 64 of physical page block_table[b * max_pages + j / 64].
 *
 * Partial-result workspace (online-softmax state of one segment split): for B requests,
 * Hq query heads and S splits, a buffer of oscar_partials_bytes(desc, B, S) bytes holding
 *   float m[B][Hq][S]     running maximum of the scores, in log2 units (score * log2 e)
 *   float l[B][Hq][S]     sum of 2^(score*log2e - m)
 *   float acc[B][Hq][S][128]  sum of 2^(score*log2e - m) * value
 * with m at byte 0, l at byte 4*B*Hq*S and acc at the next multiple of 256 bytes. An
 * empty split holds m = -inf, l = 0, acc = 0. INT2 partials hold acc in the rotated basis.
 * After acc (from the next multiple of 256 bytes) the INT2 pass keeps its per-(request,
 * query head) rotated-query data: 512 bytes of fixed-point limbs per head, then, from the
 * next multiple of 256 bytes, 32 bytes of scalars per head. oscar_merge does not read
 * that tail.
 */
#ifndef OSCAR_KV_H
#define OSCAR_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum oscar_status {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID_ARG = 1, /* null pointer, bad count or inconsistent shape */
  OSCAR_ERR_UNSUPPORTED = 2, /* a shape outside the fixed set above */
  OSCAR_ERR_WORKSPACE = 3,   /* workspace smaller than the size helper reports */
  OSCAR_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} oscar_status;

typedef struct oscar_layer_desc {
  int32_t head_dim;      /* must be 128 */
  int32_t group_size;    /* quantisation group: 128 (one per vector), or 64 / 32 (grouped pages) */
  int32_t page_tokens;   /* must be 64 */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t sink_tokens;   /* must be 64 */
  int32_t recent_tokens; /* must be 256 */
} oscar_layer_desc;

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t oscar_version(void);

/* Static text for a status code. */
const char* oscar_status_string(int32_t status);

/* Message of the last failed call on this host thread ("" if none). */
const char* oscar_last_error(void);

/* Checks a descriptor; OSCAR_OK if it is valid (group_size 128, 64 or 32; entry points
 * other than the *_grouped ones return OSCAR_ERR_UNSUPPORTED for 64 and 32). */
int32_t oscar_check_desc(const oscar_layer_desc* desc);

/* Bytes of one physical page (all KV heads): n_kv_heads * (4096 + 512 * 128 / group_size),
 * that is n_kv_heads * 4608 for one group per vector. 0 for a bad desc. */
size_t oscar_page_bytes(const oscar_layer_desc* desc);

/* BF16 window slots per request and KV head: sink_tokens + recent_tokens. */
int32_t oscar_window_tokens(const oscar_layer_desc* desc);

/* Splits oscar_decode_bf16 produces per (request, query head): window_tokens / 64, rounded up. */
int32_t oscar_window_splits(const oscar_layer_desc* desc);

/* Bytes of a partial-result workspace for `batch` requests and `n_splits` splits. */
size_t oscar_partials_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits);

/* A split count that fills the GPU for this batch and longest history (>= 1). */
int32_t oscar_default_splits(const oscar_layer_desc* desc, int32_t batch, int32_t max_hist_len);

/*
 * oscar_demote: move tokens from the BF16 recent window into INT2 history.
 * (QbitAI article on OSCAR, serving-path section: the oldest recent token is rotated,
 * clipped, quantised and packed, then stored in the INT2 history; abstracts: the
 * rotations and clipping thresholds are fixed per layer and derived offline.)
 *
 * For each token i < n and KV head h, and separately for K and V with their own R and c:
 *   y = x R, with x the bf16 row; the group extremes are taken on the exact products
 *   hi = c * max(y), lo = c * min(y)                         (fp64)
 *   s = fp16((hi - lo) / 3), z = fp16(lo)                    (round to nearest even)
 *   q_j = clamp(round_half_even((y_j - z) / s), 0, 3); all codes 0 when s == 0
 * and stores the codes, s and z at (dst_page[i], dst_slot[i]) of head h in the pool,
 * leaving every other slot's bits untouched. s, z and the codes are always exactly these:
 * below 64 tokens a per-row kernel sums in fp64 and re-sums with compensation any row its
 * error bound cannot settle; from 64 tokens on a matrix-core kernel sums in fp32 under a
 * proven any-order error bound and re-sums in fp64 (then with compensation) every extreme
 * and every value whose bound straddles a rounding boundary, so ties round to even.
 * Domain: the clipped extremes must stay within fp16 range (|c y| <= 65504). A row outside
 * it gets the fp16 rounding of its scale and zero point (infinite) and all codes 0, and
 * the other rows of the call are unaffected.
 *
 *   k_src, v_src   bf16 [n][n_kv_heads][128], the rows to demote (unrotated)
 *   dst_page       int32 [n], physical page of token i
 *   dst_slot       int32 [n], slot 0..63 of token i
 *   rot_k, rot_v   bf16 [n_kv_heads][128][128], per-head rotations
 *   clip_k, clip_v float32 [n_kv_heads], clip ratios c in (0, 1]
 *   pool           the INT2 pool (layout above), written in place
 * Two tokens of one call must not share a (page, slot). n == 0 is a no-op.
 */
int32_t oscar_demote(const oscar_layer_desc* desc, const void* k_src, const void* v_src,
                     int32_t n, const int32_t* dst_page, const int32_t* dst_slot,
                     const void* rot_k, const void* rot_v, const float* clip_k,
                     const float* clip_v, void* pool, void* stream);

/*
 * oscar_decode_int2: the INT2 history pass of decode attention.
 * (QbitAI article on OSCAR, serving-path section: the INT2 kernel unpacks, dequantises
 * with the scale and zero point and accumulates in floating point; the history is paged.)
 *
 * For request b and query head h (KV head kv): q_rot = q R_K[kv]; each history entry j
 * scores sm_scale * q_rot . (q_j * s_j + z_j); the history of b is cut into n_splits
 * contiguous page ranges and one online-softmax partial (m, l, acc in the rotated V basis)
 * is written per (b, h, split).
 *
 *   q            bf16 [batch][n_q_heads][128], the raw (unrotated) queries
 *   rot_k        bf16 [n_kv_heads][128][128]
 *   pool         INT2 pool
 *   block_table  int32 [batch][max_pages]
 *   hist_len     int32 [batch], history entries per request (0 allowed, at most
 *                64 max_pages)
 *   sm_scale     softmax scale applied to q . k (e.g. 1/sqrt(128) as a float)
 *   n_splits     1..65535, with at most 8192 pages per split: ceil(max_pages / n_splits)
 *                <= 8192, else OSCAR_ERR_UNSUPPORTED (the pass keeps int32 value sums
 *                per wave; oscar_default_splits respects the bound)
 *   partials     workspace of at least oscar_partials_bytes(desc, batch, n_splits) bytes
 */
int32_t oscar_decode_int2(const oscar_layer_desc* desc, const void* q, const void* rot_k,
                          const void* pool, const int32_t* block_table, int32_t max_pages,
                          const int32_t* hist_len, int32_t batch, float sm_scale,
                          int32_t n_splits, void* partials, size_t partials_bytes, void* stream);

/*
 * oscar_decode_bf16: the BF16 sink/recent pass of decode attention.
 * (QbitAI article on OSCAR, serving-path section: a BF16 kernel handles sink and recent.)
 *
 * Window slots [0, win_len[b]) of each request hold raw bf16 K/V rows (the sink, then
 * the recent tokens; order does not matter to attention). Writes oscar_window_splits(desc)
 * partials per (b, h), split c covering slots [64 c, 64 c + 64).
 *
 *   k_win, v_win  bf16 [batch][n_kv_heads][window_tokens][128]
 *   win_len       int32 [batch], 0..window_tokens
 *   win_partials  workspace of at least oscar_partials_bytes(desc, batch, window_splits)
 */
int32_t oscar_decode_bf16(const oscar_layer_desc* desc, const void* q, const void* k_win,
                          const void* v_win, const int32_t* win_len, int32_t batch,
                          float sm_scale, void* win_partials, size_t win_partials_bytes,
                          void* stream);

/*
 * oscar_merge: join the INT2 and BF16 segments.
 * (QbitAI article on OSCAR, serving-path section: the two parts are combined by an
 * online-softmax merge.)
 *
 * Reduces the n_splits INT2 partials of (b, h), un-rotates their value sum by R_V^T,
 * reduces the window partials, and writes
 *   out = (a acc_int2 R_V^T + w acc_win) / (a l_int2 + w l_win),
 * a = 2^(m_int2 - M), w = 2^(m_win - M), M = max of the two; 0 if both segments are empty.
 *
 *   partials      from oscar_decode_int2 with the same n_splits
 *   win_partials  from oscar_decode_bf16
 *   rot_v         bf16 [n_kv_heads][128][128]
 *   out           float32 [batch][n_q_heads][128]
 */
int32_t oscar_merge(const oscar_layer_desc* desc, const void* partials, int32_t n_splits,
                    const void* win_partials, const void* rot_v, float* out, int32_t batch,
                    void* stream);

/* Bytes of the workspace of oscar_decode / oscar_decode_step for `batch` requests and
 * `n_splits` history splits (0 for a bad desc). */
size_t oscar_decode_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits);

/*
 * oscar_decode_step: one decode step of one layer in two launches: demotion, then decode
 * attention over all three segments. The same result as oscar_demote, oscar_decode_int2,
 * oscar_decode_bf16 and oscar_merge called in that order.
 * (QbitAI article on OSCAR, serving-path section: the oldest recent token is rotated,
 * clipped, quantised, packed and demoted into the INT2 history; decode processes the BF16
 * sink/recent and the INT2 history separately and joins them by an online-softmax merge.)
 *
 * Launch 1 runs the n demotions (as oscar_demote), the BF16 window pass and the query
 * rotation; launch 2 runs the INT2 pass, and for each (request, KV head) the workgroup
 * that finishes last merges that KV head's query heads and writes `out`. Arguments are
 * those of the four calls above; in addition:
 *   workspace  at least oscar_decode_workspace_bytes(desc, batch, n_splits) bytes of device
 *              memory, owned by the caller; its contents need no initialisation and are
 *              overwritten (INT2 and window partials, query data, arrival counters)
 *   out        float32 [batch][n_q_heads][128]
 *   n_splits   1..256 (OSCAR_ERR_UNSUPPORTED above), and ceil(max_pages / n_splits) <= 8192
 *              as for oscar_decode_int2
 * Demotions land before the history is read: a token demoted by this call is part of the
 * history it attends over (hist_len must count it). n == 0 demotes nothing (then k_src,
 * v_src, dst_page, dst_slot, clip_k and clip_v may be null). Calls that share a
 * workspace must not overlap in time.
 */
int32_t oscar_decode_step(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                          const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                          const void* q, const void* rot_k, const void* rot_v, void* pool,
                          const int32_t* block_table, int32_t max_pages, const int32_t* hist_len, const void* k_win,
                          const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale,
                          int32_t n_splits, void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * oscar_decode_step_append: one decode step of one layer in a single launch, for the
 * serving loop's usual demotion: each request b appends one token, its oldest recent token,
 * to the end of its INT2 history, then decodes.
 * (QbitAI article on OSCAR, serving-path section: the oldest recent token is rotated,
 * clipped, quantised, packed and demoted into the INT2 history; decode processes the BF16
 * sink/recent and the INT2 history separately and joins them by an online-softmax merge.)
 *
 * Token b of k_src / v_src (bf16 [batch][n_kv_heads][128]) becomes history token
 * hist_len[b] - 1 of request b, in the page and slot the block table gives it (hist_len
 * counts it), demoted exactly as oscar_demote demotes it; the output is then that of
 * oscar_decode over the updated pool. That page must be one no other request of the call
 * reads (as in paged serving, where a request appends into its own last page, never into
 * a shared prefix page). k_src == NULL (with v_src, clip_k, clip_v NULL or
 * ignored) demotes nothing and decodes the pool as it is. A request with hist_len 0 while
 * appending is skipped (nothing is demoted for it).
 * One launch when its workgroups fit the chip at once (oscar_decode_step_append_launches):
 * window workgroups; one workgroup per (request, KV head) that demotes the appended token
 * and contributes that token's attention term; and INT2 workgroups that rotate the query
 * themselves and leave the appended token out. The workgroup that finishes last per
 * (request, KV head) merges. No workgroup waits for another. While the appended token's V
 * codes are written, INT2 workgroups may read the 32-bit words that hold them; that slot has
 * weight zero in their pass, so whichever value such a read returns, the result is the same.
 * Otherwise the step runs as two launches (prepare, attend), as oscar_decode_step does,
 * with the appended token's page and slot taken from the block table on the device.
 * Arguments are those of oscar_decode_step, plus:
 *   n_splits   1..255, and ceil(max_pages / n_splits) <= 8192; oscar_decode_step_append_splits
 *              gives the count for which the launch's workgroups fit the chip at once
 *   workspace  at least oscar_decode_step_append_workspace_bytes(desc, batch, n_splits)
 *              bytes of device memory, owned by the caller, whose arrival counters must be
 *              zero before the first call: zero-fill it after allocating it and again
 *              when batch or n_splits change (the counters follow the partials, whose
 *              size depends on both); every call leaves them at zero (oscar_decode_step
 *              and oscar_decode leave them at zero too, so a workspace can serve both).
 *              Calls that share a workspace must not overlap in time.
 * Errors: OSCAR_ERR_INVALID_ARG (null pointers, batch or n_splits <= 0, bad sm_scale),
 * OSCAR_ERR_UNSUPPORTED (sizes past the limits above), OSCAR_ERR_WORKSPACE (too small),
 * OSCAR_ERR_HIP (launch failure).
 */
size_t oscar_decode_step_append_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits);
int32_t oscar_decode_step_append_splits(const oscar_layer_desc* desc, int32_t batch, int32_t max_hist_len);
/* Launches oscar_decode_step_append makes for (desc, batch, n_splits): 1 (one launch) or 2
 * (prepare, attend); 0 for an invalid descriptor, batch or n_splits. Host only, no device
 * work. */
int32_t oscar_decode_step_append_launches(const oscar_layer_desc* desc, int32_t batch, int32_t n_splits);
int32_t oscar_decode_step_append(const oscar_layer_desc* desc, const void* k_src, const void* v_src,
                                 const float* clip_k, const float* clip_v, const void* q, const void* rot_k,
                                 const void* rot_v, void* pool, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* hist_len, const void* k_win, const void* v_win, const int32_t* win_len,
                                 int32_t batch, float sm_scale, int32_t n_splits, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream);
/* oscar_decode_step_append with the Lloyd-Max codebook (as oscar_demote_codebook and
 * oscar_decode_codebook). */
int32_t oscar_decode_step_append_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src,
                                          const float* clip_k, const float* clip_v, const void* q, const void* rot_k,
                                          const void* rot_v, const uint8_t* codebook, void* pool,
                                          const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                          const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                          float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                                          float* out, void* stream);

/*
 * oscar_decode_step_noalloc: oscar_decode_step without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc). The same kernels and the same result as oscar_decode_step; its
 * workspace is a static device array of oscar_decode_step_noalloc_max_bytes() bytes
 * (16 MiB) that the library holds on every GPU it runs on until the process ends.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call.
 *   Errors: OSCAR_ERR_WORKSPACE when oscar_decode_workspace_bytes(desc, batch, n_splits)
 *   exceeds the array (nothing is enqueued); otherwise those of oscar_decode_step.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU
 * (on different streams, or from different threads) race and must not be issued. The
 * array keeps the last call's contents; the step's first launch clears the arrival
 * counters it needs at zero. `stream` must belong to the current device.
 */
size_t oscar_decode_step_noalloc_max_bytes(void);
int32_t oscar_decode_step_noalloc(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                  const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                  const float* clip_v, const void* q, const void* rot_k, const void* rot_v, void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                  float sm_scale, int32_t n_splits, float* out, void* stream);

/*
 * oscar_decode: decode attention over the three segments in two launches, without
 * demotion (oscar_decode_step with n == 0; the pool is only read).
 * (QbitAI article on OSCAR, serving-path section: INT2 and BF16 segments processed
 * separately, joined by an online-softmax merge.)
 */
int32_t oscar_decode(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* rot_v,
                     const void* pool, const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                     const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale,
                     int32_t n_splits, void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * oscar_decode_multi: decode attention for n_tokens consecutive query tokens per request
 * over one pool, in two launches, without demotion (speculative verification or a
 * chunked prefill reading the compressed prefix).
 * (QbitAI article on OSCAR, serving-path section: paged KV and radix prefix cache reuse,
 * with separate BF16 and INT2 passes joined by an online-softmax merge; several query
 * tokens over one compressed prefix is this library's reading of that reuse.)
 *
 * Query token t (0 <= t < n_tokens) of request b is the token at window position
 * win_len[b] - n_tokens + t: it attends to the whole INT2 history and to window slots
 * [0, win_len[b] - (n_tokens - 1 - t)) (causal among the query tokens, whose K and V are
 * the last n_tokens window slots). With n_tokens == 1 this is oscar_decode.
 * One launch when its workgroups fit the chip at once (the window workgroups and INT2
 * workgroups that rotate their query rows themselves, as in oscar_decode_step_append
 * without an appended token; oscar_decode_multi_splits gives a split count for which they
 * do); otherwise two launches (prepare, attend).
 *   q          bf16 [batch][n_tokens][n_q_heads][128]
 *   out        float32 [batch][n_tokens][n_q_heads][128]
 *   n_tokens   a power of two with n_tokens * (n_q_heads / n_kv_heads) <= 16 (else
 *              OSCAR_ERR_UNSUPPORTED); batch * n_tokens <= 65535
 *   workspace  at least oscar_decode_workspace_bytes(desc, batch * n_tokens, n_splits)
 *              bytes, whose arrival counters must be zero before the first call (zero-fill
 *              it after allocating it and again when batch, n_tokens or n_splits change;
 *              every call leaves them at zero)
 * The other arguments are those of oscar_decode.
 */
/* Split count for oscar_decode_multi at these sizes: the one-launch count when the grid can
 * fit the chip at once, else oscar_default_splits. Host only; 1 for invalid arguments. */
int32_t oscar_decode_multi_splits(const oscar_layer_desc* desc, int32_t batch, int32_t n_tokens, int32_t max_hist_len);
int32_t oscar_decode_multi(const oscar_layer_desc* desc, const void* q, int32_t n_tokens, const void* rot_k,
                           const void* rot_v, const void* pool, const int32_t* block_table, int32_t max_pages,
                           const int32_t* hist_len, const void* k_win, const void* v_win, const int32_t* win_len,
                           int32_t batch, float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                           float* out, void* stream);

/*
 * oscar_prepare: the first launch of oscar_decode_step on its own: the n demotions, the
 * BF16 window pass and the query rotation, written into the workspace (and the pool).
 * Arguments as in oscar_decode_step. A later oscar_attend with the same desc, batch,
 * n_splits and workspace completes the step.
 */
int32_t oscar_prepare(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                      const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k, const float* clip_v,
                      const void* q, const void* rot_k, const void* rot_v, void* pool, const void* k_win,
                      const void* v_win, const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * oscar_attend: the second launch of oscar_decode_step on its own: the INT2 history pass
 * of every split, then for each (request, KV head) the merge with the window partials
 * that oscar_prepare left in the workspace, the R_V^T un-rotation and the output. It
 * only reads the workspace's prepared data, so it may be repeated without a new
 * oscar_prepare.
 */
int32_t oscar_attend(const oscar_layer_desc* desc, const void* rot_v, const void* pool, const int32_t* block_table,
                     int32_t max_pages, const int32_t* hist_len, int32_t batch, int32_t n_splits, void* workspace,
                     size_t workspace_bytes, float* out, void* stream);

/*
 * oscar_decode_dense_bf16: plain BF16 decode attention over a dense, uncompressed KV buffer:
 * the baseline the INT2 path is measured against (the pages compare OSCAR's decode speed with
 * a BF16 cache at the same context: QbitAI article on OSCAR, system section). Not part of the
 * OSCAR path; it runs the BF16 window pass's device code over the whole context in splits of
 * 64 tokens, then the merge with no INT2 part.
 *   q         bf16 [batch][n_q_heads][128]
 *   k, v      bf16 [batch][n_kv_heads][capacity][128]; request b's tokens at [0, len[b])
 *   len       int32 [batch], 0..capacity (device)
 *   capacity  a positive multiple of 64, at most 64 * 65535
 *   workspace at least oscar_dense_workspace_bytes(desc, batch, capacity) bytes
 *   out       float32 [batch][n_q_heads][128] = softmax(sm_scale q k^T) v per query head
 */
size_t oscar_dense_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t capacity);
int32_t oscar_decode_dense_bf16(const oscar_layer_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* len, int32_t capacity, int32_t batch, float sm_scale, void* workspace,
                                size_t workspace_bytes, float* out, void* stream);

/*
 * oscar_calib_covariances: the offline calibration statistics of one layer, from one
 * calibration sequence of n_tokens tokens, on the GPU.
 * (QbitAI article on OSCAR, section on aiming the rotation at attention: the key rotation's
 * U comes from the eigenvectors of the query covariance Q^T Q, the value rotation's from the
 * score-weighted value covariance V^T S^T S V, S the attention scores; both are estimated
 * offline on calibration data.)
 *
 * For each KV head kv, with G = n_q_heads / n_kv_heads and the query heads h of its group:
 *   sigma_k[kv] = sum_h sum_t q[t, h]^T q[t, h]
 *   sigma_v[kv] = sum_h (S_h V)^T (S_h V),  S_h[t, u] = softmax over u <= t of
 *                 sm_scale * q[t, h] . k[u, kv]  (causal), V = v[:, kv]
 * in fp32 (products of the bf16 inputs are exact; sums in fp32; exp in fp32).
 *   q          bf16 [n_tokens][n_q_heads][128]
 *   k, v       bf16 [n_tokens][n_kv_heads][128]
 *   workspace  at least oscar_calib_workspace_bytes(desc, n_tokens) bytes (the attention
 *              outputs S_h V and partial Gram sums, fp32); q, k, v and workspace 16-byte aligned
 *   sigma_k, sigma_v  float32 [n_kv_heads][128][128], written (exactly symmetric)
 *   n_tokens   1..65536 (OSCAR_ERR_UNSUPPORTED above)
 * The eigendecomposition that turns sigma into U, and R = U * H * P, is host work on
 * 128 x 128 matrices (not done here).
 */
size_t oscar_calib_workspace_bytes(const oscar_layer_desc* desc, int32_t n_tokens);
int32_t oscar_calib_covariances(const oscar_layer_desc* desc, const void* q, const void* k, const void* v,
                                int32_t n_tokens, float sm_scale, void* workspace, size_t workspace_bytes,
                                float* sigma_k, float* sigma_v, void* stream);

/*
 * oscar_read_probe: a measurement helper, not part of the method: reads `bytes` bytes of
 * device memory at `buf` (both multiples of 16) with a streaming kernel and writes
 * oscar_read_probe_words() uint32 words (an XOR of what was read) to `out`. Its time over a
 * buffer much larger than the last-level cache is the box's measured read ceiling, against
 * which the decode kernels' achieved bandwidth is also reported.
 */
int32_t oscar_read_probe_words(void);
int32_t oscar_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/*
 * Lloyd-Max codebook variant (QbitAI article on OSCAR, section comparing OSCAR with
 * TurboQuant: the code release pairs the attention-aware rotation with a Lloyd-Max
 * codebook in place of the uniform INT2 levels; the article gives nothing beyond that
 * name, so the format below is this library's reading).
 *
 *   codebook   uint8 [n_kv_heads][2][4], device memory, 4-byte aligned: entry
 *              [h][0][c] is level c of KV head h's K codebook, [h][1][c] of its V codebook,
 *              in sixteenths of the group's scale. Levels must be strictly increasing and
 *              within [0, 48] (other values give undefined results, never a fault). The
 *              uniform INT2 levels are 0, 16, 32, 48.
 *
 * Scale and zero point are those of the uniform scheme (same clip, s = (hi - lo) / 3,
 * fp16 each, decided exactly as in oscar_demote). A code c stands for z + s * k_c / 16
 * in the rotated basis, and the code of y is the nearest level to t = (y - z) / s, with
 * the even index at a midpoint between two levels (for the uniform levels: round half to
 * even, clamped to [0, 3]); every code is 0 when s == 0. The near-boundary exemption of
 * oscar_demote's matrix-core path applies to the midpoints between levels. The pool layout
 * is unchanged; a pool must be written and read with the same codebook.
 *
 * Each entry point below is the one named without the suffix with `codebook` added (a
 * null or misaligned codebook returns OSCAR_ERR_INVALID_ARG); every other argument and
 * rule is that entry point's.
 */
int32_t oscar_demote_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                              const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                              const float* clip_k, const float* clip_v, const uint8_t* codebook, void* pool,
                              void* stream);

int32_t oscar_decode_step_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                   const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                   const float* clip_v, const void* q, const void* rot_k, const void* rot_v,
                                   const uint8_t* codebook, void* pool, const int32_t* block_table,
                                   int32_t max_pages, const int32_t* hist_len, const void* k_win, const void* v_win,
                                   const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                                   void* workspace, size_t workspace_bytes, float* out, void* stream);

int32_t oscar_decode_codebook(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* rot_v,
                              const uint8_t* codebook, const void* pool, const int32_t* block_table,
                              int32_t max_pages, const int32_t* hist_len, const void* k_win, const void* v_win,
                              const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                              void* workspace, size_t workspace_bytes, float* out, void* stream);

int32_t oscar_prepare_codebook(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                               const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                               const float* clip_v, const void* q, const void* rot_k, const void* rot_v,
                               const uint8_t* codebook, void* pool, const void* k_win, const void* v_win,
                               const int32_t* win_len, int32_t batch, float sm_scale, int32_t n_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

int32_t oscar_decode_multi_codebook(const oscar_layer_desc* desc, const void* q, int32_t n_tokens, const void* rot_k,
                                    const void* rot_v, const uint8_t* codebook, const void* pool,
                                    const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                    const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                    float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                                    float* out, void* stream);

/* oscar_prepare_codebook must have prepared the workspace with the same codebook. */
int32_t oscar_attend_codebook(const oscar_layer_desc* desc, const void* rot_v, const uint8_t* codebook,
                              const void* pool, const int32_t* block_table, int32_t max_pages,
                              const int32_t* hist_len, int32_t batch, int32_t n_splits, void* workspace,
                              size_t workspace_bytes, float* out, void* stream);

/* ---------------------------------------------------------------- grouped pages
 * Quantisation groups of G = 64 or 32 rotated dims (desc->group_size; 128 gives the
 * one-group codes and scales in the grouped page layout below). Method: OSCAR, QbitAI
 * article, section on aiming the rotation at attention (the bit-reversal in R balances the
 * INT2 groups; scale and zero point per group).
 *
 * Grouped page layout, per head block of 4096 + 512 n_g bytes (n_g = 128 / G): the K and V
 * codes exactly as in the one-group layout (bytes 0..4095); then the K (s16, z16) pair of
 * slot t and group g at 4096 + 4 (n_g t + g); then the V pairs, from 4096 + 256 n_g, the
 * same way. Group g covers rotated dims [g G, g G + G). Pages written by one layout are
 * read only by the same layout.
 */

/* oscar_demote into grouped pages: each rotated, clipped vector takes one (scale, zero
 * point) per group, from that group's extremes. Arguments, ownership and errors as
 * oscar_demote; pool holds pages of oscar_page_bytes(desc) bytes. */
int32_t oscar_demote_grouped(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                             const int32_t* dst_page, const int32_t* dst_slot, const void* rot_k, const void* rot_v,
                             const float* clip_k, const float* clip_v, void* pool, void* stream);

/* INT2 history pass over grouped pages: each code dequantises with its own group's scale
 * and zero point. Arguments as oscar_decode_int2, with partials in the same format (so
 * oscar_decode_bf16 and oscar_merge complete the decode), the same per-split page limit
 * (ceil(max_pages / n_splits) <= 8192, else OSCAR_ERR_UNSUPPORTED); q and rot_k must be
 * 16-byte aligned (else OSCAR_ERR_INVALID_ARG). The matrix-core pass of oscar_decode_int2
 * with one K product per group (the query's limbs masked to the group's dims), the
 * per-group V scales folded into per-group softmax weights and per-group zero-point sums;
 * query heads in tiles of four. Its scores take the 22-bit fixed-point query in both terms
 * of the fold (qsc Q . (s c + z) per group), where the one-group pass takes the exact
 * sum of the rotated query for the zero-point term. */
int32_t oscar_decode_int2_grouped(const oscar_layer_desc* desc, const void* q, const void* rot_k, const void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  int32_t batch, float sm_scale, int32_t n_splits, void* partials,
                                  size_t partials_bytes, void* stream);

/* One decode step over grouped pages in two launches on `stream`, as oscar_decode_step:
 * prepare (oscar_demote_grouped's rows for the n tokens, the BF16 window pass, the query
 * preparation), then attend (the grouped INT2 pass of oscar_decode_int2_grouped, each
 * split writing its partial, the last arrival per (request, KV head) merging). The result
 * is that of oscar_demote_grouped, oscar_decode_bf16, oscar_decode_int2_grouped and
 * oscar_merge in that order. Arguments, limits (n_splits 1..256, ceil(max_pages /
 * n_splits) <= 8192), errors and workspace (oscar_decode_workspace_bytes(desc, batch,
 * n_splits) bytes, the same size as for a one-group desc, no initialisation needed) as
 * oscar_decode_step. */
int32_t oscar_decode_step_grouped(const oscar_layer_desc* desc, const void* k_src, const void* v_src, int32_t n,
                                  const int32_t* dst_page, const int32_t* dst_slot, const float* clip_k,
                                  const float* clip_v, const void* q, const void* rot_k, const void* rot_v, void* pool,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* hist_len,
                                  const void* k_win, const void* v_win, const int32_t* win_len, int32_t batch,
                                  float sm_scale, int32_t n_splits, void* workspace, size_t workspace_bytes, float* out,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_KV_H */
