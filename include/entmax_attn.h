/*
 * entmax_attn.h -- C ABI of the MI355X (gfx950) 1.5-entmax attention library.
 *
 * Method: "ADASPLASH -- ROBERTA Benchmark Result" (AdaSplash Attention module
 * specification), section 2.2 Theorem 1: each row of scores
 * s_ij = q_i . k_j / sqrt(d) is mapped to p_ij = [(s_ij - tau_i)/2]_+^2 with
 * the row threshold tau_i fixed by sum_j p_ij = 1; the attention output is
 * O_i = sum_j p_ij v_j ("RoBERTa Base with AdaSplash Attention" model card,
 * Architecture Overview).  tau_i is found by 25 bisection steps on the
 * bracket [max_j s_ij - 2, max_j s_ij - 2/sqrt(n_i)] ("DistilBERT SST-2 with
 * AdaSplash Attention" model card, Mathematical Formulation 2), n_i being
 * the number of keys row i may attend.
 *
 * Conventions shared by every entry point (the row-wise and decode-time
 * calls further down state their own shapes, masks and options):
 *  - All tensor pointers are DEVICE memory, allocated and owned by the
 *    caller, contiguous, row-major.  q, k, v, dout: [B, H, L, d] of `dtype`;
 *    out, dq, dk, dv: [B, H, L, d] float32; tau: [B, H, L] float32;
 *    key_mask: [B, L] uint8 (nonzero = the key may be attended), or NULL for
 *    "all keys valid".  Pointers to [.., d] rows must be 16-byte aligned,
 *    tau, probs and seqlens 4-byte aligned; a misaligned pointer returns
 *    ENTMAX_ERR_INVALID_ARG before anything is launched.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is only enqueued; nothing synchronises.  The library allocates and
 *    frees no memory and keeps no state between calls; calls on different
 *    streams may run concurrently as long as their outputs do not overlap.
 *  - Masking ("ADASPLASH -- ROBERTA Benchmark Result", section 3): key j is
 *    allowed for query i iff key_mask[b][j] != 0, and, when causal != 0,
 *    j <= i, and, when window > 0, j > i - window (the splash window, which
 *    the pages use for causal decoders only: window > 0 requires causal).
 *    Disallowed keys are removed from the simplex (p = 0 exactly).
 *  - A query row with no allowed key gets O = 0 and tau = +inf.  Padded
 *    query rows are computed like any other row.
 *  - Inputs must be finite (not checked).  Scale is fixed to 1/sqrt(d) and
 *    the bisection to 25 steps; alpha is 1.5 except in the row-wise
 *    entmax_bisect_rows_* calls, which take it.
 *  - Supported: d in {64, 128}; dtype ENTMAX_F32 or ENTMAX_BF16;
 *    1 <= L <= 65536.  Other values return ENTMAX_ERR_UNSUPPORTED.
 *  - Errors: integer status codes; nothing is launched when the arguments
 *    are rejected.  ENTMAX_ERR_HIP means a launch failed (see
 *    entmax_attn_last_error()); faults inside a kernel surface at the
 *    caller's next synchronisation.
 */
#ifndef ENTMAX_ATTN_H
#define ENTMAX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum entmax_status {
    ENTMAX_OK = 0,
    ENTMAX_ERR_INVALID_ARG = 1,   /* NULL required pointer, size <= 0, window < 0, window without causal */
    ENTMAX_ERR_UNSUPPORTED = 2,   /* d, dtype or L outside the supported set */
    ENTMAX_ERR_HIP = 3            /* a HIP launch failed */
};

enum entmax_dtype {
    ENTMAX_F32 = 0,
    ENTMAX_BF16 = 1
};

/*
 * Forward pass.  Writes out[b,h,i,:] = sum_j p_ij v[b,h,j,:] (float32) and,
 * when tau_out is not NULL, tau_out[b,h,i] = tau_i in score units (so that
 * p_ij = [(s_ij - tau_i)/2]_+^2).
 * Required: q, k, v, out.  Optional: key_mask, tau_out.
 */
int entmax_attn_fwd(const void *q, const void *k, const void *v,
                    const uint8_t *key_mask, int causal, int window,
                    float *out, float *tau_out,
                    int B, int H, int L, int d, int dtype, void *stream);

/*
 * Backward pass from the forward's tau ("ADASPLASH -- ROBERTA Benchmark
 * Result", section 2.4 Jacobian): with w_ij = sqrt(p_ij),
 * dp_ij = dout_i . v_j, c_i = sum_j w_ij dp_ij / sum_j w_ij and
 * dS_ij = w_ij (dp_ij - c_i):  dq = dS k / sqrt(d), dk = dS^T q / sqrt(d),
 * dv = p^T dout.  dq, dk, dv are overwritten (float32).
 * Required: q, k, v, tau, dout, dq, dk, dv, workspace.  Optional: key_mask.
 *  - workspace: caller-owned DEVICE memory, 256-byte aligned, of at least
 *    entmax_attn_bwd_workspace_bytes(B, H, L, d) bytes (c_i of every query
 *    row, a support counter per key, a flag: 8 B H L bytes plus at most
 *    768); no initialisation needed, scratch after the call.  Two calls in
 *    flight must not share a workspace.  A too small or misaligned
 *    workspace returns ENTMAX_ERR_INVALID_ARG.
 *  - dk and dv serve as scratch until the call completes (for key spans
 *    above 2048, each key's support entries are collected in its own rows).
 *  - Deterministic: every row of dq, dk and dv is summed by one thread
 *    group in an order fixed by the data (query rows by key index, key rows
 *    by query index), never by float atomics, so repeated calls on the same
 *    inputs give identical bits.
 */
size_t entmax_attn_bwd_workspace_bytes(int B, int H, int L, int d);
int entmax_attn_bwd(const void *q, const void *k, const void *v,
                    const uint8_t *key_mask, int causal, int window,
                    const float *tau, const void *dout,
                    float *dq, float *dk, float *dv,
                    int B, int H, int L, int d, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense attention weights for inspection and tests: probs[b,h,i,j] =
 * [(s_ij - tau[b,h,i])/2]_+^2 for allowed (i, j), 0 otherwise
 * ([B, H, L, L] float32), recomputing s from q and k exactly as the forward
 * does.  Required: q, k, tau, probs.  Optional: key_mask.
 */
int entmax_attn_probs(const void *q, const void *k,
                      const uint8_t *key_mask, int causal, int window,
                      const float *tau, float *probs,
                      int B, int H, int L, int d, int dtype, void *stream);

/*
 * Grouped-query variants ("ADASPLASH -- ROBERTA Benchmark Result", section 3,
 * Step-by-Step Tensor Execution Trace: K and V have H_kv heads, each repeated
 * for H / H_kv consecutive query heads).  k, v: [B, H_kv, L, d]; query head
 * h uses key/value head h / (H / H_kv).  dk, dv: [B, H_kv, L, d], each the
 * sum over the query heads of its group (in head order).  The backward's
 * workspace is sized as for the call above (by the H query heads).  H_kv
 * must divide H (else ENTMAX_ERR_INVALID_ARG).  With H_kv = H these are the
 * calls above, which are implemented through them.
 */
int entmax_attn_fwd_gqa(const void *q, const void *k, const void *v,
                        const uint8_t *key_mask, int causal, int window,
                        float *out, float *tau_out,
                        int B, int H, int H_kv, int L, int d, int dtype, void *stream);
int entmax_attn_bwd_gqa(const void *q, const void *k, const void *v,
                        const uint8_t *key_mask, int causal, int window,
                        const float *tau, const void *dout,
                        float *dq, float *dk, float *dv,
                        int B, int H, int H_kv, int L, int d, int dtype,
                        void *workspace, size_t workspace_bytes, void *stream);
int entmax_attn_probs_gqa(const void *q, const void *k,
                          const uint8_t *key_mask, int causal, int window,
                          const float *tau, float *probs,
                          int B, int H, int H_kv, int L, int d, int dtype, void *stream);

/*
 * Forward that also keeps each query row's support for the backward (the
 * keys with p_ij > 0: the sparse aggregation of the "RoBERTa Base with
 * AdaSplash Attention" model card, Architecture Overview), so that
 * entmax_attn_bwd_saved finds them without recomputing the scores.  Same
 * arguments and results as entmax_attn_fwd_gqa, plus:
 *  - tau_out is required.
 *  - saved: caller-owned DEVICE memory, 256-byte aligned, of at least
 *    entmax_attn_saved_bytes(B, H, L, d) bytes: per query row a count
 *    (int32, -1 where the row was finished by the recompute fix-up and is
 *    not kept; the counts first, 256-byte aligned), then d/2 entries per
 *    row of 8 bytes each (float w_ij = sqrt(p_ij), uint32 key index), in
 *    the order the forward summed them.  Written only where the key span
 *    exceeds 2048 keys (the wide kernels); elsewhere left untouched.  No
 *    initialisation needed; it must stay unchanged until the matching
 *    entmax_attn_bwd_saved.  A too small or misaligned buffer returns
 *    ENTMAX_ERR_INVALID_ARG.
 * entmax_attn_saved_bytes returns 0 for non-positive sizes.
 */
size_t entmax_attn_saved_bytes(int B, int H, int L, int d);
int entmax_attn_fwd_save(const void *q, const void *k, const void *v,
                         const uint8_t *key_mask, int causal, int window,
                         float *out, float *tau_out, void *saved, size_t saved_bytes,
                         int B, int H, int H_kv, int L, int d, int dtype, void *stream);

/*
 * entmax_attn_bwd_gqa on the support kept by entmax_attn_fwd_save, called
 * with the same q, k, v, key_mask, causal, window and tau: the query side
 * reads each row's support instead of recomputing the scores (rows without
 * a kept support are recomputed, as the rows whose support overflows in
 * entmax_attn_bwd_gqa).  Where the key span is at most 2048 keys it is
 * entmax_attn_bwd_gqa.  Arguments, workspace, results and determinism as
 * entmax_attn_bwd_gqa (w comes from the forward's own arithmetic, so the
 * results agree with entmax_attn_bwd_gqa's to rounding, not bit for bit);
 * saved and saved_bytes as above.
 */
int entmax_attn_bwd_saved(const void *q, const void *k, const void *v,
                          const uint8_t *key_mask, int causal, int window,
                          const float *tau, const void *dout,
                          const void *saved, size_t saved_bytes,
                          float *dq, float *dk, float *dv,
                          int B, int H, int H_kv, int L, int d, int dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/* entmax_attn_bwd_noalloc: entmax_attn_bwd_gqa for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * determinism, without the workspace: c_i lives in a scratch array built
 * into the library (8 MiB + 256 bytes per GPU, held from the library's
 * first use on that GPU until the process ends; its address is looked up
 * once per device, on the first call there).
 *  - B * H * L above 1048576 query rows returns ENTMAX_ERR_INVALID_ARG.
 *  - Calls no hipMalloc, hipFree or allocating library routine.
 *  - All calls on one GPU share its scratch: two calls in flight at once on
 *    one GPU (other streams, other host threads) race and give undefined
 *    results.  Calls on one stream are ordered and safe.
 */
int entmax_attn_bwd_noalloc(const void *q, const void *k, const void *v,
                            const uint8_t *key_mask, int causal, int window,
                            const float *tau, const void *dout,
                            float *dq, float *dk, float *dv,
                            int B, int H, int H_kv, int L, int d, int dtype,
                            void *stream);

/*
 * Row-wise 1.5-entmax as an op of its own (the pages' entmax15_bisect
 * export, "ADASPLASH -- ROBERTA Benchmark Result", section 4), with the same
 * threshold as the attention calls: scores [R, L] (dtype ENTMAX_F32 or
 * ENTMAX_BF16, row-major), mask [R, L] uint8 (nonzero = allowed) or NULL,
 * p [R, L] float32 with p_j = [(s_j - tau)/2]_+^2 over the allowed entries
 * (0 elsewhere), tau [R] float32 in score units or NULL.  A row without an
 * allowed entry gets p = 0 and tau = +inf.  L must be a multiple of 4
 * (ENTMAX_ERR_UNSUPPORTED otherwise); pointers 16-byte aligned.  Rows of up
 * to 4096 entries are solved in registers; longer rows are re-read from
 * memory at each of the 25 bisection steps.
 */
int entmax15_rows_fwd(const void *scores, const uint8_t *mask, float *p, float *tau,
                      int R, int L, int dtype, void *stream);

/*
 * Its backward (section 2.4 Jacobian): ds_j = w_j (dp_j - sum_k w_k dp_k /
 * sum_k w_k) with w = sqrt(p); p, dp, ds [R, L] float32 (ds overwritten).
 */
int entmax15_rows_bwd(const float *p, const float *dp, float *ds, int R, int L, void *stream);

/*
 * The same for a general alpha in (1, 2] (section 2.1 defines alpha-entmax
 * through the Tsallis entropy; section 4 gives its bisection): p_j =
 * [(alpha - 1)(s_j - tau)]_+^(1/(alpha - 1)) over the allowed entries with
 * sum p = 1, tau in score units, 25 bisection steps on the bracket
 * [max - 1/(alpha-1), max - n^(1-alpha)/(alpha-1)].  alpha = 2 is sparsemax;
 * alpha = 1.5 gives the calls above (which are these with alpha = 1.5).
 * Backward: ds_j = w_j (dp_j - sum_k w_k dp_k / sum_k w_k), w = p^(2 - alpha)
 * on the support.  alpha outside (1, 2] returns ENTMAX_ERR_INVALID_ARG.
 */
int entmax_bisect_rows_fwd(const void *scores, const uint8_t *mask, float *p, float *tau,
                           int R, int L, float alpha, int dtype, void *stream);
int entmax_bisect_rows_bwd(const float *p, const float *dp, float *ds, int R, int L, float alpha,
                           void *stream);

/*
 * Decode-time forward: the newest Lq queries of each sequence against a
 * key/value cache (the causal decoders of "ADASPLASH -- ROBERTA Benchmark
 * Result", section 3, with the splash window of the decoder configuration in
 * section 7.1).  Lq = 1 is one decode step; Lq > 1 a chunk of new tokens
 * (query length below key length).
 *
 *  - q: [B, H, Lq, d] of `dtype`, the new tokens' queries per head.
 *  - k_cache, v_cache: [B, H_kv, S, d] of `dtype` (H_kv divides H; query head
 *    h reads key/value head h / (H / H_kv)).
 *  - seqlens: [B] int32, DEVICE memory: sequence b holds n_b = seqlens[b]
 *    valid cache positions, the new tokens' own keys and values included
 *    (values outside [0, S] are clamped to it).  causal != 0: query i sits
 *    at position n_b - Lq + i and may attend keys j <= n_b - Lq + i, and
 *    with window W > 0 only keys j > n_b - Lq + i - W (W keys including its
 *    own).  causal == 0: every query may attend all n_b keys (window must
 *    be 0).
 *  - out: [B, H, Lq, d] float32; tau_out: [B, H, Lq] float32 (score units) or
 *    NULL.  A query with no key to attend (n_b - Lq + i < 0) gets O = 0 and
 *    tau = +inf.
 *  - workspace: caller-owned DEVICE memory, 256-byte aligned, of at least
 *    entmax_attn_decode_workspace_size(B, H, H_kv, Lq, S, d, window) bytes
 *    (scores of the span, per-chunk maxima, partial outputs); its contents
 *    need no initialisation and are scratch after the call.  Two calls in
 *    flight must not share a workspace.
 *  - Supported: d in {64, 128}; dtype ENTMAX_F32 or ENTMAX_BF16;
 *    1 <= Lq <= S <= 2^24; B * H_kv <= 65535.  A too small or misaligned
 *    workspace, or a window without causal, returns ENTMAX_ERR_INVALID_ARG.
 * entmax_attn_decode_workspace_size returns 0 for non-positive sizes or an
 * H_kv that does not divide H.
 */
size_t entmax_attn_decode_workspace_size(int B, int H, int H_kv, int Lq, int S, int d, int window);
int entmax_attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens,
                       int causal, int window, float *out, float *tau_out, void *workspace,
                       size_t workspace_bytes, int B, int H, int H_kv, int Lq, int S, int d, int dtype,
                       void *stream);

/*
 * Backward of the decode-time forward (query length below key length),
 * from the forward's tau ("ADASPLASH -- ROBERTA Benchmark Result", section
 * 2.4 Jacobian over the rows of section 3's decoders): per query row,
 * w_j = sqrt(p_j), dp_j = dout . v_j, c = sum w dp / sum w,
 * dS_j = w_j (dp_j - c); dq = dS k / sqrt(d), and every key j of the row's
 * key/value head gets dS_j q / sqrt(d) in dk and p_j dout in dv.
 *  - q, k_cache, v_cache, seqlens, causal, window, B, H, H_kv, Lq, S, d,
 *    dtype: as for entmax_attn_decode (the same call's arguments).
 *  - tau: [B, H, Lq] float32, the forward's tau_out.  dout: [B, H, Lq, d] of
 *    `dtype`.  dq: [B, H, Lq, d], dk and dv: [B, H_kv, S, d], float32,
 *    overwritten; keys that no query may attend (past n_b, or outside every
 *    window) get zero; dk and dv of a shared key/value head sum its query
 *    heads.
 *  - workspace: caller-owned DEVICE memory, 256-byte aligned, of at least
 *    entmax_attn_decode_bwd_workspace_size(B, H, H_kv, Lq, S, d, window)
 *    bytes (scores and dS of every row's span); scratch after the call.
 *  - Deterministic: every row of dq, dk and dv is summed by one wave in a
 *    fixed order (no atomics).
 *  - Errors as entmax_attn_decode.
 */
size_t entmax_attn_decode_bwd_workspace_size(int B, int H, int H_kv, int Lq, int S, int d, int window);
int entmax_attn_decode_bwd(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens,
                           int causal, int window, const float *tau, const void *dout,
                           float *dq, float *dk, float *dv, void *workspace, size_t workspace_bytes,
                           int B, int H, int H_kv, int Lq, int S, int d, int dtype, void *stream);

const char *entmax_attn_status_string(int status);

/* Message describing the most recent failure on the calling thread
 * (thread-local storage, valid until the next call on that thread). */
const char *entmax_attn_last_error(void);

/* Library ABI version (incremented on incompatible changes). */
int entmax_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAX_ATTN_H */
