/*
 * parallax.h -- C ABI of the MI355X (gfx950) Parallax attention library.
 *
 * Parallax (parameterized Local Linear Attention) keeps softmax attention's
 * weights and adds a correction read from the key/value covariance by a
 * learned probe rho_i = x_i W_R, in place of Local Linear Attention's
 * per-token linear solve (review page "Parallax: Parameterized Local Linear
 * Attention for Language Modeling", sec. 1 "Key Terms & Definitions" and
 * sec. 3 "Method & Key Results"; tilnote note on Parallax, section on its
 * starting point, Local Linear Attention).  For query position i with visible
 * key set V(i):
 *
 *     p_ij   = softmax_j (scale * q_i . k_j)           over j in V(i)
 *     kbar_i = sum_j p_ij k_j
 *     o_i    = sum_j p_ij (1 + rho_i . (k_j - kbar_i)) v_j
 *     lse_i  = log sum_{j in V(i)} exp(scale * q_i . k_j)    (natural log)
 *
 * The probe term carries no softmax scale.  Visible set (causal, optional
 * sliding window and attention sinks; "Sliding-window beats linear
 * attention" review, sec. 1):
 *
 *     j in V(i)  iff  j <= i  and  (window == 0 or i - j < window or j < n_sink)
 *
 * so a window of W keys includes the query's own key, and sink keys are
 * still causal.
 *
 * Conventions shared by every entry point:
 *   - Inputs q, k, v, r are bfloat16 (raw 16-bit storage, passed as void*);
 *     outputs o and lse are float32.  The feature dimension d is 64 or 128.
 *   - All pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises.  The prefill takes a device
 *     workspace from the caller (parallax_attn_fwd_workspace_size); its
 *     contents need no initialisation and are scratch once the call's
 *     work on `stream` has finished.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously.  Calls are stateless and thread-safe.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     non-OK status means nothing was launched and no output was touched.
 *     PARALLAX_ERR_LAUNCH reports a failed kernel launch.
 *   - Outputs must not alias inputs.  Non-finite inputs give undefined
 *     results.
 *   - Accuracy of the prefill.  Its value products take the values and two
 *     weights per key as float16 matrix-core operands: the un-normalised
 *     softmax weight p~ (at most 2^5) and p~ * rho_i.k_j, each rounded once
 *     (relative error up to 2^-11).  A perturbation of the softmax weights
 *     moves the probe correction in proportion to the probe scores, so the
 *     O error of row i grows with R_i = max over j in V(i) of
 *     |rho_i . k_j|.  Against the exact result on the same bf16 inputs,
 *     parallax_attn_fwd and parallax_attn_fwd_train stay within
 *         2e-2 * max(1, R_i / 24)
 *     for values of unit scale (the bound scales with |v|); this is tested
 *     at R = 24, 256 and 2000 with diffuse and with concentrated attention,
 *     d = 64 and 128, causal and windowed with sinks.  The five reference
 *     workloads (i.i.d. N(0,1) inputs, R up to about 70) stay within 2e-2.
 *     parallax_attn_fwd_precise passes each weight as the sum of two
 *     float16 values (its rounding and the rounded residual, about 22
 *     significant bits), which doubles the matrix-core work of the value
 *     products (the kernel's grows 1.5 times), and stays within
 *         2e-2 * max(1, R_i / 256)
 *     (tested at R = 256 and 2000, same cases).  What limits it is the fp32
 *     rounding of the scores q.k themselves: where a row's weight is split
 *     between keys whose probe scores differ by about R_i, one rounding
 *     step of a score moves o_i by about R_i |v| times that step.
 *   - Range.  float16 holds at most 65504, so |v| must stay at or below it
 *     and, in the prefill, |rho_i . k_j| below 2047 (2^5 * 2047 < 65504);
 *     beyond that the f16 weights overflow and the affected rows' outputs
 *     are infinite or NaN (not finite and wrong).
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PARALLAX_OK = 0,
    PARALLAX_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, bad stride,
                                     negative window or n_sink, scale not > 0 and finite */
    PARALLAX_ERR_UNSUPPORTED = 2, /* d not in {64,128}, num_splits not in {1,2,4,8,16},
                                     problem too large for the launch grid */
    PARALLAX_ERR_LAUNCH = 3       /* the HIP runtime rejected the kernel launch */
} parallax_status;

/* Element strides (not bytes) of a [B, H, L, d] tensor along B, H and L.
 * The d dimension must be contiguous (stride 1). */
typedef struct {
    int64_t b, h, l;
} parallax_strides;

/*
 * Bytes of device workspace parallax_attn_fwd needs for these sizes: the
 * values converted to float16 and laid out per 32-key stage,
 * I = B * H * ceil(L / 32) * 32 * d * 2 bytes, then 256 bytes of counters
 * (I + 256 in all; 0 when B, H or L is 0).  Returns 0 for sizes
 * parallax_attn_fwd would reject (negative sizes, d not in {64, 128}).
 *
 * Diagnostics: once a call's work has finished, the 4 bytes at offset I of
 * its workspace hold, as an unsigned 32-bit integer, the number of
 * 128-row query tiles whose workgroup took the exact second pass (the
 * first pass fixes each row's softmax offset at its first stage; a row
 * whose scores later rise more than 2^5 above it makes its tile repeat
 * with the exact row maximum).  Calls that take the windowed kernel (a
 * window of at most 128 keys with at most 32 sinks) recompute per
 * 16-row wavefront and leave these bytes unwritten.
 */
size_t parallax_attn_fwd_workspace_size(int B, int H, int L, int d);

/*
 * Causal prefill forward.
 *
 *   q, k, v, r : bf16 tensors of logical shape [B, H, L, d] with strides
 *                sq, sk, sv, sr (r is the probe rho = x W_R, one row per
 *                query position).  Base pointers 16-byte aligned; every
 *                stride a multiple of 8 elements.
 *   o          : fp32 [B, H, L, d] with strides so (16-byte aligned; strides
 *                multiples of 4 elements).
 *   lse        : fp32 [B, H, L], contiguous (4-byte aligned).
 *   B, H, L    : >= 0; if any is 0 the call returns PARALLAX_OK and does
 *                nothing.
 *   d          : 64 or 128.
 *   softmax_scale : multiplies q.k only (usually 1/sqrt(d)); must be > 0
 *                and finite.
 *   window     : 0 = plain causal; W > 0 = key j visible iff i - j < W
 *                (or j is a sink).  Must be >= 0.
 *   n_sink     : number of leading sink keys (always visible once causal);
 *                >= 0; only matters when window > 0.
 *   workspace  : device memory of at least workspace_bytes >=
 *                parallax_attn_fwd_workspace_size(B, H, L, d) bytes, 16-byte
 *                aligned, not aliasing any input or output; NULL is allowed
 *                only when that size is 0.  Two calls in flight at once need
 *                two workspaces.
 *
 * Two kernels run on `stream`: the first converts v into the workspace,
 * the second computes o and lse.
 */
parallax_status parallax_attn_fwd(const void *q, const void *k, const void *v, const void *r,
                                  float *o, float *lse,
                                  int B, int H, int L, int d,
                                  parallax_strides sq, parallax_strides sk,
                                  parallax_strides sv, parallax_strides sr,
                                  parallax_strides so,
                                  float softmax_scale, int window, int n_sink,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * Causal prefill forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): parallax_attn_fwd without the workspace arguments.  The
 * library keeps the workspace itself, in one device array of 64 MiB + 256
 * bytes (67109120 bytes) per GPU that holds it until the process ends;
 * this call allocates and frees nothing.  The array of the current device is used,
 * so `stream` must belong to that device.
 *
 *   Sizes whose workspace (parallax_attn_fwd_workspace_size) exceeds that
 *   -- e.g. more than 2 x 16 heads x 8192 tokens at d = 128 -- return
 *   PARALLAX_ERR_UNSUPPORTED.  Every call on a GPU shares that GPU's array
 *   and overwrites it in full before reading it (no contents carry over
 *   between calls), so two calls whose work overlaps on one GPU (other
 *   streams, other host threads) race and give wrong results: order them.
 *   Other arguments, outputs and errors as for parallax_attn_fwd;
 *   PARALLAX_ERR_LAUNCH also reports a failed lookup of the array.
 */
parallax_status parallax_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                          const void *r, float *o, float *lse, int B, int H,
                                          int L, int d, parallax_strides sq, parallax_strides sk,
                                          parallax_strides sv, parallax_strides sr,
                                          parallax_strides so, float softmax_scale, int window,
                                          int n_sink, void *stream);

/*
 * Causal prefill forward in fp32, for fp32 inputs: the same operation as
 * parallax_attn_fwd (same visible set, scale, outputs), with every product,
 * exponential and sum taken in fp32 (expf, logf) instead of bf16/f16
 * matrix-core operands, so the inputs keep their fp32 precision (the bf16
 * rounding of fp32 inputs alone moves o by about 0.07 on the tiny reference
 * workload).  Against the exact result it is accurate to fp32 rounding
 * (about 1e-5 relative).  It is untiled: O(L^2 d) arithmetic per head and
 * one wavefront per query row, meant for small problems; large ones belong
 * on parallax_attn_fwd.
 *
 *   q, k, v, r : fp32 [B, H, L, d] with strides sq, sk, sv, sr (element
 *                strides >= 0; d contiguous; 4-byte aligned).
 *   o          : fp32 [B, H, L, d] with strides so (4-byte aligned).
 *   lse        : fp32 [B, H, L], contiguous (4-byte aligned).
 *   B, H, L, d, softmax_scale, window, n_sink : as for parallax_attn_fwd.
 *
 * No workspace; one kernel on `stream`.  Errors as for parallax_attn_fwd.
 */
parallax_status parallax_attn_fwd_f32(const float *q, const float *k, const float *v,
                                      const float *r, float *o, float *lse, int B, int H, int L,
                                      int d, parallax_strides sq, parallax_strides sk,
                                      parallax_strides sv, parallax_strides sr,
                                      parallax_strides so, float softmax_scale, int window,
                                      int n_sink, void *stream);

/*
 * Causal prefill forward with two-part float16 weights: the same operation,
 * arguments, workspace and errors as parallax_attn_fwd, accurate to 2e-2
 * absolute for probe scores |rho_i . k_j| up to 256, eight times the range
 * of parallax_attn_fwd (see "Accuracy of the prefill" above).  Each key's weights p~ and p~ * rho_i.k_j reach the
 * matrix cores as an f16 value plus its f16 residual, which doubles the
 * value and row-sum products (the score products are unchanged).
 */
parallax_status parallax_attn_fwd_precise(const void *q, const void *k, const void *v,
                                          const void *r, float *o, float *lse, int B, int H,
                                          int L, int d, parallax_strides sq, parallax_strides sk,
                                          parallax_strides sv, parallax_strides sr,
                                          parallax_strides so, float softmax_scale, int window,
                                          int n_sink, void *workspace, size_t workspace_bytes,
                                          void *stream);

/*
 * Prefill forward for training: parallax_attn_fwd plus two saved
 * quantities that parallax_attn_bwd needs (same arguments otherwise).
 *
 *   sbar : fp32 [B, H, L] contiguous (4-byte aligned): sbar_i =
 *          sum_j p_ij rho_i . k_j, the softmax-weighted mean of the probe
 *          scores (so that rho_i . (k_j - kbar_i) = rho_i . k_j - sbar_i).
 *   pv   : fp32 [B, H, L, d] contiguous (16-byte aligned): pv_i =
 *          sum_j p_ij v_j, the plain softmax-attention output of row i.
 *
 * o and lse are bit-identical to those of parallax_attn_fwd.
 */
parallax_status parallax_attn_fwd_train(const void *q, const void *k, const void *v,
                                        const void *r, float *o, float *lse, float *sbar,
                                        float *pv, int B, int H, int L, int d,
                                        parallax_strides sq, parallax_strides sk,
                                        parallax_strides sv, parallax_strides sr,
                                        parallax_strides so, float softmax_scale, int window,
                                        int n_sink, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Bytes of device workspace parallax_attn_bwd needs: per (b, h) and 32-row
 * stage, 512 bytes of row statistics plus five bf16 operand blocks of
 * 32 * d elements (q, r, dout, k and v), i.e.
 * B * H * ceil(L / 32) * (512 + 320 * d)
 * bytes (0 when B, H or L is 0, or for sizes parallax_attn_bwd would
 * reject).
 */
size_t parallax_attn_bwd_workspace_size(int B, int H, int L, int d);

/*
 * Prefill backward: gradients of a scalar loss through o (lse carries no
 * gradient) with respect to q, k, v and the probe r.  With
 * s_ij = rho_i . k_j, t_ij = 1 + s_ij - sbar_i, g_ij = dout_i . v_j,
 * G_i = dout_i . pv_i and Y_i = dout_i . o_i (review page "Parallax:
 * Parameterized Local Linear Attention for Language Modeling", sec. 1 and
 * sec. 3 define the forward; this is its derivative):
 *
 *     dv_j   = sum_i p_ij t_ij dout_i
 *     dS_ij  = p_ij (g_ij - G_i)
 *     dZ_ij  = p_ij ((g_ij - G_i) t_ij + G_i - Y_i)
 *     dq_i   = scale sum_j dZ_ij k_j          dr_i = sum_j dS_ij k_j
 *     dk_j   = scale sum_i dZ_ij q_i + sum_i dS_ij r_i
 *
 * over the same visible pairs as the forward.
 *
 *   q, k, v, r : the forward's bf16 inputs (same rules as parallax_attn_fwd).
 *   dout       : bf16 [B, H, L, d] with strides sdo: gradient of the loss
 *                with respect to o.
 *   o, lse, sbar, pv : the outputs of parallax_attn_fwd_train for these
 *                inputs, all contiguous (o 16-byte aligned).
 *   dq, dk, dv, dr : fp32 [B, H, L, d] contiguous, 16-byte aligned, written
 *                in full (no accumulation into existing contents).
 *   softmax_scale, window, n_sink : as passed to the forward.
 *   workspace  : at least parallax_attn_bwd_workspace_size(B, H, L, d)
 *                bytes, 256-byte aligned; scratch after the call.
 *
 * Four kernels run on `stream`: row statistics, operand blocks in the
 * workspace, then dk/dv and dq/dr.  With window > 0 and n_sink > 0 the rows past the
 * window add into the sink keys' dk and dv with float atomics, so those
 * rows of dk and dv can differ from run to run by rounding; everything
 * else is deterministic.
 */
parallax_status parallax_attn_bwd(const void *q, const void *k, const void *v, const void *r,
                                  const void *dout, const float *o, const float *lse,
                                  const float *sbar, const float *pv, float *dq, float *dk,
                                  float *dv, float *dr, int B, int H, int L, int d,
                                  parallax_strides sq, parallax_strides sk, parallax_strides sv,
                                  parallax_strides sr, parallax_strides sdo,
                                  float softmax_scale, int window, int n_sink, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Decode step: one query (and probe) per sequence against a contiguous KV
 * cache.  A decoding Parallax model reads a KV cache like softmax attention
 * does (tilnote note on Parallax, section explaining that it is a different
 * estimator and not a linear-time attention).
 *
 *   q, r       : bf16 [B, H, d], contiguous, 16-byte aligned.
 *   k_cache,
 *   v_cache    : bf16 [B, H, Lmax, d] with strides sk, sv (16-byte aligned
 *                base, strides multiples of 8 elements; row strides sk.l,
 *                sv.l below 2^24 elements, else PARALLAX_ERR_UNSUPPORTED).
 *   seqlens    : DEVICE int32 [B] or NULL (= Lmax for every sequence).  The
 *                cache already holds the current token: the query sits at
 *                position seqlen-1 and sees keys 0 .. seqlen-1.  Values are
 *                clamped to [0, Lmax]; a length of 0 gives o = 0 and
 *                lse = -inf.
 *   o          : fp32 [B, H, d] contiguous (16-byte aligned).
 *   lse        : fp32 [B, H] contiguous.
 *   B, H       : >= 0 (0 -> OK, nothing done); Lmax >= 0; d 64 or 128.
 *   softmax_scale : as for the prefill (> 0, finite).
 *   num_splits : 1, 2, 4, 8 or 16 -- the cache of each (b, h) is cut into
 *                this many contiguous chunks, processed by separate
 *                wavefronts and merged on chip.  The result does not depend
 *                on it beyond rounding.
 */
parallax_status parallax_attn_decode(const void *q, const void *r,
                                     const void *k_cache, const void *v_cache,
                                     const int32_t *seqlens,
                                     float *o, float *lse,
                                     int B, int H, int Lmax, int d,
                                     parallax_strides sk, parallax_strides sv,
                                     float softmax_scale, int num_splits,
                                     void *stream);

/*
 * General decode step: paged or contiguous KV cache, grouped kv heads
 * (GQA/MQA) and an optional sliding window with attention sinks.  The
 * arithmetic is parallax_attn_decode's; a windowed query at position
 * seqlen-1 sees keys j with seqlen-1-j < window or j < n_sink, the
 * prefill's visibility rule ("Sliding-window beats linear attention"
 * review, sec. 1: window over preceding tokens plus sink tokens kept
 * visible, which bounds the KV cache).
 *
 *   q, r       : bf16 [B, Hq, d], contiguous, 16-byte aligned.
 *   k_cache,
 *   v_cache    : bf16 caches addressed by element strides sk, sv with the
 *                fields meaning (b: page, h: kv head, l: row in the page);
 *                d contiguous, 16-byte aligned base, strides multiples of
 *                8.  A vLLM-style pool [num_pages, page_size, Hkv, d] has
 *                strides (page_size*Hkv*d, d, Hkv*d).
 *   block_table: DEVICE int32 [B, max_pages] or NULL.  Paged: key j of
 *                sequence b lives in page block_table[b*max_pages +
 *                j / page_size] at row j % page_size; page_size must be a
 *                power of two; entries for the pages that hold keys
 *                0 .. seqlen-1 must be in [0, num_pages) (others are never
 *                read; out-of-range entries are clamped into the pool, so
 *                a bad table gives wrong results, not a fault).
 *                NULL: contiguous cache, sequence b is "page" b and
 *                page_size is the cache length Lmax (num_pages and
 *                max_pages are ignored).
 *   seqlens    : DEVICE int32 [B] or NULL (= the cache length: max_pages *
 *                page_size when paged, page_size when contiguous); clamped
 *                to [0, that length].
 *   o, lse     : fp32 [B, Hq, d] and [B, Hq], contiguous.
 *   Hq, Hkv    : query and kv heads, Hq a multiple of Hkv; query head h
 *                reads kv head h / (Hq / Hkv).
 *   window, n_sink : as for the prefill (0 = no window).
 *   num_splits : 1, 2, 4, 8 or 16 key chunks per (sequence, query head),
 *                as for parallax_attn_decode.  With Hq/Hkv < 4 a workgroup
 *                serves 16 / num_splits query heads of one kv head when
 *                Hq/Hkv allows (the largest power of two dividing it), so
 *                that they share the rows they read.  With Hq/Hkv >= 4 the
 *                query heads of a kv head (up to 16 per workgroup) are the
 *                columns of matrix-core tiles and every row is read once
 *                per workgroup; the keys are split min(num_splits, 8) ways.
 *                That path feeds the values to the matrix cores as float16
 *                (|v| <= 65504) and each weight as an f16 value plus its
 *                f16 residual, like parallax_attn_fwd_precise, with the
 *                same accuracy (the online softmax keeps p~ <= 1, so
 *                |rho.k| < 65504); the other path computes in fp32.
 */
parallax_status parallax_attn_decode_paged(const void *q, const void *r,
                                           const void *k_cache, const void *v_cache,
                                           const int32_t *block_table, int num_pages,
                                           int page_size, int max_pages,
                                           const int32_t *seqlens, float *o, float *lse,
                                           int B, int Hq, int Hkv, int d,
                                           parallax_strides sk, parallax_strides sv,
                                           float softmax_scale, int window, int n_sink,
                                           int num_splits, void *stream);

/*
 * parallax_attn_decode_paged with a caller workspace: the same operation,
 * arguments, validation and results.  With four or more query heads per kv
 * head, a call that has fewer (sequence, kv head) workgroups than the GPU
 * has compute units (MQA over a small batch) splits each kv head's visible
 * keys over up to 8 workgroups whose partial states (m, ell, S, A, C per
 * query head, the same quantities the single-workgroup merge combines)
 * meet in the workspace and are merged by a second launch; otherwise the
 * workspace is not touched.  The workspace is device memory of at least
 * parallax_attn_decode_paged_workspace_size(B, Hq, d) bytes, 16-byte
 * aligned, owned by the caller; its contents need no initialisation and are
 * scratch once the call's work on `stream` has finished.  A missing,
 * misaligned or short workspace returns PARALLAX_ERR_INVALID_ARG before
 * anything is launched.
 */
size_t parallax_attn_decode_paged_workspace_size(int B, int Hq, int d);
parallax_status parallax_attn_decode_paged_ws(const void *q, const void *r,
                                              const void *k_cache, const void *v_cache,
                                              const int32_t *block_table, int num_pages,
                                              int page_size, int max_pages,
                                              const int32_t *seqlens, float *o, float *lse,
                                              int B, int Hq, int Hkv, int d,
                                              parallax_strides sk, parallax_strides sv,
                                              float softmax_scale, int window, int n_sink,
                                              int num_splits, void *workspace,
                                              size_t workspace_bytes, void *stream);

/*
 * Fused input projections: Y = X W^T with W the row-wise stack of W_Q, W_K,
 * W_V and the probe projection W_R (review page "Parallax: Parameterized
 * Local Linear Attention for Language Modeling", sec. 1 and sec. 3: the
 * probe is a learned projection of the layer input, rho_i = x_i W_R).  Row
 * i of Y is then [q_i | k_i | v_i | rho_i]; with H heads of d features each
 * part is H*d wide, and the prefill and decode entry points take the parts
 * as strided [B, H, L, d] views of Y (strides b = L*ldy, h = d, l = ldy,
 * base Y + part*H*d for tokens ordered (b, l)), without copies.
 *
 *   x : bf16 [M, K], row stride ldx (M tokens, K model width);
 *   w : bf16 [N, K], row stride ldw (N = 4*H*d output features);
 *   y : bf16 [M, N], row stride ldy; written in full, fp32 accumulation
 *       rounded to nearest even.
 * K must be a positive multiple of 32 and N a multiple of 8; strides
 * multiples of 8 elements, at least the row width, below 2^24; pointers
 * 16-byte aligned; y must not alias x or w.  M or N of 0: OK, no work.
 */
parallax_status parallax_qkvr_project(const void *x, const void *w, void *y, int M, int N,
                                      int K, int64_t ldx, int64_t ldw, int64_t ldy,
                                      void *stream);

/*
 * Walsh-Hadamard output projection (review page "Rethinking Attention
 * Output Projection: Structured Hadamard Transforms for Efficient
 * Transformers", sec. 2 "Methodology"): in place of the dense output
 * projection, the concatenated head outputs of each token are mixed by a
 * fixed Walsh-Hadamard transform and rescaled per feature,
 *
 *     y_t = alpha (.) (O_t H_n / sqrt(n)) + beta,   n = H * d,
 *
 * where O_t = [o_t(head 0) | ... | o_t(head H-1)] and H_n is the Sylvester
 * Hadamard matrix (entry (i, c) = (-1)^popcount(i & c)); with the 1/sqrt(n)
 * factor the transform is orthogonal and keeps each row's l2 norm.
 *
 *   o     : fp32 [B, H, L, d] (an attention output), element strides so,
 *           d contiguous; 16-byte aligned base, strides multiples of 4.
 *           A plain row-major [M, n] matrix is B = M, L = 1, H = n / d with
 *           strides (n, d, anything).
 *   alpha, beta : fp32 [n], 16-byte aligned, or NULL (ones / zeros).
 *   y     : bf16 [B * L, n], rows ordered (b, l), row stride ldy (a multiple
 *           of 4, at least n); 8-byte aligned; fp32 arithmetic, rounded to
 *           nearest even.  Must not alias o, alpha or beta.
 * d is 64 or 128 and n = H * d a power of two in [256, 4096]
 * (PARALLAX_ERR_UNSUPPORTED otherwise).  B * L == 0: OK, no work.
 */
parallax_status parallax_hadamard_out(const float *o, parallax_strides so, int B, int H, int L,
                                      int d, const float *alpha, const float *beta, void *y,
                                      int64_t ldy, void *stream);

/*
 * Based linear attention (review page "Simple linear attention language
 * models balance the recall-throughput tradeoff", "Proposed method"): the
 * linear-attention half of the Based hybrid, whose other half is softmax
 * attention over a small sliding window (parallax_attn_fwd with rho = 0,
 * a window of 64 or 128 keys and, optionally, sinks).  Linear attention
 * replaces exp(scale q.k) by a kernel phi(q).phi(k), so the causal sum is
 * carried as a state whose size the feature dimension sets.  Here phi is
 * the feature map of the second-order Taylor expansion of exp: with
 * x = scale * q_i . k_j,
 *
 *     w_ij = phi(q_i) . phi(k_j) = 1 + x + x^2 / 2      (always > 0)
 *     o_i  = sum_{j <= i} w_ij v_j / sum_{j <= i} w_ij
 *
 * The query/key feature dimension dk must be 16 (phi then has 153
 * features: 1, 16 linear, 136 distinct quadratic products); dv is 64 or
 * 128.  PARALLAX_ERR_UNSUPPORTED otherwise.
 *
 * State (decoding): fp32 [B, H, 160, NC] with NC = 16 * (dv / 16 + 1),
 * contiguous; parallax_based_state_floats(dk, dv) = 160 * NC floats per
 * (batch, head).  Entry [f][c] is sum_j phi_f(k_j) v_jc for c < dv and
 * sum_j phi_f(k_j) for every c >= dv, with the feature order
 *     f = 16 d + a (f < 128): k_a k_{(a+d) mod 16} * (scale/sqrt2 if d == 0
 *                             else scale);
 *     f = 128 + a (a < 8): scale k_a k_{a+8};  f = 136 + a: sqrt(scale) k_a;
 *     f = 152: 1;  f = 153..159: 0.
 *
 * Numerics: the prefill feeds phi(k) and v to the matrix cores as float16
 * (|v| <= 65504, |k_a k_b| * scale <= 65504) and the prefix state and
 * phi(q) as bfloat16, with fp32 sums; the decode works in fp32.
 */
size_t parallax_based_state_floats(int dk, int dv);

/*
 * Bytes of device workspace parallax_based_fwd needs: per (batch, head) and
 * per 512-token segment, the segment's state in fp32 plus the prefix state
 * as bf16 fragments, i.e. B * H * ceil(L / 512) * 160 * NC * 6 bytes.  0 for
 * sizes parallax_based_fwd would reject.
 */
size_t parallax_based_workspace_size(int B, int H, int L, int dk, int dv);

/*
 * Causal Based linear-attention prefill.
 *   q, k : bf16 [B, H, L, 16]; v: bf16 [B, H, L, dv]; element strides
 *          sq, sk, sv (last dimension contiguous, strides multiples of 8,
 *          16-byte aligned bases).
 *   o    : fp32 [B, H, L, dv], strides so (multiples of 4), 16-byte aligned.
 *   state: NULL, or fp32 [B, H, 160, NC] (16-byte aligned): receives the
 *          state after the last token, for parallax_based_decode.
 *   scale: > 0 and finite (x = scale * q.k; 1/4 is 1/sqrt(dk)).
 *   workspace: device memory of parallax_based_workspace_size bytes,
 *          16-byte aligned; scratch once the call's work has finished.
 * B * H * L == 0: OK, no work.
 */
parallax_status parallax_based_fwd(const void *q, const void *k, const void *v, float *o,
                                   float *state, int B, int H, int L, int dk, int dv,
                                   parallax_strides sq, parallax_strides sk, parallax_strides sv,
                                   parallax_strides so, float scale, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * One Based decode step per (batch, head): adds phi(k)[v | 1]^T to the
 * state (in place) and writes o = phi(q).S[:, :dv] / phi(q).S[:, dv], the
 * output of the new token over every token so far (the state's and its
 * own).  q, k: bf16 [B, H, 16]; v: bf16 [B, H, dv]; state: fp32
 * [B, H, 160, NC]; o: fp32 [B, H, dv]; all contiguous.  A zero state starts
 * a new sequence.  B * H == 0: OK, no work.
 */
parallax_status parallax_based_decode(const void *q, const void *k, const void *v, float *state,
                                      float *o, int B, int H, int dk, int dv, float scale,
                                      void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *parallax_status_string(parallax_status s);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
