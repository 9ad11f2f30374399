// C-ABI entry points of the Parallax library: host-side argument checks,
// then the kernel launches on the caller's stream.  No allocation, no
// synchronisation, no global state.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "launch.h"
#include "parallax.h"

namespace {

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Strides of a bf16 tensor used with 16-byte vector loads: non-negative
// multiples of 8 elements.
bool bf16_strides_ok(const parallax_strides &s) {
    return s.b >= 0 && s.h >= 0 && s.l >= 0 && s.b % 8 == 0 && s.h % 8 == 0 && s.l % 8 == 0;
}

// Strides of the fp32 output written with 16-byte stores.
bool f32_strides_ok(const parallax_strides &s) {
    return s.b >= 0 && s.h >= 0 && s.l >= 0 && s.b % 4 == 0 && s.h % 4 == 0 && s.l % 4 == 0;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// Row strides are used in 32-bit byte offsets inside a tile of rows.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;
bool row_stride_ok(const parallax_strides &s) { return s.l < kMaxRowStride; }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

const char *parallax_status_string(parallax_status s) {
    switch (s) {
    case PARALLAX_OK: return "PARALLAX_OK";
    case PARALLAX_ERR_INVALID_ARG: return "PARALLAX_ERR_INVALID_ARG";
    case PARALLAX_ERR_UNSUPPORTED: return "PARALLAX_ERR_UNSUPPORTED";
    case PARALLAX_ERR_LAUNCH: return "PARALLAX_ERR_LAUNCH";
    }
    return "PARALLAX_ERR_UNKNOWN";
}

size_t parallax_attn_fwd_workspace_size(int B, int H, int L, int d) {
    if (B < 0 || H < 0 || L < 0 || (d != 64 && d != 128))
        return 0;
    return plx::fwd_workspace_bytes(B, H, L, d);
}

}  // extern "C"

namespace {

parallax_status fwd_common(const void *q, const void *k, const void *v, const void *r, float *o,
                           float *lse, float *sbar, float *pv, int B, int H, int L, int d,
                           parallax_strides sq, parallax_strides sk, parallax_strides sv,
                           parallax_strides sr, parallax_strides so, float softmax_scale,
                           int window, int n_sink, void *workspace, size_t workspace_bytes,
                           void *stream, bool train, bool precise, bool use_scratch = false) {
    if (B < 0 || H < 0 || L < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(softmax_scale) || window < 0 || n_sink < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H * L == 0)
        return PARALLAX_OK;
    if (!q || !k || !v || !r || !o || !lse || (train && (!sbar || !pv)))
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(r, 16) ||
        !aligned(o, 16) || !aligned(lse, 4) || !aligned(sbar, 4) || !aligned(pv, 16))
        return PARALLAX_ERR_INVALID_ARG;
    if (!bf16_strides_ok(sq) || !bf16_strides_ok(sk) || !bf16_strides_ok(sv) ||
        !bf16_strides_ok(sr) || !f32_strides_ok(so))
        return PARALLAX_ERR_INVALID_ARG;
    if (!row_stride_ok(sq) || !row_stride_ok(sk) || !row_stride_ok(sv) || !row_stride_ok(sr))
        return PARALLAX_ERR_UNSUPPORTED;
    if (use_scratch) {
        // The library's own device array replaces the caller's workspace.
        if (plx::fwd_workspace_bytes(B, H, L, d) > plx::kFwdScratchBytes)
            return PARALLAX_ERR_UNSUPPORTED;
    } else if (!workspace || !aligned(workspace, 16) ||
               workspace_bytes < plx::fwd_workspace_bytes(B, H, L, d)) {
        return PARALLAX_ERR_INVALID_ARG;
    }

    const int bm = plx::fwd_block_rows(d);
    const int64_t n_qtiles = ((int64_t)L + bm - 1) / bm;
    if ((int64_t)B * H * n_qtiles > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    if (use_scratch && plx::fwd_scratch(&workspace) != hipSuccess)
        return PARALLAX_ERR_LAUNCH;

    plx::FwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.r = static_cast<const uint16_t *>(r);
    a.o = o;
    a.lse = lse;
    a.sbar = train ? sbar : nullptr;
    a.pv = train ? pv : nullptr;
    a.vt = static_cast<uint16_t *>(workspace);
    a.counters = reinterpret_cast<unsigned *>(static_cast<char *>(workspace) +
                                              plx::fwd_image_bytes(B, H, L, d));
    a.q_b = sq.b; a.q_h = sq.h; a.q_l = sq.l;
    a.k_b = sk.b; a.k_h = sk.h; a.k_l = sk.l;
    a.v_b = sv.b; a.v_h = sv.h; a.v_l = sv.l;
    a.r_b = sr.b; a.r_h = sr.h; a.r_l = sr.l;
    a.o_b = so.b; a.o_h = so.h; a.o_l = so.l;
    a.B = B;
    a.H = H;
    a.L = L;
    a.n_qtiles = (int)n_qtiles;
    a.n_st = (int)(((int64_t)L + plx::kStageKeys - 1) / plx::kStageKeys);
    a.scale_log2 = softmax_scale * kLog2e;
    a.window = window;
    a.n_sink = n_sink;
    hipError_t e = plx::launch_fwd(a, d, precise, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

}  // namespace

extern "C" {

parallax_status parallax_attn_fwd(const void *q, const void *k, const void *v, const void *r,
                                  float *o, float *lse, int B, int H, int L, int d,
                                  parallax_strides sq, parallax_strides sk, parallax_strides sv,
                                  parallax_strides sr, parallax_strides so, float softmax_scale,
                                  int window, int n_sink, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return fwd_common(q, k, v, r, o, lse, nullptr, nullptr, B, H, L, d, sq, sk, sv, sr, so,
                      softmax_scale, window, n_sink, workspace, workspace_bytes, stream, false,
                      false);
}

parallax_status parallax_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                          const void *r, float *o, float *lse, int B, int H,
                                          int L, int d, parallax_strides sq, parallax_strides sk,
                                          parallax_strides sv, parallax_strides sr,
                                          parallax_strides so, float softmax_scale, int window,
                                          int n_sink, void *stream) {
    return fwd_common(q, k, v, r, o, lse, nullptr, nullptr, B, H, L, d, sq, sk, sv, sr, so,
                      softmax_scale, window, n_sink, nullptr, 0, stream, false, false, true);
}

parallax_status parallax_attn_fwd_f32(const float *q, const float *k, const float *v,
                                      const float *r, float *o, float *lse, int B, int H, int L,
                                      int d, parallax_strides sq, parallax_strides sk,
                                      parallax_strides sv, parallax_strides sr,
                                      parallax_strides so, float softmax_scale, int window,
                                      int n_sink, void *stream) {
    if (B < 0 || H < 0 || L < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(softmax_scale) || window < 0 || n_sink < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H * L == 0)
        return PARALLAX_OK;
    if (!q || !k || !v || !r || !o || !lse)
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(r, 4) || !aligned(o, 4) ||
        !aligned(lse, 4))
        return PARALLAX_ERR_INVALID_ARG;
    for (const parallax_strides *s : {&sq, &sk, &sv, &sr, &so})
        if (s->b < 0 || s->h < 0 || s->l < 0)
            return PARALLAX_ERR_INVALID_ARG;
    if (plx::fwd_f32_blocks(B, H, L) > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    plx::F32Args a;
    a.q = q; a.k = k; a.v = v; a.r = r; a.o = o; a.lse = lse;
    a.q_b = sq.b; a.q_h = sq.h; a.q_l = sq.l;
    a.k_b = sk.b; a.k_h = sk.h; a.k_l = sk.l;
    a.v_b = sv.b; a.v_h = sv.h; a.v_l = sv.l;
    a.r_b = sr.b; a.r_h = sr.h; a.r_l = sr.l;
    a.o_b = so.b; a.o_h = so.h; a.o_l = so.l;
    a.B = B; a.H = H; a.L = L;
    a.scale = softmax_scale;
    a.window = window;
    a.n_sink = n_sink;
    hipError_t e = plx::launch_fwd_f32(a, d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

parallax_status parallax_attn_fwd_precise(const void *q, const void *k, const void *v,
                                          const void *r, float *o, float *lse, int B, int H,
                                          int L, int d, parallax_strides sq, parallax_strides sk,
                                          parallax_strides sv, parallax_strides sr,
                                          parallax_strides so, float softmax_scale, int window,
                                          int n_sink, void *workspace, size_t workspace_bytes,
                                          void *stream) {
    return fwd_common(q, k, v, r, o, lse, nullptr, nullptr, B, H, L, d, sq, sk, sv, sr, so,
                      softmax_scale, window, n_sink, workspace, workspace_bytes, stream, false,
                      true);
}

parallax_status parallax_attn_fwd_train(const void *q, const void *k, const void *v,
                                        const void *r, float *o, float *lse, float *sbar,
                                        float *pv, int B, int H, int L, int d,
                                        parallax_strides sq, parallax_strides sk,
                                        parallax_strides sv, parallax_strides sr,
                                        parallax_strides so, float softmax_scale, int window,
                                        int n_sink, void *workspace, size_t workspace_bytes,
                                        void *stream) {
    return fwd_common(q, k, v, r, o, lse, sbar, pv, B, H, L, d, sq, sk, sv, sr, so,
                      softmax_scale, window, n_sink, workspace, workspace_bytes, stream, true,
                      false);
}

size_t parallax_attn_bwd_workspace_size(int B, int H, int L, int d) {
    if (B < 0 || H < 0 || L < 0 || (d != 64 && d != 128))
        return 0;
    return plx::bwd_workspace_bytes(B, H, L, d);
}

parallax_status parallax_attn_bwd(const void *q, const void *k, const void *v, const void *r,
                                  const void *dout, const float *o, const float *lse,
                                  const float *sbar, const float *pv, float *dq, float *dk,
                                  float *dv, float *dr, int B, int H, int L, int d,
                                  parallax_strides sq, parallax_strides sk, parallax_strides sv,
                                  parallax_strides sr, parallax_strides sdo,
                                  float softmax_scale, int window, int n_sink, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (B < 0 || H < 0 || L < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(softmax_scale) || window < 0 || n_sink < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H * L == 0)
        return PARALLAX_OK;
    if (!q || !k || !v || !r || !dout || !o || !lse || !sbar || !pv || !dq || !dk || !dv || !dr)
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(r, 16) ||
        !aligned(dout, 16) || !aligned(o, 16) || !aligned(lse, 4) || !aligned(sbar, 4) ||
        !aligned(pv, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(dr, 16))
        return PARALLAX_ERR_INVALID_ARG;
    if (!bf16_strides_ok(sq) || !bf16_strides_ok(sk) || !bf16_strides_ok(sv) ||
        !bf16_strides_ok(sr) || !bf16_strides_ok(sdo))
        return PARALLAX_ERR_INVALID_ARG;
    if (!row_stride_ok(sq) || !row_stride_ok(sk) || !row_stride_ok(sv) || !row_stride_ok(sr) ||
        !row_stride_ok(sdo))
        return PARALLAX_ERR_UNSUPPORTED;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < plx::bwd_workspace_bytes(B, H, L, d))
        return PARALLAX_ERR_INVALID_ARG;

    const int64_t BH = (int64_t)B * H;
    const int64_t n_st = ((int64_t)L + plx::kStageKeys - 1) / plx::kStageKeys;
    const int64_t bt = 128;  // rows per workgroup of the backward kernels
    const int64_t n_kb = ((int64_t)L + bt - 1) / bt;
    // Key blocks holding sink keys, and the chunks of rows past their window.
    int64_t n_sb = 0, n_chunks = 0;
    if (window > 0 && n_sink > 0) {
        n_sb = (std::min<int64_t>(n_sink, L) + bt - 1) / bt;
        const int64_t first_past = std::min<int64_t>(n_st, (bt - 1 + window - 1) / 32 + 1);
        n_chunks = (n_st - first_past + plx::kBwdChunk - 1) / plx::kBwdChunk;
    }
    if (BH * (n_kb + n_sb * n_chunks) > INT_MAX ||
        n_st * (int64_t)plx::bwd_kv_record_bytes(d) > INT32_MAX || n_st * 512 > INT32_MAX)
        return PARALLAX_ERR_UNSUPPORTED;

    char *ws = static_cast<char *>(workspace);
    plx::BwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.r = static_cast<const uint16_t *>(r);
    a.dout = static_cast<const uint16_t *>(dout);
    a.o = o;
    a.lse = lse;
    a.sbar = sbar;
    a.pv = pv;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dr = dr;
    a.stats = reinterpret_cast<float *>(ws);
    a.kvrec = reinterpret_cast<uint16_t *>(ws + plx::bwd_stats_bytes(BH, n_st));
    a.qrec = reinterpret_cast<uint16_t *>(ws + plx::bwd_stats_bytes(BH, n_st) +
                                          (size_t)(BH * n_st) * plx::bwd_kv_record_bytes(d));
    a.q_b = sq.b; a.q_h = sq.h; a.q_l = sq.l;
    a.k_b = sk.b; a.k_h = sk.h; a.k_l = sk.l;
    a.v_b = sv.b; a.v_h = sv.h; a.v_l = sv.l;
    a.r_b = sr.b; a.r_h = sr.h; a.r_l = sr.l;
    a.do_b = sdo.b; a.do_h = sdo.h; a.do_l = sdo.l;
    a.B = B;
    a.H = H;
    a.L = L;
    a.n_st = (int)n_st;
    a.scale = softmax_scale;
    a.window = window;
    a.n_sink = n_sink;
    a.n_sb = (int)n_sb;
    a.n_chunks = (int)n_chunks;
    a.zero_rows = (int)std::min<int64_t>(L, n_sb * bt);
    hipError_t e = plx::launch_bwd(a, d, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

parallax_status parallax_attn_decode(const void *q, const void *r, const void *k_cache,
                                     const void *v_cache, const int32_t *seqlens, float *o,
                                     float *lse, int B, int H, int Lmax, int d,
                                     parallax_strides sk, parallax_strides sv,
                                     float softmax_scale, int num_splits, void *stream) {
    if (B < 0 || H < 0 || Lmax < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    if (num_splits != 1 && num_splits != 2 && num_splits != 4 && num_splits != 8 &&
        num_splits != 16)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(softmax_scale))
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H == 0)
        return PARALLAX_OK;
    if (!q || !r || !o || !lse || (Lmax > 0 && (!k_cache || !v_cache)))
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(r, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(o, 4) || !aligned(lse, 4) || !aligned(seqlens, 4))
        return PARALLAX_ERR_INVALID_ARG;
    if (!bf16_strides_ok(sk) || !bf16_strides_ok(sv))
        return PARALLAX_ERR_INVALID_ARG;
    // The kernel forms per-lane row offsets in 32 bits (a few rows apart).
    if (!row_stride_ok(sk) || !row_stride_ok(sv) || (int64_t)B * H > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;

    plx::DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.r = static_cast<const uint16_t *>(r);
    a.k = static_cast<const uint16_t *>(k_cache);
    a.v = static_cast<const uint16_t *>(v_cache);
    a.seqlens = seqlens;
    a.o = o;
    a.lse = lse;
    a.k_b = sk.b; a.k_h = sk.h; a.k_l = sk.l;
    a.v_b = sv.b; a.v_h = sv.h; a.v_l = sv.l;
    a.B = B;
    a.H = H;
    a.Lmax = Lmax;
    a.scale_log2 = softmax_scale * kLog2e;
    hipError_t e = plx::launch_decode(a, d, num_splits, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

namespace {

// The general decode; `part` is the key-split workspace of
// parallax_attn_decode_paged_ws (nullptr: no key splits).
parallax_status decode_paged(const void *q, const void *r, const void *k_cache,
                             const void *v_cache, const int32_t *block_table, int num_pages,
                             int page_size, int max_pages, const int32_t *seqlens, float *o,
                             float *lse, int B, int Hq, int Hkv, int d, parallax_strides sk,
                             parallax_strides sv, float softmax_scale, int window, int n_sink,
                             int num_splits, float *part, void *stream) {
    if (B < 0 || Hq < 0 || Hkv < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    if (num_splits != 1 && num_splits != 2 && num_splits != 4 && num_splits != 8 &&
        num_splits != 16)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(softmax_scale) || window < 0 || n_sink < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * Hq == 0)
        return PARALLAX_OK;
    if (Hkv <= 0 || Hq % Hkv != 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (page_size <= 0 || (block_table && ((page_size & (page_size - 1)) != 0 ||
                                            num_pages <= 0 || max_pages <= 0)))
        return PARALLAX_ERR_INVALID_ARG;
    if (!q || !r || !o || !lse || !k_cache || !v_cache)
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(r, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(o, 4) || !aligned(lse, 4) || !aligned(seqlens, 4) || !aligned(block_table, 4))
        return PARALLAX_ERR_INVALID_ARG;
    if (!bf16_strides_ok(sk) || !bf16_strides_ok(sv))
        return PARALLAX_ERR_INVALID_ARG;
    const int64_t max_len = block_table ? (int64_t)max_pages * page_size : page_size;
    const int64_t g = Hq / Hkv;
    if (max_len > INT_MAX || (((int64_t)B * Hkv + 7) / 8) * 8 * g > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;

    plx::PagedDecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.r = static_cast<const uint16_t *>(r);
    a.k = static_cast<const uint16_t *>(k_cache);
    a.v = static_cast<const uint16_t *>(v_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.o = o;
    a.lse = lse;
    a.k_p = sk.b; a.k_h = sk.h; a.k_l = sk.l;
    a.v_p = sv.b; a.v_h = sv.h; a.v_l = sv.l;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    int shift = 0;
    while (block_table && (1 << shift) < page_size)
        ++shift;
    a.page_shift = shift;
    a.max_pages = block_table ? max_pages : 1;
    a.num_pages = block_table ? num_pages : B;
    a.max_len = (int)max_len;
    a.scale_log2 = softmax_scale * kLog2e;
    a.window = window;
    a.n_sink = n_sink;
    a.ksplit = 1;
    a.part = part;
    hipError_t e =
        plx::launch_decode_paged(a, d, num_splits, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

}  // namespace

parallax_status parallax_attn_decode_paged(const void *q, const void *r, const void *k_cache,
                                           const void *v_cache, const int32_t *block_table,
                                           int num_pages, int page_size, int max_pages,
                                           const int32_t *seqlens, float *o, float *lse, int B,
                                           int Hq, int Hkv, int d, parallax_strides sk,
                                           parallax_strides sv, float softmax_scale, int window,
                                           int n_sink, int num_splits, void *stream) {
    return decode_paged(q, r, k_cache, v_cache, block_table, num_pages, page_size, max_pages,
                        seqlens, o, lse, B, Hq, Hkv, d, sk, sv, softmax_scale, window, n_sink,
                        num_splits, nullptr, stream);
}

size_t parallax_attn_decode_paged_workspace_size(int B, int Hq, int d) {
    if (B <= 0 || Hq <= 0 || (d != 64 && d != 128))
        return 0;
    return plx::decode_paged_workspace_bytes(B, Hq, d);
}

parallax_status parallax_attn_decode_paged_ws(const void *q, const void *r, const void *k_cache,
                                              const void *v_cache, const int32_t *block_table,
                                              int num_pages, int page_size, int max_pages,
                                              const int32_t *seqlens, float *o, float *lse,
                                              int B, int Hq, int Hkv, int d, parallax_strides sk,
                                              parallax_strides sv, float softmax_scale,
                                              int window, int n_sink, int num_splits,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream) {
    if (B > 0 && Hq > 0 && (d == 64 || d == 128) &&
        (!workspace || !aligned(workspace, 16) ||
         workspace_bytes < plx::decode_paged_workspace_bytes(B, Hq, d)))
        return PARALLAX_ERR_INVALID_ARG;
    return decode_paged(q, r, k_cache, v_cache, block_table, num_pages, page_size, max_pages,
                        seqlens, o, lse, B, Hq, Hkv, d, sk, sv, softmax_scale, window, n_sink,
                        num_splits, static_cast<float *>(workspace), stream);
}

parallax_status parallax_qkvr_project(const void *x, const void *w, void *y, int M, int N,
                                      int K, int64_t ldx, int64_t ldw, int64_t ldy,
                                      void *stream) {
    if (M < 0 || N < 0 || K < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)M * N == 0)
        return PARALLAX_OK;
    if (K % 32 != 0 || N % 8 != 0)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!x || !w || !y || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16))
        return PARALLAX_ERR_INVALID_ARG;
    if (ldx < K || ldw < K || ldy < N || ldx % 8 || ldw % 8 || ldy % 8)
        return PARALLAX_ERR_INVALID_ARG;
    if (K == 0 || ldx >= kMaxRowStride || ldw >= kMaxRowStride || ldy >= kMaxRowStride ||
        plx::proj_tiles(M, N) > (size_t)INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    plx::ProjArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w);
    a.y = static_cast<uint16_t *>(y);
    a.ldx = ldx;
    a.ldw = ldw;
    a.ldy = ldy;
    a.M = M;
    a.N = N;
    a.K = K;
    hipError_t e = plx::launch_proj(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

parallax_status parallax_hadamard_out(const float *o, parallax_strides so, int B, int H, int L,
                                      int d, const float *alpha, const float *beta, void *y,
                                      int64_t ldy, void *stream) {
    if (B < 0 || H < 0 || L < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return PARALLAX_ERR_UNSUPPORTED;
    const int64_t n = (int64_t)H * d;
    if ((int64_t)B * L == 0)
        return PARALLAX_OK;
    if (n < 256 || n > 4096 || (n & (n - 1)) != 0)
        return PARALLAX_ERR_UNSUPPORTED;
    if (!o || !y || !aligned(o, 16) || !aligned(y, 8) || !aligned(alpha, 16) ||
        !aligned(beta, 16) || !f32_strides_ok(so) || ldy < n || ldy % 4 != 0)
        return PARALLAX_ERR_INVALID_ARG;
    int log2n = 0;
    while ((int64_t(1) << log2n) < n)
        ++log2n;
    const int64_t M = (int64_t)B * L;
    if (M > (int64_t)INT_MAX - 256 || plx::hadamard_blocks(M, log2n) > (int64_t)INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    plx::HadArgs a;
    a.o = o;
    a.o_b = so.b;
    a.o_h = so.h;
    a.o_l = so.l;
    a.alpha = alpha;
    a.beta = beta;
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    a.M = (int)M;
    a.L = L;
    a.log2d = d == 64 ? 6 : 7;
    hipError_t e = plx::launch_hadamard(a, log2n, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

size_t parallax_based_state_floats(int dk, int dv) {
    if (dk != 16 || (dv != 64 && dv != 128))
        return 0;
    return plx::based_state_floats(dv);
}

size_t parallax_based_workspace_size(int B, int H, int L, int dk, int dv) {
    if (B < 0 || H < 0 || L < 0 || dk != 16 || (dv != 64 && dv != 128))
        return 0;
    return plx::based_workspace_bytes(B, H, L, dv);
}

parallax_status parallax_based_fwd(const void *q, const void *k, const void *v, float *o,
                                   float *state, int B, int H, int L, int dk, int dv,
                                   parallax_strides sq, parallax_strides sk, parallax_strides sv,
                                   parallax_strides so, float scale, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (B < 0 || H < 0 || L < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (dk != 16 || (dv != 64 && dv != 128))
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(scale))
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H * L == 0)
        return PARALLAX_OK;
    if (!q || !k || !v || !o || !workspace)
        return PARALLAX_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(state, 16) || !aligned(workspace, 16))
        return PARALLAX_ERR_INVALID_ARG;
    if (!bf16_strides_ok(sq) || !bf16_strides_ok(sk) || !bf16_strides_ok(sv) ||
        !f32_strides_ok(so))
        return PARALLAX_ERR_INVALID_ARG;
    if (workspace_bytes < plx::based_workspace_bytes(B, H, L, dv))
        return PARALLAX_ERR_INVALID_ARG;
    const int64_t n_seg = ((int64_t)L + plx::kBasedSegment - 1) / plx::kBasedSegment;
    const int64_t n_qt = ((int64_t)L + plx::kBasedQueryTile - 1) / plx::kBasedQueryTile;
    if ((int64_t)B * H * n_qt > INT_MAX || (int64_t)B * H * n_seg * 64 * 9 * 5 > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    plx::BasedArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = o;
    a.q_b = sq.b, a.q_h = sq.h, a.q_l = sq.l;
    a.k_b = sk.b, a.k_h = sk.h, a.k_l = sk.l;
    a.v_b = sv.b, a.v_h = sv.h, a.v_l = sv.l;
    a.o_b = so.b, a.o_h = so.h, a.o_l = so.l;
    a.B = B;
    a.H = H;
    a.L = L;
    a.n_seg = (int)n_seg;
    a.n_qt = (int)n_qt;
    a.scale = scale;
    a.dstate = static_cast<float *>(workspace);
    a.sfrag = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) +
                                           (size_t)B * H * n_seg *
                                               plx::based_state_floats(dv) * 4);
    a.state = state;
    hipError_t e = plx::launch_based_fwd(a, dv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

parallax_status parallax_based_decode(const void *q, const void *k, const void *v, float *state,
                                      float *o, int B, int H, int dk, int dv, float scale,
                                      void *stream) {
    if (B < 0 || H < 0)
        return PARALLAX_ERR_INVALID_ARG;
    if (dk != 16 || (dv != 64 && dv != 128))
        return PARALLAX_ERR_UNSUPPORTED;
    if (!scale_ok(scale))
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H == 0)
        return PARALLAX_OK;
    if (!q || !k || !v || !state || !o || !aligned(q, 2) || !aligned(k, 2) || !aligned(v, 2) ||
        !aligned(state, 4) || !aligned(o, 4))
        return PARALLAX_ERR_INVALID_ARG;
    if ((int64_t)B * H > INT_MAX)
        return PARALLAX_ERR_UNSUPPORTED;
    plx::BasedArgs a = {};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = o;
    a.B = B;
    a.H = H;
    a.L = 1;
    a.scale = scale;
    a.state = state;
    hipError_t e = plx::launch_based_decode(a, dv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_LAUNCH;
}

}  // extern "C"
