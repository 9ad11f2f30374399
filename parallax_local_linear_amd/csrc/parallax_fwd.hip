// Causal Parallax prefill forward for gfx950 (MI355X).
//
// Method: Parallax, a parameterized Local Linear Attention, keeps the softmax
// weights p_ij and adds the probe correction rho_i.(k_j - kbar_i) to each
// weight (review page "Parallax: Parameterized Local Linear Attention for
// Language Modeling", sec. 1 and sec. 3).  Expanding kbar_i gives a one-pass
// form with running sums per query row:
//
//     A = sum_j p~_j v_j,   C = sum_j p~_j s_j v_j,   S = sum_j p~_j s_j,
//     ell = sum_j p~_j,     s_j = rho_i . k_j (unscaled),
//     o_i = (A (1 - S/ell) + C) / ell,
//
// where p~_j = 2^(x_j - m) are un-normalised softmax weights with a per-row
// offset m.  The review says the authors' kernel reaches a higher arithmetic
// intensity than FlashAttention 2/3 (sec. 3); here that shows as two score
// products (Q K^T and R K^T) per key tile sharing one K operand, and two
// value products (P~ V and (P~ o S) V) sharing one V operand.
//
// Mapping onto CDNA4:
//   * A workgroup = 4 wavefronts x 16 query rows = 64 rows; two workgroups
//     share a CU, so every SIMD runs two independent wavefronts and the
//     hardware overlaps one's exponentials, memory waits and barrier with
//     the other's matrix-core work.  Each wavefront keeps its Q and R
//     fragments and its fp32 accumulators in registers (<= 256 per lane).
//   * Keys stream through LDS in stages of 32 keys with three buffers; the
//     global loads of a stage are issued two stages ahead through buffer
//     resources that end at the last valid row, so rows past the sequence
//     end read as zeros without per-lane branches.  K is stored row-major
//     (bf16); V is stored transposed and converted to f16, with the keys of
//     each stage permuted so that one 16-byte LDS read gives each lane the
//     8 keys the value MFMA needs.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_bf16.  In that accumulator layout each lane holds
//     one query row (4 lanes, l ^ 16 and l ^ 32 apart, share a row), so row
//     max and row sums are in-lane reductions plus two exchanges, and the
//     f16-rounded weights are already in the B-operand layout of
//     O^T = V^T P~^T (v_mfma_f32_16x16x32_f16): no LDS round trip for P.
//   * ell and S are summed from the same f16-rounded weights that enter the
//     value MFMAs (v_dot2_f32_f16), keeping A, C, ell and S consistent.
//   * Each row's offset m is fixed at its first visible stage (that stage's
//     max + kMargin), so the accumulators are never rescaled inside the
//     loop.  Rows whose scores later exceed m + kTauHi make the workgroup
//     recompute once with the exact row max as offset; weights stay
//     <= 2^kTauHi in the first pass and <= 1 in the second.
//   * Causal, sliding-window and sink masks ("Sliding-window beats linear
//     attention" review, sec. 1) skip whole stages per workgroup.  Stages
//     visible to every row of the workgroup run mask-free; the others apply
//     per-element masks (no branches either way).
//   * Workgroups are issued heaviest query tile first; the block index keeps
//     all tiles of one (batch, head) on one XCD when B*H is a multiple of 8,
//     so their K/V reuse stays in that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace plx {
namespace {

constexpr int ROWS = 16;              // query rows per wavefront
constexpr int NWAVES = 4;
constexpr int BM = ROWS * NWAVES;     // query rows per workgroup
constexpr int BN = 32;                // keys per stage
constexpr int NBUF = 3;               // LDS stage buffers
constexpr int NTHREADS = 64 * NWAVES;
static_assert(BM == kFwdBlockM, "host and kernel must agree on the query tile");
// Softmax offsets, log2 units (see above).
constexpr float kMargin = 3.0f;
constexpr float kTauHi = 5.0f;

typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;

template <int D>
struct Cfg {
    // Row pitches in LDS.  With the MFMA fragment reads (16 rows, 4 adjacent
    // 16-byte blocks per row), a pitch of an odd multiple of 8 dwords keeps
    // ds_read_b128 free of bank conflicts on gfx950 (measured).
    static constexpr int KP = D + 16;   // K: 72 dwords at d = 128, 40 at d = 64
    static constexpr int VP = BN + 16;  // V^T: 24 dwords
    static constexpr int K_ELEMS = BN * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int KC = D / 32;   // reduction chunks of the score MFMA
    static constexpr int DT = D / 16;   // output tiles of the value MFMA
    static constexpr int K_LOADS = BN * (D / 8) / NTHREADS;  // 16-byte K loads per thread
    // Each thread transposes KQ consecutive keys x 8 features of V.
    static constexpr int KQ = BN * (D / 8) / NTHREADS;
    static_assert(K_LOADS >= 1 && K_LOADS * NTHREADS == BN * (D / 8), "K stage must split evenly");
    static_assert(KQ == 1 || KQ == 2, "V transpose handles 1 or 2 keys per thread");
};

template <int D>
struct StageRegs {
    u32x4 k[Cfg<D>::K_LOADS];
    u32x4 v[Cfg<D>::KQ];
};

// Position of stage key j (0..31) inside the transposed V stage.  The score
// accumulator gives lane group G (lane / 16) the keys 4G..4G+3 and
// 16+4G..16+4G+3; the value MFMA reads them as reduction positions 8G..8G+7.
__device__ __forceinline__ int vt_pos(int j) {
    return ((j >> 2) & 3) * 8 + (j >> 4) * 4 + (j & 3);
}

__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over the four lanes that share a query row (l, l^16, l^32, l^48).
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return xor32_max(x);
}

__device__ __forceinline__ float row_sum4(float x) {
    x = x + __shfl_xor(x, 16, 64);
    return xor32_sum(x);
}

// Per-thread byte offsets of this thread's K and V chunks inside a stage.
template <int D>
struct StageOffsets {
    uint32_t k[Cfg<D>::K_LOADS];
    uint32_t v[Cfg<D>::KQ];
};

template <int D>
__device__ __forceinline__ StageOffsets<D> stage_offsets(int64_t k_l, int64_t v_l, int tid) {
    using C = Cfg<D>;
    StageOffsets<D> o;
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u) {
        const int c = tid + NTHREADS * u;
        o.k[u] = (uint32_t)((c / (D / 8)) * k_l * 2 + (c % (D / 8)) * 16);
    }
    const int a = tid % (BN / C::KQ);
    const int cc = tid / (BN / C::KQ);
#pragma unroll
    for (int u = 0; u < C::KQ; ++u)
        o.v[u] = (uint32_t)((C::KQ * a + u) * v_l * 2 + cc * 16);
    return o;
}

// Global -> registers for the stage starting at key j0, through buffer
// resources that end at the last valid row: rows past the sequence end read
// as zeros and nothing outside the tensors is touched.
template <int D>
__device__ __forceinline__ void load_stage(StageRegs<D> &t, const uint16_t *kbase,
                                           const uint16_t *vbase, int64_t k_l, int64_t v_l,
                                           int j0, int L, const StageOffsets<D> &off) {
    using C = Cfg<D>;
    j0 = __builtin_amdgcn_readfirstlane(j0);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)j0 * k_l, rows_bytes(j0, L, k_l, D));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)j0 * v_l, rows_bytes(j0, L, v_l, D));
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u)
        t.k[u] = bufld16(rk, off.k[u]);
#pragma unroll
    for (int u = 0; u < C::KQ; ++u)
        t.v[u] = bufld16(rv, off.v[u]);
}

// Registers -> LDS: K row-major; V converted to f16 and transposed.
template <int D>
__device__ __forceinline__ void store_stage(const StageRegs<D> &t, uint16_t *sk, uint16_t *sv,
                                            int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u) {
        const int c = tid + NTHREADS * u;
        const int row = c / (D / 8);
        const int col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4 *>(sk + row * C::KP + col) = t.k[u];
    }
    const int a = tid % (BN / C::KQ);
    const int cc = tid / (BN / C::KQ);
    const int pos = vt_pos(C::KQ * a);
    if constexpr (C::KQ == 2) {
        // keys 2a, 2a+1 sit next to each other in the permuted order
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w0 = t.v[0][e >> 1], w1 = t.v[1][e >> 1];
            const float f0 = (e & 1) ? bf16_hi(w0) : bf16_lo(w0);
            const float f1 = (e & 1) ? bf16_hi(w1) : bf16_lo(w1);
            *reinterpret_cast<uint32_t *>(sv + (8 * cc + e) * C::VP + pos) =
                __builtin_bit_cast(uint32_t, cvt_f16x2(f0, f1));
        }
    } else {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t w = t.v[0][e2];
            const f16x2 hh = cvt_f16x2(bf16_lo(w), bf16_hi(w));
            const uint32_t bits = __builtin_bit_cast(uint32_t, hh);
            sv[(8 * cc + 2 * e2) * C::VP + pos] = (uint16_t)(bits & 0xffffu);
            sv[(8 * cc + 2 * e2 + 1) * C::VP + pos] = (uint16_t)(bits >> 16);
        }
    }
}

// Visibility class of the 32-key stage starting at j0 for rows [r0, r1]:
// 0 = no visible pair, 1 = every pair visible, 2 = needs a per-element mask.
__device__ __forceinline__ int classify(int j0, int r0, int r1, int L, int window, int n_sink) {
    const int j1 = j0 + BN - 1;
    if (r1 < r0 || j0 > r1 || j0 >= L)
        return 0;
    if (window > 0 && j1 < r0 - window + 1 && j0 >= n_sink)
        return 0;
    if (j1 <= r0 && j1 < L && (window <= 0 || r1 - j0 < window || j1 < n_sink))
        return 1;
    return 2;
}

template <int D>
struct Ctx {
    bf16x8 qf[Cfg<D>::KC], rf[Cfg<D>::KC];
    f32x4 accA[Cfg<D>::DT], accC[Cfg<D>::DT];
    float m_ref;  // this row's softmax offset (scaled log2 units)
    float xmax;   // running max of the row's raw scores
    float ell, ssum;
};

// Scores of one stage: S^T tiles (16 keys x 16 rows) for keys 0-15 and 16-31.
struct Scores {
    f32x4 q[2], r[2];
};

// S^T = K Q^T and R K^T for one stage: 2 key tiles x KC chunks x 2 MFMAs,
// each K fragment shared by the Q and the R product.
template <int D>
__device__ __forceinline__ void score_stage(const Ctx<D> &cx, const uint16_t *sk, int l16, int G,
                                            Scores &s) {
    using C = Cfg<D>;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        bf16x8 kf[C::KC];
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc)
            kf[kc] = *reinterpret_cast<const bf16x8 *>(sk + (16 * kt + l16) * C::KP + 32 * kc + 8 * G);
        f32x4 zq = {0.f, 0.f, 0.f, 0.f}, zr = {0.f, 0.f, 0.f, 0.f};
        s.q[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], cx.qf[0], zq, 0, 0, 0);
        s.r[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], cx.rf[0], zr, 0, 0, 0);
#pragma unroll
        for (int kc = 1; kc < C::KC; ++kc) {
            s.q[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc], cx.qf[kc], s.q[kt], 0, 0, 0);
            s.r[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc], cx.rf[kc], s.r[kt], 0, 0, 0);
        }
    }
}

// Per-element mask of a stage: invisible scores become -inf (bitwise logic
// and a select, no branches).
__device__ __forceinline__ void mask_scores(Scores &s, int j0, int row, int G, int L, int window,
                                            int n_sink) {
    const int lim = min(row, L - 1);                            // causal and sequence end
    const int wlo = window > 0 ? row - window + 1 : INT32_MIN;  // oldest window key
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 16 * kt + 4 * G + e;
            const bool vis = (j <= lim) & ((j >= wlo) | (j < n_sink));
            s.q[kt][e] = vis ? s.q[kt][e] : kNegInf;
        }
    }
}

// Weights of one stage: track the row max and fix the row's offset at its
// first visible stage (per-lane selects; the accumulators are never
// touched), form the f16 weights in the value MFMA's B-operand order, add
// them to ell and S, and run the value MFMAs on the stage's V fragments.
template <int D>
struct VFrags {
    f16x8 f[Cfg<D>::DT];
};

// V^T fragments of one stage (A operand of the value MFMAs): V^T row
// 16 dt + l16, reduction positions 8G .. 8G+7.
template <int D>
__device__ __forceinline__ void read_vfrags(VFrags<D> &vf, const uint16_t *sv, int l16, int G) {
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt)
        vf.f[dt] = *reinterpret_cast<const f16x8 *>(sv + (16 * dt + l16) * Cfg<D>::VP + 8 * G);
}

template <int D>
__device__ __forceinline__ void value_stage(Ctx<D> &cx, const Scores &s, const VFrags<D> &vf,
                                            float c) {
    using C = Cfg<D>;

    float mt = fmaxf(fmaxf(fmaxf(s.q[0][0], s.q[0][1]), s.q[0][2]),
                     fmaxf(fmaxf(s.q[0][3], s.q[1][0]), s.q[1][1]));
    mt = fmaxf(fmaxf(mt, s.q[1][2]), s.q[1][3]);
    mt = row_max4(mt);
    cx.xmax = fmaxf(cx.xmax, mt);
    cx.m_ref = (cx.m_ref == kNegInf) ? fmaf(mt, c, kMargin) : cx.m_ref;
    const float msub = (cx.m_ref == kNegInf) ? 0.f : cx.m_ref;

    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    f16x8 pf, wf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * e2;
            const float p0 = exp2_fast(fmaf(s.q[kt][e], c, -msub));
            const float p1 = exp2_fast(fmaf(s.q[kt][e + 1], c, -msub));
            const f16x2 ph = cvt_f16x2(p0, p1);
            const f16x2 wh = cvt_f16x2(p0 * s.r[kt][e], p1 * s.r[kt][e + 1]);
            cx.ell = __builtin_amdgcn_fdot2(ph, ones, cx.ell, false);
            cx.ssum = __builtin_amdgcn_fdot2(wh, ones, cx.ssum, false);
            pf[4 * kt + e] = ph[0];
            pf[4 * kt + e + 1] = ph[1];
            wf[4 * kt + e] = wh[0];
            wf[4 * kt + e + 1] = wh[1];
        }
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
        cx.accA[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pf, cx.accA[dt], 0, 0, 0);
        cx.accC[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], wf, cx.accC[dt], 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(NTHREADS, 2) void parallax_fwd_kernel(FwdArgs a) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][C::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int G = lane >> 4;

    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int L = a.L;
    const int i0 = qt * BM;
    const int i1 = min(i0 + BM, L) - 1;
    const int row = i0 + ROWS * wave + l16;
    const int window = a.window;
    const int n_sink = a.n_sink;
    const float c = a.scale_log2;

    const uint16_t *qb = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h;
    const uint16_t *rb = a.r + (int64_t)b * a.r_b + (int64_t)h * a.r_h;
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;

    Ctx<D> cx;
    {
        // Rows past the sequence end read as zeros; their outputs are not stored.
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(qb + (int64_t)i0 * a.q_l, rows_bytes(i0, L, a.q_l, D));
        const __amdgpu_buffer_rsrc_t rr =
            make_rsrc(rb + (int64_t)i0 * a.r_l, rows_bytes(i0, L, a.r_l, D));
        const uint32_t qoff = (uint32_t)((row - i0) * a.q_l * 2);
        const uint32_t roff = (uint32_t)((row - i0) * a.r_l * 2);
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
            const uint32_t col = (32 * kc + 8 * G) * 2;
            cx.qf[kc] = __builtin_bit_cast(bf16x8, bufld16(rq, qoff + col));
            cx.rf[kc] = __builtin_bit_cast(bf16x8, bufld16(rr, roff + col));
        }
        cx.m_ref = kNegInf;
        cx.xmax = kNegInf;
    }

    // Stages with at least one visible pair for rows [i0, i1]: the sink
    // stages that lie before the window, then the window/causal span.
    const int st_hi = i1 / BN;
    int st_lo = 0, n_ss = 0;
    if (window > 0) {
        const int lo = i0 - window + 1;
        st_lo = lo > 0 ? lo / BN : 0;
        n_ss = min((n_sink + BN - 1) / BN, st_lo);
    }
    const int n = n_ss + (st_hi - st_lo + 1);
    auto stage_j0 = [&](int t) { return (t < n_ss ? t : st_lo + (t - n_ss)) * BN; };

    // Stages fully visible to every row of the workgroup: [f_lo, f_hi).
    // Causal stages before the diagonal (with a window: those well inside
    // it) are full; sink stages, window edges and the diagonal are not.
    int f_lo = n, f_hi = n;
    for (int t = 0; t < n; ++t) {
        if (classify(stage_j0(t), i0, i1, L, window, n_sink) == 1) {
            f_lo = t;
            break;
        }
    }
    if (f_lo < n) {
        f_hi = f_lo + 1;
        while (f_hi < n && classify(stage_j0(f_hi), i0, i1, L, window, n_sink) == 1)
            ++f_hi;
    }

    // Global prefetches past the last stage reload the last stage into a
    // buffer nobody reads again, which keeps the loop bodies branch-free.
    const StageOffsets<D> soff = stage_offsets<D>(a.k_l, a.v_l, tid);
    auto fetch = [&](StageRegs<D> &p, int t) __attribute__((always_inline)) {
        load_stage<D>(p, kb, vb, a.k_l, a.v_l, stage_j0(min(t, n - 1)), L, soff);
    };

    // Stage t: prefetch stage t+3 into p_ld, scores, (mask), weights and
    // value MFMAs of stage t from LDS buffer t%3, store stage t+2 (p_st) into
    // buffer (t+2)%3, barrier.  Between stages p0 holds stage t+2.
    StageRegs<D> p0, p1;
    Scores sc;
    VFrags<D> vf;
    auto stage = [&](int t, bool masked, StageRegs<D> &p_st, StageRegs<D> &p_ld)
        __attribute__((always_inline)) {
        const int buf = t % NBUF;
        fetch(p_ld, t + 3);
        // V fragments first: they arrive while the score MFMAs run.
        read_vfrags<D>(vf, sV[buf], l16, G);
        score_stage<D>(cx, sK[buf], l16, G, sc);
        if (masked)
            mask_scores(sc, stage_j0(t), row, G, L, window, n_sink);
        value_stage<D>(cx, sc, vf, c);
        const int bst = (t + 2) % NBUF;
        store_stage<D>(p_st, sK[bst], sV[bst], tid);
        __syncthreads();
    };

    // Pass 0 uses offsets fixed at each row's first visible stage; if any
    // row's scores later rose more than kTauHi above its offset, pass 1
    // recomputes the workgroup with the exact row max as offset.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            cx.accA[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
            cx.accC[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        cx.ell = 0.f;
        cx.ssum = 0.f;

        fetch(p0, 0);
        store_stage<D>(p0, sK[0], sV[0], tid);
        fetch(p0, 1);
        store_stage<D>(p0, sK[1], sV[1], tid);
        fetch(p0, 2);
        __syncthreads();

        int t = 0;
        for (; t < f_lo; ++t) {
            stage(t, true, p0, p1);
            p0 = p1;
        }
        for (; t + 1 < f_hi; t += 2) {
            stage(t, false, p0, p1);
            stage(t + 1, false, p1, p0);
        }
        for (; t < n; ++t) {
            stage(t, t >= f_hi, p0, p1);
            p0 = p1;
        }

        const bool overflow = pass == 0 && cx.xmax * c > cx.m_ref + kTauHi;
        if (!__syncthreads_or(overflow))
            break;
        // Exact offsets for the recomputation: each row's true max.
        cx.m_ref = cx.xmax * c;
    }

    // Epilogue: combine the partial sums of the four lanes of each row.
    const float ell_t = row_sum4(cx.ell);
    const float s_t = row_sum4(cx.ssum);
    if (row < L) {
        const float inv = 1.f / ell_t;
        const float keep = 1.f - s_t * inv;
        float *ob = a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)row * a.o_l;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            f32x4 out;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                out[u] = (cx.accA[dt][u] * keep + cx.accC[dt][u]) * inv;
            *reinterpret_cast<f32x4 *>(ob + 16 * dt + 4 * G) = out;
        }
        if (G == 0)
            a.lse[(int64_t)bh * L + row] = (cx.m_ref + log2f(ell_t)) * kLn2;
    }
}

template <int D>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H * a.n_qtiles));
    const dim3 block(NTHREADS);
    FwdArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_fwd_kernel<D>), grid, block,
                           params, 0, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int d, hipStream_t stream) {
    return d == 64 ? launch_fwd_t<64>(a, stream) : launch_fwd_t<128>(a, stream);
}

}  // namespace plx
