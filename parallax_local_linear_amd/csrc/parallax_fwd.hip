// Causal Parallax prefill forward for gfx950 (MI355X).
//
// Method: Parallax, a parameterized Local Linear Attention, keeps the softmax
// weights p_ij and adds the probe correction rho_i.(k_j - kbar_i) to each
// weight (review page "Parallax: Parameterized Local Linear Attention for
// Language Modeling", sec. 1 and sec. 3).  Expanding kbar_i gives a one-pass
// form with three running sums per query row:
//
//     A = sum_j p~_j v_j,   C = sum_j p~_j s_j v_j,   S = sum_j p~_j s_j,
//     ell = sum_j p~_j,     s_j = rho_i . k_j (unscaled),
//     o_i = (A (1 - S/ell) + C) / ell,
//
// where p~_j = 2^(x_j - m) are un-normalised softmax weights with a running
// offset m.  The review says the authors' kernel reaches a higher arithmetic
// intensity than FlashAttention 2/3 (sec. 3); here that shows as two score
// products (Q K^T and R K^T) per key tile sharing one K operand, and two
// value products (P~ V and (P~ o S) V) sharing one V operand.
//
// Mapping onto CDNA4:
//   * A workgroup = 4 wavefronts = 128 query rows; each wavefront owns 32
//     rows and keeps its Q and R fragments in registers for the whole loop.
//   * Keys stream through LDS in tiles of 64, double-buffered: the next
//     tile's global loads are in flight while the current one is computed.
//     K is stored row-major (bf16); V is stored transposed and converted to
//     f16, with the keys of each 16-key chunk permuted so that one 16-byte
//     LDS read gives each lane the 8 keys the value MFMA needs.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16.  In that accumulator layout every lane holds
//     a single query row (lanes l and l^32 share a row), so row max and row
//     sums are in-lane reductions plus one exchange with the other half-wave,
//     and the f16-rounded weights are already in the B-operand layout of
//     O^T = V^T P~^T (v_mfma_f32_32x32x16_f16): no LDS round trip for P.
//   * ell and S are summed from the same f16-rounded weights that enter the
//     value MFMAs (v_dot2_f32_f16), keeping A, C, ell and S consistent.
//   * The running max is updated lazily: the accumulators are rescaled only
//     when some row's max grows by more than 2^kTau, so weights stay <= 2^4.
//   * Causal, sliding-window and sink masks ("Sliding-window beats linear
//     attention" review, sec. 1) skip whole 64-key tiles per workgroup and
//     whole 32-key sub-tiles per wavefront; only boundary sub-tiles apply a
//     per-element mask.
//   * Workgroups are issued heaviest query tile first; the block index keeps
//     all tiles of one (batch, head) on one XCD when B*H is a multiple of 8,
//     so their K/V reuse stays in that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace plx {
namespace {

constexpr int BM = kFwdBlockM;  // query rows per workgroup
constexpr int BN = 64;          // keys per LDS tile
constexpr int NWAVES = BM / 32;
constexpr int NTHREADS = 64 * NWAVES;
constexpr float kTau = 4.0f;    // lazy-rescale threshold, log2 units

template <int D>
struct Tile {
    static constexpr int KP = D + 8;    // K row pitch in LDS (bf16 elements)
    static constexpr int VP = BN + 8;   // V^T row pitch in LDS (f16 elements)
    static constexpr int K_ELEMS = BN * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int KC = D / 16;   // reduction chunks of the score MFMA
    static constexpr int NT = D / 32;   // output tiles of the value MFMA
    static constexpr int K_LOADS = BN * (D / 8) / NTHREADS;  // 16-byte K loads per thread
    static constexpr int V_ITEMS = (BN / 4) * (D / 8);       // (key quad, 8 columns) items
    static_assert(K_LOADS * NTHREADS == BN * (D / 8), "K tile must split evenly");
    static_assert(V_ITEMS <= NTHREADS, "one V item per thread at most");
};

template <int D>
struct TileRegs {
    u32x4 k[Tile<D>::K_LOADS];
    u32x4 v[4];
};

// Position of local key j inside the transposed V tile: within each chunk of
// 16 keys, the 4-key blocks are stored in the order 0, 2, 1, 3.
__device__ __forceinline__ int vt_pos(int j) {
    const int kb = (j >> 2) & 3;
    const int pb = ((kb & 1) << 1) | (kb >> 1);
    return (j & ~15) | (pb << 2) | (j & 3);
}

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &t, const uint16_t *kbase,
                                          const uint16_t *vbase, int64_t k_l, int64_t v_l,
                                          int j0, int L, int tid) {
    using T = Tile<D>;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < T::K_LOADS; ++u) {
        const int c = tid + NTHREADS * u;
        const int row = c / (D / 8);
        const int col = (c % (D / 8)) * 8;
        const int j = j0 + row;
        t.k[u] = (j < L) ? ldg16(kbase + (int64_t)j * k_l + col) : zero;
    }
    if (tid < T::V_ITEMS) {
        const int a = tid & 15;
        const int cc = tid >> 4;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 4 * a + u;
            t.v[u] = (j < L) ? ldg16(vbase + (int64_t)j * v_l + 8 * cc) : zero;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &t, uint16_t *sk, uint16_t *sv,
                                           int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int u = 0; u < T::K_LOADS; ++u) {
        const int c = tid + NTHREADS * u;
        const int row = c / (D / 8);
        const int col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4 *>(sk + row * T::KP + col) = t.k[u];
    }
    if (tid < T::V_ITEMS) {
        const int a = tid & 15;
        const int cc = tid >> 4;
        const int pos = vt_pos(4 * a);
        float f[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                f[u][2 * w] = bf16_lo(t.v[u][w]);
                f[u][2 * w + 1] = bf16_hi(t.v[u][w]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f16x2 lo = cvt_f16x2(f[0][e], f[1][e]);
            const f16x2 hi = cvt_f16x2(f[2][e], f[3][e]);
            u32x2 w;
            w[0] = __builtin_bit_cast(uint32_t, lo);
            w[1] = __builtin_bit_cast(uint32_t, hi);
            *reinterpret_cast<u32x2 *>(sv + (8 * cc + e) * T::VP + pos) = w;
        }
    }
}

// 0 = no visible pair, 1 = every pair visible, 2 = needs a per-element mask.
__device__ __forceinline__ int classify(int j0, int r0, int r1, int L, int window, int n_sink) {
    const int j1 = j0 + 31;
    if (r1 < r0 || j0 > r1 || j0 >= L)
        return 0;
    if (window > 0 && j1 < r0 - window + 1 && j0 >= n_sink)
        return 0;
    if (j1 <= r0 && j1 < L && (window <= 0 || r1 - j0 < window || j1 < n_sink))
        return 1;
    return 2;
}

template <int D>
__global__ __launch_bounds__(NTHREADS) void parallax_fwd_kernel(FwdArgs a) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][T::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][T::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int L = a.L;
    const int i0 = qt * BM;
    const int i1 = min(i0 + BM, L) - 1;
    const int r0 = i0 + 32 * wave;
    const int r1 = min(r0 + 31, L - 1);
    const int row = r0 + l32;
    const int window = a.window;
    const int n_sink = a.n_sink;
    const float c = a.scale_log2;

    const uint16_t *qb = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h;
    const uint16_t *rb = a.r + (int64_t)b * a.r_b + (int64_t)h * a.r_h;
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;

    // Q and R fragments: B operand of S^T = K Q^T (lane: row l32, 8 features).
    bf16x8 qf[T::KC], rf[T::KC];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) {
            const int col = 16 * kc + 8 * g;
            const u32x4 qw = row < L ? ldg16(qb + (int64_t)row * a.q_l + col) : zero;
            const u32x4 rw = row < L ? ldg16(rb + (int64_t)row * a.r_l + col) : zero;
            qf[kc] = __builtin_bit_cast(bf16x8, qw);
            rf[kc] = __builtin_bit_cast(bf16x8, rw);
        }
    }

    // Key tiles with at least one visible pair for rows [i0, i1]: the sink
    // tiles that lie before the window, then the window/causal span.
    const int kt_hi = i1 / BN;
    int kt_lo = 0, n_st = 0;
    if (window > 0) {
        const int lo = i0 - window + 1;
        kt_lo = lo > 0 ? lo / BN : 0;
        n_st = min((n_sink + BN - 1) / BN, kt_lo);
    }
    const int n_tiles = n_st + (kt_hi - kt_lo + 1);

    f32x16 accA[T::NT], accC[T::NT];
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            accA[nt][e] = 0.f;
            accC[nt][e] = 0.f;
        }
    }
    float m_run = kNegInf, ell = 0.f, ssum = 0.f;
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    TileRegs<D> pre;
    load_tile<D>(pre, kb, vb, a.k_l, a.v_l, (n_st > 0 ? 0 : kt_lo) * BN, L, tid);
    store_tile<D>(pre, sK[0], sV[0], tid);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const int kt = t < n_st ? t : kt_lo + (t - n_st);
        if (t + 1 < n_tiles) {
            const int kn = (t + 1) < n_st ? (t + 1) : kt_lo + (t + 1 - n_st);
            load_tile<D>(pre, kb, vb, a.k_l, a.v_l, kn * BN, L, tid);
        }

        const int jt = kt * BN;
        int mode[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            mode[ks] = classify(jt + 32 * ks, r0, r1, L, window, n_sink);

        if (mode[0] | mode[1]) {
            const uint16_t *sk = sK[buf];
            const uint16_t *sv = sV[buf];
            f32x16 sq[2], sr[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sq[ks][e] = kNegInf;
                    sr[ks][e] = 0.f;
                }
                if (mode[ks] == 0)
                    continue;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sq[ks][e] = 0.f;
#pragma unroll
                for (int kc = 0; kc < T::KC; ++kc) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                        sk + (32 * ks + l32) * T::KP + 16 * kc + 8 * g);
                    sq[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kc], sq[ks], 0, 0, 0);
                    sr[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, rf[kc], sr[ks], 0, 0, 0);
                }
                if (mode[ks] == 2) {
                    const int j0 = jt + 32 * ks;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = j0 + 8 * (e >> 2) + 4 * g + (e & 3);
                        const bool vis = j <= row && j < L &&
                                         (window <= 0 || row - j < window || j < n_sink);
                        if (!vis)
                            sq[ks][e] = kNegInf;
                    }
                }
            }

            // Row max of this tile (raw scores; the scale is positive).
            float mt = kNegInf;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    mt = fmaxf(mt, sq[ks][e]);
            mt = fmaxf(mt, xor32(mt));
            const float mx = mt * c;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
                m_run = m_new;
                ell *= alpha;
                ssum *= alpha;
#pragma unroll
                for (int nt = 0; nt < T::NT; ++nt) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        accA[nt][e] *= alpha;
                        accC[nt][e] *= alpha;
                    }
                }
            }
            const float msub = (m_run == kNegInf) ? 0.f : m_run;

#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (mode[ks] == 0)
                    continue;
                f16x8 pf[2], wf[2];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int e = 8 * ch + 2 * e2;
                        const float p0 = exp2_fast(fmaf(sq[ks][e], c, -msub));
                        const float p1 = exp2_fast(fmaf(sq[ks][e + 1], c, -msub));
                        const f16x2 ph = cvt_f16x2(p0, p1);
                        const f16x2 wh = cvt_f16x2(p0 * sr[ks][e], p1 * sr[ks][e + 1]);
                        ell = __builtin_amdgcn_fdot2(ph, ones, ell, false);
                        ssum = __builtin_amdgcn_fdot2(wh, ones, ssum, false);
                        pf[ch][2 * e2] = ph[0];
                        pf[ch][2 * e2 + 1] = ph[1];
                        wf[ch][2 * e2] = wh[0];
                        wf[ch][2 * e2 + 1] = wh[1];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < T::NT; ++nt) {
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch) {
                        const f16x8 vf = *reinterpret_cast<const f16x8 *>(
                            sv + (32 * nt + l32) * T::VP + 32 * ks + 16 * ch + 8 * g);
                        accA[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ch], accA[nt], 0, 0, 0);
                        accC[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, wf[ch], accC[nt], 0, 0, 0);
                    }
                }
            }
        }

        if (t + 1 < n_tiles)
            store_tile<D>(pre, sK[buf ^ 1], sV[buf ^ 1], tid);
        __syncthreads();
    }

    // Epilogue: combine the two half-wave partial sums of each row.
    const float ell_t = ell + xor32(ell);
    const float s_t = ssum + xor32(ssum);
    if (row < L) {
        const float inv = 1.f / ell_t;
        const float keep = 1.f - s_t * inv;
        float *ob = a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)row * a.o_l;
#pragma unroll
        for (int nt = 0; nt < T::NT; ++nt) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                f32x4 out;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = 4 * grp + u;
                    out[u] = (accA[nt][e] * keep + accC[nt][e]) * inv;
                }
                *reinterpret_cast<f32x4 *>(ob + 32 * nt + 8 * grp + 4 * g) = out;
            }
        }
        if (g == 0)
            a.lse[(int64_t)bh * L + row] = (m_run + log2f(ell_t)) * kLn2;
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
