// Parallax decode step for gfx950: one query and probe per (sequence, head)
// against a contiguous bf16 KV cache.
//
// A decoding Parallax model keeps a KV cache like softmax attention (tilnote
// note on Parallax, section on it being a different estimator rather than a
// linear-time attention), and reading that cache is the cost: the KV cache
// is the memory bottleneck of inference ("Simple linear attention language
// models balance the recall-throughput tradeoff" review, abstract and
// motivation; "Sliding-window beats linear attention" review, sec. 1).  The
// kernel is therefore built to stream K and V from HBM once, with many
// 16-byte loads in flight, and to keep all arithmetic in fp32.
//
// Work split: one workgroup per (b, h) with NS wavefronts; wavefront s owns
// one contiguous chunk of the cache.  Inside a wavefront, D/8 lanes share a
// key (16 bytes = 8 features each), so a wave step covers 512/D keys and
// every global load is fully coalesced.  Loads go through buffer resources
// that end at the chunk's last row (rows past it read as zeros, no
// branches), the per-key dot products are summed across the D/8 lanes with
// DPP moves, and two wave steps per iteration keep the kernel within 64
// VGPRs: eight wavefronts per SIMD, so two workgroups share a CU and one
// streams while the other merges.  Each lane group keeps running
//     m, ell = sum p~, S = sum p~ s, A = sum p~ v, C = sum p~ s v
// (s = rho . k, p~ = 2^(x - m)) for its 8 features.  The partial states are
// merged first across lane groups with shuffles, then across wavefronts
// through LDS, by rescaling each (ell, S, A, C) with 2^(m_s - M).  The
// normalised pair (o, lse) would NOT merge correctly for Parallax because
// the correction's key mean depends on the whole visible set; the
// un-normalised sums do.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace plx {
namespace {

// Sum over aligned groups of N lanes (N = 8 or 16) with DPP moves on the
// VALU: quad swaps, then the half-row and row mirrors pair the quads and the
// half-rows.  Every lane of a group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                               0xF, 0xF, false));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (N == 16)
        x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
    return x;
}

template <int D, int NS>
__global__ __launch_bounds__(64 * NS) void parallax_decode_kernel(DecodeArgs a) {
    constexpr int LPK = D / 8;     // lanes per key
    constexpr int KPS = 64 / LPK;  // keys per wave step
    constexpr int U = 2;           // wave steps per iteration (loads in flight)

    __shared__ float s_m[NS], s_l[NS], s_s[NS];
    __shared__ float s_A[NS][D], s_C[NS][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    const int bh = blockIdx.x;
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const float c = a.scale_log2;

    int n = a.seqlens ? a.seqlens[b] : a.Lmax;
    n = n < 0 ? 0 : (n > a.Lmax ? a.Lmax : n);
    const int chunk = (n + NS - 1) / NS;
    const int start = min(wave * chunk, n);
    const int end = min(start + chunk, n);

    float qv[8], rv[8];
    {
        const u32x4 qw = ldg16(a.q + (int64_t)bh * D + 8 * sub);
        const u32x4 rw = ldg16(a.r + (int64_t)bh * D + 8 * sub);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            qv[2 * w] = bf16_lo(qw[w]);
            qv[2 * w + 1] = bf16_hi(qw[w]);
            rv[2 * w] = bf16_lo(rw[w]);
            rv[2 * w + 1] = bf16_hi(rw[w]);
        }
    }
    // Each iteration reads rows [j, j + KPS*U) through buffer resources that
    // end at the chunk's last row, so rows past it read as zeros.
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h + (int64_t)start * a.k_l;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h + (int64_t)start * a.v_l;
    const uint32_t koff = (uint32_t)(grp * a.k_l * 2 + 16 * sub);
    const uint32_t voff = (uint32_t)(grp * a.v_l * 2 + 16 * sub);
    const uint32_t kstep = (uint32_t)(KPS * a.k_l * 2);
    const uint32_t vstep = (uint32_t)(KPS * a.v_l * 2);

    float m = kNegInf, ell = 0.f, ssum = 0.f;
    float A[8], C[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        A[e] = 0.f;
        C[e] = 0.f;
    }

    for (int j = start; j < end; j += KPS * U) {
        const __amdgpu_buffer_rsrc_t ks =
            make_rsrc(kb + (int64_t)(j - start) * a.k_l, rows_bytes(j, end, a.k_l, D));
        const __amdgpu_buffer_rsrc_t vs =
            make_rsrc(vb + (int64_t)(j - start) * a.v_l, rows_bytes(j, end, a.v_l, D));
        u32x4 kw[U], vw[U];
        bool valid[U];
        // The cache is read once per call: non-temporal loads (nt) keep it
        // from displacing other data in L2 and the MALL.
        constexpr int kNonTemporal = 2;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            valid[u] = j + u * KPS + grp < end;
            kw[u] = __builtin_amdgcn_raw_buffer_load_b128(ks, (int)koff, (int)(u * kstep), kNonTemporal);
            vw[u] = __builtin_amdgcn_raw_buffer_load_b128(vs, (int)voff, (int)(u * vstep), kNonTemporal);
        }
        float x[U], sr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float dq = 0.f, dr = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float k0 = bf16_lo(kw[u][w]);
                const float k1 = bf16_hi(kw[u][w]);
                dq = fmaf(qv[2 * w], k0, dq);
                dq = fmaf(qv[2 * w + 1], k1, dq);
                dr = fmaf(rv[2 * w], k0, dr);
                dr = fmaf(rv[2 * w + 1], k1, dr);
            }
            dq = group_sum<LPK>(dq);
            dr = group_sum<LPK>(dr);
            x[u] = valid[u] ? dq * c : kNegInf;
            sr[u] = dr;
        }
        float mt = x[0];
#pragma unroll
        for (int u = 1; u < U; ++u)
            mt = fmaxf(mt, x[u]);
        const float m_new = fmaxf(m, mt);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m - m_new);
        m = m_new;
        const float msub = (m == kNegInf) ? 0.f : m;
        ell *= alpha;
        ssum *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            A[e] *= alpha;
            C[e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = exp2_fast(x[u] - msub);
            const float w = p * sr[u];
            ell += p;
            ssum += w;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const float v0 = bf16_lo(vw[u][q2]);
                const float v1 = bf16_hi(vw[u][q2]);
                A[2 * q2] = fmaf(p, v0, A[2 * q2]);
                A[2 * q2 + 1] = fmaf(p, v1, A[2 * q2 + 1]);
                C[2 * q2] = fmaf(w, v0, C[2 * q2]);
                C[2 * q2 + 1] = fmaf(w, v1, C[2 * q2 + 1]);
            }
        }
    }

    // Merge the lane groups of this wavefront (same features, disjoint keys).
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m, off, 64);
        const float lo = __shfl_xor(ell, off, 64);
        const float so = __shfl_xor(ssum, off, 64);
        const float M = fmaxf(m, mo);
        const float f = (M == kNegInf) ? 0.f : exp2_fast(m - M);
        const float fo = (M == kNegInf) ? 0.f : exp2_fast(mo - M);
        ell = ell * f + lo * fo;
        ssum = ssum * f + so * fo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            A[e] = A[e] * f + __shfl_xor(A[e], off, 64) * fo;
            C[e] = C[e] * f + __shfl_xor(C[e], off, 64) * fo;
        }
        m = M;
    }
    if (lane < LPK) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s_A[wave][8 * sub + e] = A[e];
            s_C[wave][8 * sub + e] = C[e];
        }
        if (lane == 0) {
            s_m[wave] = m;
            s_l[wave] = ell;
            s_s[wave] = ssum;
        }
    }
    __syncthreads();

    // Merge the wavefronts' chunks and write the row.
    float M = kNegInf;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        M = fmaxf(M, s_m[s]);
    float lt = 0.f, st = 0.f;
    float f[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        f[s] = (M == kNegInf) ? 0.f : exp2_fast(s_m[s] - M);
        lt += f[s] * s_l[s];
        st += f[s] * s_s[s];
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float keep = 1.f - st * inv;
    for (int nidx = tid; nidx < D; nidx += 64 * NS) {
        float at = 0.f, ct = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            at += f[s] * s_A[s][nidx];
            ct += f[s] * s_C[s][nidx];
        }
        a.o[(int64_t)bh * D + nidx] = (at * keep + ct) * inv;
    }
    if (tid == 0)
        a.lse[bh] = lt > 0.f ? (M + log2f(lt)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// General decode: a paged (or contiguous) cache, grouped kv heads, and a
// sliding window with attention sinks at decode ("Sliding-window beats linear
// attention" review, sec. 1 and sec. 3: windowed attention with sink tokens
// keeps a fixed-size KV cache).  The same partial-state scheme as above;
// what changes is which rows are read and where they live.
//   * Query head h reads kv head h / (Hq / Hkv).  A workgroup serves GW
//     query heads of one kv head with NS wavefronts each (wavefront w:
//     head w % GW, key chunk w / GW), so the GW wavefronts of a chunk read
//     the same cache rows on one CU.  Workgroups of one kv head get block
//     indices with the same residue mod 8 (one XCD, one L2) when the group
//     needs several of them.  Loads are cached when rows are shared and
//     non-temporal when they are not (Hq = Hkv).
//   * The query at position n-1 sees the sink keys [0, ns) and the window
//     [lo, n) (all of [0, n) without a window); the NS wavefronts split the
//     concatenation of the two segments evenly.
//   * Paged: key j lives in page block_table[b][j >> page_shift] (clamped
//     into the pool), row j & (page size - 1).  Contiguous: page b, row j.  A lane's key index
//     is clamped into its segment before the address is formed, so every
//     load reads a visible row of the sequence; the results of clamped
//     lanes are masked.

template <int D, int NS, int GW, bool PAGED, bool NT>
__global__ __launch_bounds__(64 * NS * GW) void parallax_decode_paged_kernel(PagedDecodeArgs a) {
    constexpr int LPK = D / 8;     // lanes per key
    constexpr int KPS = 64 / LPK;  // keys per wave step
    constexpr int U = 2;           // wave steps per iteration

    __shared__ float s_m[GW][NS], s_l[GW][NS], s_s[GW][NS];
    __shared__ float s_A[GW][NS][D], s_C[GW][NS][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = wv % GW;     // query head of the workgroup's group
    const int wave = wv / GW;     // key chunk
    const int grp = lane / LPK;
    const int sub = lane % LPK;

    // Block -> (sequence, kv head, group of GW query heads).
    const int g = a.Hq / a.Hkv;
    const int ng = g / GW;        // workgroups per kv head
    const int x = blockIdx.x;
    const int slot = x >> 3;
    const int pair = (slot / ng) * 8 + (x & 7);
    if (pair >= a.B * a.Hkv)
        return;
    const int b = pair / a.Hkv;
    const int hk = pair - b * a.Hkv;
    const int hq = hk * g + (slot - (slot / ng) * ng) * GW + head;
    const int64_t row_q = (int64_t)b * a.Hq + hq;
    const float c = a.scale_log2;

    int n = a.seqlens ? a.seqlens[b] : a.max_len;
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    int lo = 0, ns = 0;
    if (a.window > 0) {
        lo = max(0, n - a.window);
        ns = min(a.n_sink, lo);
    }
    const int total = ns + (n - lo);
    const int chunk = (total + NS - 1) / NS;
    const int ts = min(wave * chunk, total);
    const int te = min(ts + chunk, total);

    float qv[8], rv[8];
    {
        const u32x4 qw = ldg16(a.q + row_q * D + 8 * sub);
        const u32x4 rw = ldg16(a.r + row_q * D + 8 * sub);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            qv[2 * w] = bf16_lo(qw[w]);
            qv[2 * w + 1] = bf16_hi(qw[w]);
            rv[2 * w] = bf16_lo(rw[w]);
            rv[2 * w + 1] = bf16_hi(rw[w]);
        }
    }
    const uint16_t *kbase = a.k + (int64_t)hk * a.k_h + 8 * sub;
    const uint16_t *vbase = a.v + (int64_t)hk * a.v_h + 8 * sub;
    const int32_t *bt = PAGED ? a.block_table + (int64_t)b * a.max_pages : nullptr;
    const int pmask = (1 << a.page_shift) - 1;

    float m = kNegInf, ell = 0.f, ssum = 0.f;
    float A[8], C[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        A[e] = 0.f;
        C[e] = 0.f;
    }

    // Keys [j0, j1) of the sequence (j0 < j1).
    auto process = [&](int j0, int j1) __attribute__((always_inline)) {
        for (int j = j0; j < j1; j += KPS * U) {
            u32x4 kw[U], vw[U];
            bool valid[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kj = j + u * KPS + grp;
                valid[u] = kj < j1;
                const int kc = valid[u] ? kj : j1 - 1;
                int64_t page, row;
                if constexpr (PAGED) {
                    page = min(max(bt[kc >> a.page_shift], 0), a.num_pages - 1);
                    row = kc & pmask;
                } else {
                    page = b;
                    row = kc;
                }
                // One query head per kv head: the rows are read once
                // (non-temporal loads); otherwise the other heads of the
                // group read them too (cached loads).
                const u32x4 *kp = reinterpret_cast<const u32x4 *>(kbase + page * a.k_p + row * a.k_l);
                const u32x4 *vp = reinterpret_cast<const u32x4 *>(vbase + page * a.v_p + row * a.v_l);
                if constexpr (NT) {
                    kw[u] = __builtin_nontemporal_load(kp);
                    vw[u] = __builtin_nontemporal_load(vp);
                } else {
                    kw[u] = *kp;
                    vw[u] = *vp;
                }
            }
            float xs[U], sr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dq = 0.f, dr = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float k0 = bf16_lo(kw[u][w]);
                    const float k1 = bf16_hi(kw[u][w]);
                    dq = fmaf(qv[2 * w], k0, dq);
                    dq = fmaf(qv[2 * w + 1], k1, dq);
                    dr = fmaf(rv[2 * w], k0, dr);
                    dr = fmaf(rv[2 * w + 1], k1, dr);
                }
                dq = group_sum<LPK>(dq);
                dr = group_sum<LPK>(dr);
                xs[u] = valid[u] ? dq * c : kNegInf;
                sr[u] = dr;
            }
            float mt = xs[0];
#pragma unroll
            for (int u = 1; u < U; ++u)
                mt = fmaxf(mt, xs[u]);
            const float m_new = fmaxf(m, mt);
            const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m - m_new);
            m = m_new;
            const float msub = (m == kNegInf) ? 0.f : m;
            ell *= alpha;
            ssum *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                A[e] *= alpha;
                C[e] *= alpha;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = exp2_fast(xs[u] - msub);
                const float w = p * sr[u];
                ell += p;
                ssum += w;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const float v0 = bf16_lo(vw[u][q2]);
                    const float v1 = bf16_hi(vw[u][q2]);
                    A[2 * q2] = fmaf(p, v0, A[2 * q2]);
                    A[2 * q2 + 1] = fmaf(p, v1, A[2 * q2 + 1]);
                    C[2 * q2] = fmaf(w, v0, C[2 * q2]);
                    C[2 * q2 + 1] = fmaf(w, v1, C[2 * q2 + 1]);
                }
            }
        }
    };
    // Segment 1: sink keys [ts, min(te, ns)); segment 2: window keys.
    if (ts < ns)
        process(ts, min(te, ns));
    if (te > ns) {
        const int v0 = max(ts, ns);
        process(lo + (v0 - ns), lo + (te - ns));
    }

    // Merge the lane groups, then the wavefronts (as in the kernel above).
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m, off, 64);
        const float lo2 = __shfl_xor(ell, off, 64);
        const float so = __shfl_xor(ssum, off, 64);
        const float M = fmaxf(m, mo);
        const float f = (M == kNegInf) ? 0.f : exp2_fast(m - M);
        const float fo = (M == kNegInf) ? 0.f : exp2_fast(mo - M);
        ell = ell * f + lo2 * fo;
        ssum = ssum * f + so * fo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            A[e] = A[e] * f + __shfl_xor(A[e], off, 64) * fo;
            C[e] = C[e] * f + __shfl_xor(C[e], off, 64) * fo;
        }
        m = M;
    }
    if (lane < LPK) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s_A[head][wave][8 * sub + e] = A[e];
            s_C[head][wave][8 * sub + e] = C[e];
        }
        if (lane == 0) {
            s_m[head][wave] = m;
            s_l[head][wave] = ell;
            s_s[head][wave] = ssum;
        }
    }
    __syncthreads();

    // Merge the chunks of each head: index t covers feature t % D of head
    // t / D of the group.
    for (int t = tid; t < GW * D; t += 64 * NS * GW) {
        const int hj = t / D;
        const int nidx = t - hj * D;
        float M = kNegInf;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            M = fmaxf(M, s_m[hj][s]);
        float lt = 0.f, st = 0.f, at = 0.f, ct = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float f = (M == kNegInf) ? 0.f : exp2_fast(s_m[hj][s] - M);
            lt += f * s_l[hj][s];
            st += f * s_s[hj][s];
            at += f * s_A[hj][s][nidx];
            ct += f * s_C[hj][s][nidx];
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const float keep = 1.f - st * inv;
        const int64_t row = row_q - head + hj;
        a.o[row * D + nidx] = (at * keep + ct) * inv;
        if (nidx == 0)
            a.lse[row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// General decode on the matrix cores for grouped heads (Hq / Hkv >= 4).  The
// query heads that share a kv head become the columns of MFMA tiles, so a
// workgroup reads every cache row once and the per-key products run on the
// matrix cores instead of the VALU (with 16 lanes per key, the VALU kernel
// above spends about 17 wavefront instructions per key and query head,
// which bounds it once the rows are shared by several heads):
//   * a workgroup serves (sequence, kv head, GQ query heads); its NS
//     wavefronts split the visible keys (sink segment, then window) evenly;
//   * per 32-key stage a wavefront loads K straight into the A fragments of
//     S^T = K Q^T (16 keys x 32 features: one 16-byte load per lane), and V
//     as 8 keys x 8 features per lane, transposed in registers into its own
//     LDS stage as the V^T fragments of the value MFMAs;
//   * S^T = K Q^T and K R^T (bf16, columns past the group's heads are zero),
//     an online softmax per column, weights p~ and p~ s each as an f16 value
//     plus its f16 residual, then O^T += V^T P~^T and V^T (P~ o S)^T, with
//     the sums of p~ and p~ s from an all-ones operand (f16 MFMAs, fp32
//     sums), as in the prefill's precise mode;
//   * the NS partial states of each head merge in LDS (the stage memory,
//     reused after one barrier);
//   * with a caller workspace and fewer workgroups than CUs, several
//     workgroups take consecutive slices of the visible keys, write their
//     merged (m, ell, S, A, C) per query head to the workspace, and
//     parallax_decode_split_merge_kernel combines them the same way.
// Each wavefront's stage count differs, so the loop synchronises within the
// wavefront only.
// 16-byte slot of chunk q (reduction positions 8q .. 8q+7) of V^T row r in a
// [D][32] f16 stage: rows 4 apart share banks, so the chunk is rotated.
__device__ __forceinline__ int gqa_slot(int r, int q) { return 4 * r + (q ^ ((r >> 2) & 3)); }

template <int D, int NS, int GQ>
struct GqaShape {
    static constexpr int KC = D / 32;
    static constexpr int DT = D / 16;
    static constexpr int FCH = D / 8;                  // 16-byte feature chunks
    static constexpr int VT_HALVES = D * 32;           // one wavefront's V^T stage
    static constexpr int MERGE_FLOATS = NS * GQ * (2 * D + 3);
    static constexpr int LDS_HALVES =
        NS * VT_HALVES > 2 * MERGE_FLOATS ? NS * VT_HALVES : 2 * MERGE_FLOATS;
};

template <int D, int NS, int GQ, bool PAGED>
__global__ __launch_bounds__(64 * NS) void parallax_decode_gqa_kernel(PagedDecodeArgs a) {
    using S = GqaShape<D, NS, GQ>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_HALVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;

    const int g = a.Hq / a.Hkv;
    const int ngrp = (g + GQ - 1) / GQ;
    // Block v serves query group (v / 8) % ngrp of (sequence, kv head) pair
    // 8 ((v / 8) / ngrp) + v % 8: the ngrp workgroups of a pair share an XCD
    // (block v runs on XCD v % 8) and read its cache rows through one L2.
    // Blocks past the last pair (the grid is rounded up to 8 pairs) exit.
    // With key splits, block ks * nbase + v takes split ks of block v's keys
    // (nbase is a multiple of 8, so the mapping above is unchanged).
    const int nbase = ((a.B * a.Hkv + 7) / 8) * 8 * ngrp;
    const int ks = (int)blockIdx.x / nbase;
    const int vblk = (int)blockIdx.x - ks * nbase;
    const int vb = vblk >> 3;
    const int pair = (vb / ngrp) * 8 + (vblk & 7);
    const int grp = vb % ngrp;
    if (pair >= a.B * a.Hkv)
        return;
    const int b = pair / a.Hkv;
    const int hk = pair - b * a.Hkv;
    const int q0 = hk * g + grp * GQ;            // first query head of the workgroup
    const int ncol = min(GQ, g - grp * GQ);      // query heads it serves
    const float c = a.scale_log2;

    int n = a.seqlens ? a.seqlens[b] : a.max_len;
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    int lo = 0, ns = 0;
    if (a.window > 0) {
        lo = max(0, n - a.window);
        ns = min(a.n_sink, lo);
    }
    const int total = ns + (n - lo);
    // This workgroup's split of the visible keys, then each wavefront's chunk.
    const int kchunk = (total + a.ksplit - 1) / a.ksplit;
    const int sub_lo = min(ks * kchunk, total);
    const int sub_hi = min(sub_lo + kchunk, total);
    const int chunk = (sub_hi - sub_lo + NS - 1) / NS;
    const int ts = min(sub_lo + wave * chunk, sub_hi);
    const int te = min(ts + chunk, sub_hi);

    // Q^T and R^T B fragments: column l16 = query head q0 + l16, features
    // 32 kc + 8G .. +7 (zeros past the group's heads).
    bf16x8 qf[S::KC], rf[S::KC];
#pragma unroll
    for (int kc = 0; kc < S::KC; ++kc) {
        u32x4 qw = {0u, 0u, 0u, 0u}, rw = {0u, 0u, 0u, 0u};
        if (l16 < ncol) {
            const int64_t row = (int64_t)b * a.Hq + q0 + l16;
            qw = ldg16(a.q + row * D + 32 * kc + 8 * G);
            rw = ldg16(a.r + row * D + 32 * kc + 8 * G);
        }
        qf[kc] = __builtin_bit_cast(bf16x8, qw);
        rf[kc] = __builtin_bit_cast(bf16x8, rw);
    }

    const uint16_t *kbase = a.k + (int64_t)hk * a.k_h;
    const uint16_t *vbase = a.v + (int64_t)hk * a.v_h;
    const int32_t *bt = PAGED ? a.block_table + (int64_t)b * a.max_pages : nullptr;
    const int pmask = (1 << a.page_shift) - 1;
    // Offset (elements) of visible key li's row, li clamped into [ts, te).
    auto row_of = [&](int li, const uint16_t *base, int64_t sp, int64_t sl) __attribute__((always_inline)) {
        const int lc = min(li, te - 1);
        const int kp = lc < ns ? lc : lo + (lc - ns);
        int64_t page, r;
        if constexpr (PAGED) {
            page = min(max(bt[kp >> a.page_shift], 0), a.num_pages - 1);
            r = kp & pmask;
        } else {
            page = b;
            r = kp;
        }
        return base + page * sp + r * sl;
    };

    uint16_t *vt = lds + wave * S::VT_HALVES;  // this wavefront's V^T stage
    f32x4 accA[S::DT], accC[S::DT], accL, accS;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
        accA[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        accC[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    accL = accS = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = kNegInf;  // running offset of column l16 (scaled log2 units)
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    // V loads: lane (vg = lane % 4, vm = lane / 4) holds features 8 vm .. +7
    // of the keys at reduction positions 8 vg .. 8 vg + 7.
    const int vg = lane & 3, vm = lane >> 2;

    for (int s0 = ts; s0 < te; s0 += 32) {
        bf16x8 kf[2][S::KC];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint16_t *kr = row_of(s0 + 16 * kt + l16, kbase, a.k_p, a.k_l);
#pragma unroll
            for (int kc = 0; kc < S::KC; ++kc)
                kf[kt][kc] = __builtin_bit_cast(bf16x8, ldg16(kr + 32 * kc + 8 * G));
        }
        u32x4 vw[8];
        if (vm < S::FCH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * vg + e;  // reduction position -> stage key
                const int key = ((j >> 2) & 1) * 16 + (j >> 3) * 4 + (j & 3);
                vw[e] = ldg16(row_of(s0 + key, vbase, a.v_p, a.v_l) + 8 * vm);
            }
        }
        // Scores: S^T tiles (16 keys x 16 heads) for keys 0-15 and 16-31.
        f32x4 sq[2], sr[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sq[kt] = sr[kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < S::KC; ++kc) {
                sq[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][kc], qf[kc], sq[kt], 0, 0, 0);
                sr[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][kc], rf[kc], sr[kt], 0, 0, 0);
            }
        }
        // V^T into this wavefront's stage: 8 feature rows of 16 bytes.
        if (vm < S::FCH) {
            uint32_t h[8][4];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    h[e][w] = __builtin_bit_cast(uint32_t, cvt_f16x2(bf16_lo(vw[e][w]), bf16_hi(vw[e][w])));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x4 out;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const uint32_t x0 = h[2 * pp][i / 2], x1 = h[2 * pp + 1][i / 2];
                    out[pp] = (i & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
                }
                *reinterpret_cast<u32x4 *>(vt + gqa_slot(8 * vm + i, vg) * 8) = out;
            }
        }
        // Online softmax per column: the stage max over the lane's 8 keys
        // and the 4 lanes of the column.
        float x[8];
        float mt = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool valid = s0 + 16 * kt + 4 * G + e < te;
                x[4 * kt + e] = valid ? sq[kt][e] * c : kNegInf;
                mt = fmaxf(mt, x[4 * kt + e]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m, mt);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m - m_new);
        m = m_new;
        const float msub = (m == kNegInf) ? 0.f : m;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                accA[dt][e] *= alpha;
                accC[dt][e] *= alpha;
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            accL[e] *= alpha;
            accS[e] *= alpha;
        }
        // Each weight reaches the matrix core as two f16 parts, the rounded
        // value and its rounded residual (about 22 significant bits): the
        // loop is bound by the cache reads, so the extra products are free,
        // and the output keeps its accuracy for large probe scores.
        f16x8 wp, ws, wpl, wsl;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = exp2_fast(x[4 * kt + e] - msub);
                const float w = p * sr[kt][e];
                wp[4 * kt + e] = (_Float16)p;
                ws[4 * kt + e] = (_Float16)w;
                wpl[4 * kt + e] = (_Float16)(p - (float)wp[4 * kt + e]);
                wsl[4 * kt + e] = (_Float16)(w - (float)ws[4 * kt + e]);
            }
        // The stage's V^T writes are visible to the whole wavefront.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f16x8 vf[S::DT];
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
            vf[dt] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                   vt + gqa_slot(16 * dt + l16, G) * 8));
        accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, wp, accL, 0, 0, 0);
        accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, ws, accS, 0, 0, 0);
        accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, wpl, accL, 0, 0, 0);
        accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, wsl, accS, 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
            accA[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], wp, accA[dt], 0, 0, 0);
            accC[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], ws, accC[dt], 0, 0, 0);
            accA[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], wpl, accA[dt], 0, 0, 0);
            accC[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], wsl, accC[dt], 0, 0, 0);
        }
        // The next stage rewrites the V^T stage: its reads are done first.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Merge: wavefront w's state of column c at [w][c] (m, ell, S, A[D],
    // C[D]) in the stage memory, once every wavefront is done with it.
    __syncthreads();
    float *mg = reinterpret_cast<float *>(lds);
    auto rec = [&](int w, int col) { return mg + (w * GQ + col) * (2 * D + 3); };
    if (l16 < GQ) {
        float *r0 = rec(wave, l16);
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r0[3 + 16 * dt + 4 * G + e] = accA[dt][e];
                r0[3 + D + 16 * dt + 4 * G + e] = accC[dt][e];
            }
        if (G == 0) {
            r0[0] = m;
            r0[1] = accL[0];
            r0[2] = accS[0];
        }
    }
    __syncthreads();
    for (int t = tid; t < GQ * D; t += 64 * NS) {
        const int col = t / D;
        const int f = t - col * D;
        if (col >= ncol)
            continue;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NS; ++w)
            M = fmaxf(M, rec(w, col)[0]);
        float lt = 0.f, st = 0.f, at = 0.f, ct = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) {
            const float *r0 = rec(w, col);
            const float fw = (M == kNegInf) ? 0.f : exp2_fast(r0[0] - M);
            lt += fw * r0[1];
            st += fw * r0[2];
            at += fw * r0[3 + f];
            ct += fw * r0[3 + D + f];
        }
        const int64_t row = (int64_t)b * a.Hq + q0 + col;
        if (a.ksplit > 1) {
            // This split's partial state; the merge launch finishes the row.
            float *pr = a.part + (row * a.ksplit + ks) * (2 * D + 3);
            pr[3 + f] = at;
            pr[3 + D + f] = ct;
            if (f == 0) {
                pr[0] = M;
                pr[1] = lt;
                pr[2] = st;
            }
            continue;
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const float keep = 1.f - st * inv;
        a.o[row * D + f] = (at * keep + ct) * inv;
        if (f == 0)
            a.lse[row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : kNegInf;
    }
}

// Merge of the key splits' partial states of each (sequence, query head):
// the same rescaled sums as the merge across wavefronts, then the epilogue.
// One workgroup of D threads per row, thread f owning feature f.
template <int D>
__global__ __launch_bounds__(D) void parallax_decode_split_merge_kernel(PagedDecodeArgs a) {
    const int64_t row = blockIdx.x;
    const int f = threadIdx.x;
    const int S = a.ksplit;
    const float *pr = a.part + row * S * (2 * D + 3);
    float M = kNegInf;
    for (int s = 0; s < S; ++s)
        M = fmaxf(M, pr[s * (2 * D + 3)]);
    float lt = 0.f, st = 0.f, at = 0.f, ct = 0.f;
    for (int s = 0; s < S; ++s) {
        const float *r0 = pr + s * (2 * D + 3);
        const float fw = (M == kNegInf) ? 0.f : exp2_fast(r0[0] - M);
        lt += fw * r0[1];
        st += fw * r0[2];
        at += fw * r0[3 + f];
        ct += fw * r0[3 + D + f];
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float keep = 1.f - st * inv;
    a.o[row * D + f] = (at * keep + ct) * inv;
    if (f == 0)
        a.lse[row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : kNegInf;
}

// With a workspace, calls with fewer workgroups than the chip has CUs split
// each kv head's keys over up to kDecodeMaxKeySplits workgroups (MQA over 64
// sequences: 4 splits, 256 workgroups); each workgroup's wavefronts walk a
// shorter chain of stages, and a merge launch combines the splits.
constexpr int kDecodeCUs = 256;  // compute units of the MI355X
template <int D, int NS, int GQ>
hipError_t launch_decode_gqa_t(const PagedDecodeArgs &a, hipStream_t stream) {
    const int g = a.Hq / a.Hkv;
    const int64_t pairs8 = ((int64_t)a.B * a.Hkv + 7) / 8 * 8;
    const int64_t nbase = pairs8 * ((g + GQ - 1) / GQ);
    PagedDecodeArgs args = a;
    args.ksplit = 1;
    if (a.part && nbase < kDecodeCUs)
        args.ksplit = (int)std::min<int64_t>(kDecodeMaxKeySplits, (kDecodeCUs + nbase - 1) / nbase);
    void *params[] = {&args};
    const void *fn = a.block_table
                         ? reinterpret_cast<const void *>(&parallax_decode_gqa_kernel<D, NS, GQ, true>)
                         : reinterpret_cast<const void *>(&parallax_decode_gqa_kernel<D, NS, GQ, false>);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(nbase * args.ksplit)), dim3(64 * NS), params,
                                   0, stream);
    if (e != hipSuccess || args.ksplit == 1)
        return e;
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_decode_split_merge_kernel<D>),
                           dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(D), params, 0, stream);
}

// Columns per workgroup: 4, 8 or 16 (the group, rounded up, at most 16).
// (Smaller groups for calls with few (sequence, kv head) pairs, e.g. MQA
// over 64 sequences as 256 workgroups of 4 query heads instead of 64 of 16,
// measured the same: each wavefront still walks the same chain of stages.)
// Wavefronts: the requested splits, at most 8 (up to 256 registers per lane;
// with 16 columns also the LDS of the merge).
template <int D>
hipError_t launch_decode_gqa(const PagedDecodeArgs &a, int num_splits, hipStream_t stream) {
    const int g = a.Hq / a.Hkv;
    const int gq = g <= 4 ? 4 : (g <= 8 ? 8 : 16);
    const int ns = min(num_splits, 8);
#define PLX_GQA(NSV)                                                   \
    if (ns == NSV) {                                                   \
        if (gq == 4) return launch_decode_gqa_t<D, NSV, 4>(a, stream); \
        if (gq == 8) return launch_decode_gqa_t<D, NSV, 8>(a, stream); \
        return launch_decode_gqa_t<D, NSV, 16>(a, stream);             \
    }
    PLX_GQA(1)
    PLX_GQA(2)
    PLX_GQA(4)
    PLX_GQA(8)
#undef PLX_GQA
    return hipErrorInvalidValue;
}

template <int D, int NS, int GW>
hipError_t launch_decode_paged_t(const PagedDecodeArgs &a, hipStream_t stream) {
    const int pairs = a.B * a.Hkv;
    const int ng = a.Hq / a.Hkv / GW;
    const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * ng));
    const dim3 block(64 * NS * GW);
    PagedDecodeArgs args = a;
    void *params[] = {&args};
    const void *fn;
    if (a.Hq == a.Hkv)
        fn = a.block_table
                 ? reinterpret_cast<const void *>(&parallax_decode_paged_kernel<D, NS, GW, true, true>)
                 : reinterpret_cast<const void *>(&parallax_decode_paged_kernel<D, NS, GW, false, true>);
    else
        fn = a.block_table
                 ? reinterpret_cast<const void *>(&parallax_decode_paged_kernel<D, NS, GW, true, false>)
                 : reinterpret_cast<const void *>(&parallax_decode_paged_kernel<D, NS, GW, false, false>);
    return hipLaunchKernel(fn, grid, block, params, 0, stream);
}

// Heads per workgroup: the largest power of two dividing Hq/Hkv with at
// most 16 wavefronts per workgroup (NS key chunks per head come first:
// they keep enough workgroups in flight when B * Hkv is small).
template <int D, int NS>
hipError_t launch_decode_paged_g(const PagedDecodeArgs &a, hipStream_t stream) {
    const int g = a.Hq / a.Hkv;
    int gw = 1;
    while (gw * 2 * NS <= 16 && g % (gw * 2) == 0)
        gw *= 2;
    if constexpr (NS <= 1) {
        if (gw == 16) return launch_decode_paged_t<D, NS, 16>(a, stream);
    }
    if constexpr (NS <= 2) {
        if (gw == 8) return launch_decode_paged_t<D, NS, 8>(a, stream);
    }
    if constexpr (NS <= 4) {
        if (gw == 4) return launch_decode_paged_t<D, NS, 4>(a, stream);
    }
    if constexpr (NS <= 8) {
        if (gw == 2) return launch_decode_paged_t<D, NS, 2>(a, stream);
    }
    return launch_decode_paged_t<D, NS, 1>(a, stream);
}

template <int D>
hipError_t launch_decode_paged_d(const PagedDecodeArgs &a, int num_splits, hipStream_t stream) {
    if (a.Hq / a.Hkv >= 4)
        return launch_decode_gqa<D>(a, num_splits, stream);
    switch (num_splits) {
    case 1: return launch_decode_paged_g<D, 1>(a, stream);
    case 2: return launch_decode_paged_g<D, 2>(a, stream);
    case 4: return launch_decode_paged_g<D, 4>(a, stream);
    case 8: return launch_decode_paged_g<D, 8>(a, stream);
    default: return launch_decode_paged_g<D, 16>(a, stream);
    }
}

template <int D, int NS>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H));
    const dim3 block(64 * NS);
    DecodeArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_decode_kernel<D, NS>), grid,
                           block, params, 0, stream);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, int num_splits, hipStream_t stream) {
    switch (num_splits) {
    case 1: return launch_decode_t<D, 1>(a, stream);
    case 2: return launch_decode_t<D, 2>(a, stream);
    case 4: return launch_decode_t<D, 4>(a, stream);
    case 8: return launch_decode_t<D, 8>(a, stream);
    default: return launch_decode_t<D, 16>(a, stream);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, int num_splits, hipStream_t stream) {
    return d == 64 ? launch_decode_d<64>(a, num_splits, stream)
                   : launch_decode_d<128>(a, num_splits, stream);
}

hipError_t launch_decode_paged(const PagedDecodeArgs &a, int d, int num_splits,
                               hipStream_t stream) {
    return d == 64 ? launch_decode_paged_d<64>(a, num_splits, stream)
                   : launch_decode_paged_d<128>(a, num_splits, stream);
}

}  // namespace plx
