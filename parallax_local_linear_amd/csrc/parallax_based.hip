// Based linear attention for gfx950 (review page "Simple linear attention
// language models balance the recall-throughput tradeoff", "Proposed
// method": linear attention whose feature dimension sets the size of a fixed
// recurrent state, paired with small-window softmax attention).
//
// The kernel of the linear attention is the second-order Taylor expansion
// of exp, with x = scale * q . k:
//     phi(q) . phi(k) = 1 + x + x^2 / 2
//     o_i = sum_{j <= i} phi(q_i).phi(k_j) v_j / sum_{j <= i} phi(q_i).phi(k_j)
// With 16 query/key features the map has one constant, 16 linear and 136
// quadratic features (the distinct products k_a k_b, a <= b, with weight
// scale / sqrt 2 on the diagonal and scale off it), 153 in all, padded to
// NF = 160.  Feature order (shared by every kernel here and by the state
// layout of the C ABI):
//     f = 16 delta + a  (f < 128):  k_a k_{(a + delta) mod 16}, delta = 0..7
//     f = 128 + a       (a < 8)  :  k_a k_{a + 8}
//     f = 136 + a       (a < 16) :  sqrt(scale) k_a
//     f = 152                    :  1
//     f = 153 .. 159             :  0
//
// Prefill, three kernels (one pass over q, k, v; the state never leaves
// the chip inside a segment):
//   1. parallax_based_state_kernel: per (batch, head, 512-token segment),
//      dS = Phi(K)^T [V | 1] on the matrix cores (f16 operands, fp32 sums).
//      Each 32-token stage puts K^T in LDS, builds the Phi(K) fragments
//      there once, and every wavefront multiplies them with its 16 value
//      columns (the last wavefront's "columns" are all ones: the normaliser).
//   2. parallax_based_scan_kernel: exclusive prefix sums of dS over the
//      segments, written as bf16 matrix-core fragments of S^T for kernel 3,
//      and the final state (fp32) for decoding.
//   3. parallax_based_out_kernel: per 256 queries, O^T = S^T Phi(Q)^T (the
//      state before the segment, Phi(Q) built in registers) plus the causal
//      sum over the segment's earlier keys, O^T += [V | 1]^T W^T with
//      W = 1 + x + x^2/2 computed from transposed scores S^T = K Q^T, as the
//      Parallax prefill does with its softmax weights.  o = numerator /
//      normaliser at the end.
// Decode: parallax_based_decode_kernel adds phi(k)[v | 1]^T to the state and
// reads phi(q) against it, one workgroup per (batch, head).
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

constexpr int BK = 16;     // query/key features
constexpr int NF = 160;    // expanded features (153 used)
constexpr int NFC = 5;     // 32-feature chunks
constexpr int TS = kBasedSegment;  // tokens per segment
constexpr int BS = 32;     // tokens per stage
constexpr int QT = 256;    // queries per output workgroup
constexpr int QW = 32;     // queries per output wavefront
constexpr int OW = QT / QW;
static_assert(TS % QT == 0 && TS % BS == 0, "segment tiling");

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int DV>
struct BCfg {
    static constexpr int VB = DV / 16;    // value column blocks
    static constexpr int CB = VB + 1;     // plus the normaliser block
    static constexpr int NC = 16 * CB;    // state columns
};

// Position of stage token j (0..31) in the reduction order of the
// 16x16x32 MFMAs: lane group G (lane / 16) holds tokens 4G..4G+3 of each
// 16-token score tile, and reads them as positions 8G..8G+7.
__device__ __forceinline__ int tok_pos(int j) {
    return ((j >> 2) & 3) * 8 + (j >> 4) * 4 + (j & 3);
}
// Token at reduction position p (inverse of tok_pos).
__device__ __forceinline__ int pos_tok(int p) {
    return ((p >> 2) & 1) * 16 + (p >> 3) * 4 + (p & 3);
}

// 16-byte slot of chunk g (positions 8g .. 8g+7) of row r in a [rows][32]
// f16 stage: rows 4 apart share banks, so the chunk index is rotated.
__device__ __forceinline__ int vslot(int r, int g) { return 4 * r + (g ^ ((r >> 2) & 3)); }

// Feature f of a 16-vector given by two of its components (u_a, u_b are
// the components the feature reads: see feat_ab).
struct FeatAB {
    int a, b;     // component indices (b unused for linear, both unused for constants)
    int kind;     // 0 product, 1 linear, 2 one, 3 zero
    float coef;
};
__device__ __forceinline__ FeatAB feat_ab(int f, float scale) {
    FeatAB r;
    if (f < 128) {
        const int delta = f >> 4;
        r.a = f & 15;
        r.b = (r.a + delta) & 15;
        r.kind = 0;
        r.coef = delta == 0 ? scale * 0.70710678118654752f : scale;
    } else if (f < 136) {
        r.a = f - 128;
        r.b = r.a + 8;
        r.kind = 0;
        r.coef = scale;
    } else if (f < 152) {
        r.a = r.b = f - 136;
        r.kind = 1;
        r.coef = __builtin_sqrtf(scale);
    } else {
        r.a = r.b = 0;
        r.kind = f == 152 ? 2 : 3;
        r.coef = 0.f;
    }
    return r;
}
__device__ __forceinline__ float feat_val(const FeatAB &fa, float ua, float ub) {
    return fa.kind == 0 ? fa.coef * ua * ub : fa.kind == 1 ? fa.coef * ua : fa.kind == 2 ? 1.f : 0.f;
}

// ---------------------------------------------------------------------------
// 1. Segment states.

template <int DV>
struct StateLds {
    float kt[BK][BS];                       // K^T of the stage, positions in MFMA order
    uint16_t vt[DV * BS];                   // V^T of the stage, f16, vslot layout
    u32x4 phi[NF / 16][64];                 // Phi(K) B fragments of the stage
};

template <int DV>
__global__ __launch_bounds__(64 * BCfg<DV>::CB) void parallax_based_state_kernel(BasedArgs a) {
    using C = BCfg<DV>;
    constexpr int NT = 64 * C::CB;
    __shared__ StateLds<DV> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15, G = lane >> 4;
    const int bh = blockIdx.x / a.n_seg;
    const int seg = blockIdx.x - bh * a.n_seg;
    const int b = bh / a.H, h = bh - b * a.H;
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;
    const int t_begin = seg * TS;
    const int n_st = (min(a.L - t_begin, TS) + BS - 1) / BS;

    // Loads of one stage into registers: K by threads 0..63 (8 features of
    // one token each), V by all threads (8 columns of one token each).
    constexpr int VCH = DV / 8;             // 16-byte chunks per V row
    constexpr int VLOADS = (BS * VCH + NT - 1) / NT;
    u32x4 kreg = {0u, 0u, 0u, 0u};
    u32x4 vreg[VLOADS];
    auto load_stage = [&](int st) __attribute__((always_inline)) {
        const int t0 = t_begin + st * BS;
        if (tid < 2 * BS) {
            const int j = tid >> 1, t = t0 + j;
            kreg = t < a.L ? *reinterpret_cast<const u32x4 *>(kb + (int64_t)t * a.k_l + 8 * (tid & 1))
                           : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < VLOADS; ++u) {
            const int idx = tid + u * NT;
            vreg[u] = (u32x4){0u, 0u, 0u, 0u};
            if (idx < BS * VCH) {
                const int j = idx / VCH, t = t0 + j;
                if (t < a.L)
                    vreg[u] = *reinterpret_cast<const u32x4 *>(vb + (int64_t)t * a.v_l +
                                                               8 * (idx % VCH));
            }
        }
    };
    auto store_stage = [&]() __attribute__((always_inline)) {
        if (tid < 2 * BS) {
            const int j = tid >> 1, p = tok_pos(j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s.kt[8 * (tid & 1) + 2 * e][p] = bf16_lo(kreg[e]);
                s.kt[8 * (tid & 1) + 2 * e + 1][p] = bf16_hi(kreg[e]);
            }
        }
#pragma unroll
        for (int u = 0; u < VLOADS; ++u) {
            const int idx = tid + u * NT;
            if (idx < BS * VCH) {
                const int j = idx / VCH, c0 = 8 * (idx % VCH), p = tok_pos(j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f16x2 hv = cvt_f16x2(bf16_lo(vreg[u][e]), bf16_hi(vreg[u][e]));
                    s.vt[vslot(c0 + 2 * e, p >> 3) * 8 + (p & 7)] =
                        __builtin_bit_cast(uint32_t, hv) & 0xffffu;
                    s.vt[vslot(c0 + 2 * e + 1, p >> 3) * 8 + (p & 7)] =
                        __builtin_bit_cast(uint32_t, hv) >> 16;
                }
            }
        }
    };

    f32x4 acc[NF / 16];
#pragma unroll
    for (int fb = 0; fb < NF / 16; ++fb)
        acc[fb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};

    load_stage(0);
    for (int st = 0; st < n_st; ++st) {
        __syncthreads();  // the previous stage's fragments have been read
        store_stage();
        __syncthreads();
        if (st + 1 < n_st)
            load_stage(st + 1);
        // Phi(K) fragments: fragment-lane (fb, l) holds feature 16 fb + l%16
        // at positions 8 (l/16) .. +7; tokens past L get zeros.
        const int t0 = t_begin + st * BS;
        for (int fl = tid; fl < (NF / 16) * 64; fl += NT) {
            const int fb = fl >> 6, fl16 = fl & 15, fG = (fl >> 4) & 3;
            const FeatAB fa = feat_ab(16 * fb + fl16, a.scale);
            const f32x4 ua0 = *reinterpret_cast<const f32x4 *>(&s.kt[fa.a][8 * fG]);
            const f32x4 ua1 = *reinterpret_cast<const f32x4 *>(&s.kt[fa.a][8 * fG + 4]);
            const f32x4 ub0 = *reinterpret_cast<const f32x4 *>(&s.kt[fa.b][8 * fG]);
            const f32x4 ub1 = *reinterpret_cast<const f32x4 *>(&s.kt[fa.b][8 * fG + 4]);
            f16x8 out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ua = e < 4 ? ua0[e] : ua1[e - 4];
                const float ub = e < 4 ? ub0[e] : ub1[e - 4];
                const bool live = t0 + pos_tok(8 * fG + e) < a.L;
                out[e] = (_Float16)(live ? feat_val(fa, ua, ub) : 0.f);
            }
            s.phi[fb][fl & 63] = __builtin_bit_cast(u32x4, out);
        }
        __syncthreads();
        // This wavefront's 16 columns of [V | 1]^T times Phi(K).
        const f16x8 va = wave < C::VB
                             ? __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                              &s.vt[vslot(16 * wave + l16, G) * 8]))
                             : ones;
#pragma unroll
        for (int fb = 0; fb < NF / 16; ++fb)
            acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                va, __builtin_bit_cast(f16x8, s.phi[fb][lane]), acc[fb], 0, 0, 0);
    }

    // dS [feature][column], fp32: lane holds columns 16 wave + 4G .. +3 of
    // feature 16 fb + l16.
    float *dst = a.dstate + ((int64_t)bh * a.n_seg + seg) * (NF * C::NC);
#pragma unroll
    for (int fb = 0; fb < NF / 16; ++fb)
        *reinterpret_cast<f32x4 *>(dst + (16 * fb + l16) * C::NC + 16 * wave + 4 * G) = acc[fb];
}

// ---------------------------------------------------------------------------
// 2. Exclusive prefix over segments.  Thread (bh, cb, kc, lane) owns the 8
// state entries of one S^T fragment lane: column 16 cb + l16, features
// 32 kc + 8G .. +7.

template <int DV>
__global__ __launch_bounds__(256) void parallax_based_scan_kernel(BasedArgs a) {
    using C = BCfg<DV>;
    constexpr int PER_BH = C::CB * NFC * 64;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)a.B * a.H * PER_BH)
        return;
    const int bh = (int)(gid / PER_BH);
    const int r = (int)(gid - (int64_t)bh * PER_BH);
    const int cb = r / (NFC * 64), kc = (r / 64) % NFC, lane = r & 63;
    const int col = 16 * cb + (lane & 15);
    const int f0 = 32 * kc + 8 * (lane >> 4);
    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < a.n_seg; ++seg) {
        const int64_t sidx = (int64_t)bh * a.n_seg + seg;
        bf16x8 frag;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            frag[e] = (__bf16)run[e];
        *reinterpret_cast<bf16x8 *>(a.sfrag + ((sidx * C::CB + cb) * NFC + kc) * 512 + lane * 8) =
            frag;
        const float *ds = a.dstate + sidx * (NF * C::NC);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            run[e] += ds[(f0 + e) * C::NC + col];
    }
    if (a.state) {
        float *st = a.state + (int64_t)bh * (NF * C::NC);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            st[(f0 + e) * C::NC + col] = run[e];
    }
}

// ---------------------------------------------------------------------------
// 3. Outputs.

template <int DV>
struct OutLds {
    u32x4 sfrag[BCfg<DV>::CB][NFC][64];     // S^T fragments (bf16) of the segment's prefix
    uint16_t k[BS][BK];                     // K of the stage, bf16, row-major
    uint16_t vt[DV * BS];                   // V^T of the stage, f16, vslot layout
};

// Phi(q)^T B fragment kc for the query whose 16 features are u[]: lane
// group G holds features 32 kc + 8G .. +7.  The component indices depend on
// G only through the rotations built in phi_setup, so all register indices
// are compile-time.
struct PhiQ {
    float ua[8];    // u[8 (G & 1) + i]
    float ub[16];   // u[(8 (G & 1) + (G >> 1) + j) mod 16]
    float lo[8], hi8[8];  // u[i], u[8 + i]
};

__device__ __forceinline__ void phi_setup(PhiQ &p, const float (&u)[BK], int G) {
    const bool odd = G & 1, up = G >> 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p.lo[i] = u[i];
        p.hi8[i] = u[8 + i];
        p.ua[i] = odd ? u[8 + i] : u[i];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float r0 = u[j & 15], r1 = u[(j + 1) & 15], r8 = u[(j + 8) & 15],
                    r9 = u[(j + 9) & 15];
        p.ub[j] = odd ? (up ? r9 : r8) : (up ? r1 : r0);
    }
}

__device__ __forceinline__ bf16x8 phi_frag(const PhiQ &p, int kc, int G, float scale) {
    bf16x8 out;
    if (kc < 4) {
        // delta = 2 kc + (G >> 1), a = 8 (G & 1) + i, b = (a + delta) mod 16
        const float c0 = (kc == 0 && G < 2) ? scale * 0.70710678118654752f : scale;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i] = (__bf16)(c0 * p.ua[i] * p.ub[(i + 2 * kc) & 15]);
    } else {
        const float sq = __builtin_sqrtf(scale);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v0 = scale * p.lo[i] * p.hi8[i];       // f = 128 + i
            const float v1 = sq * p.lo[i];                     // f = 136 + i
            const float v2 = sq * p.hi8[i];                    // f = 144 + i
            const float v3 = i == 0 ? 1.f : 0.f;               // f = 152 + i
            out[i] = (__bf16)(G == 0 ? v0 : G == 1 ? v1 : G == 2 ? v2 : v3);
        }
    }
    return out;
}

template <int DV>
__global__ __launch_bounds__(64 * OW) void parallax_based_out_kernel(BasedArgs a) {
    using C = BCfg<DV>;
    constexpr int NT = 64 * OW;
    __shared__ OutLds<DV> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15, G = lane >> 4;
    const int bh = blockIdx.x / a.n_qt;
    const int qt = blockIdx.x - bh * a.n_qt;
    const int b = bh / a.H, h = bh - b * a.H;
    const int q0 = qt * QT;
    const int seg = q0 / TS;
    const int seg_begin = seg * TS;
    const uint16_t *qb = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h;
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;

    // The prefix state's fragments of this segment into LDS.
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(
            a.sfrag + ((int64_t)bh * a.n_seg + seg) * (C::CB * NFC * 512));
        u32x4 *dst = &s.sfrag[0][0][0];
        for (int i = tid; i < C::CB * NFC * 64; i += NT)
            dst[i] = src[i];
    }

    // This wavefront's queries: 16 g + l16 of rows q0 + 32 wave .. +31.
    const int wq0 = q0 + QW * wave;
    float u[2][BK];
    bf16x4 qfrag[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int row = min(wq0 + 16 * g + l16, a.L - 1);
        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(qb + (int64_t)row * a.q_l);
        const u32x4 x1 = *reinterpret_cast<const u32x4 *>(qb + (int64_t)row * a.q_l + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[g][2 * e] = bf16_lo(x0[e]);
            u[g][2 * e + 1] = bf16_hi(x0[e]);
            u[g][8 + 2 * e] = bf16_lo(x1[e]);
            u[g][8 + 2 * e + 1] = bf16_hi(x1[e]);
        }
        // Score B fragment: features 4G .. 4G+3 of the query.
        const uint32_t w0 = (G < 2 ? x0 : x1)[2 * (G & 1)];
        const uint32_t w1 = (G < 2 ? x0 : x1)[2 * (G & 1) + 1];
        qfrag[g] = __builtin_bit_cast(bf16x4, (u32x2){w0, w1});
    }

    f32x4 acc[C::CB][2];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 2; ++g)
            acc[cb][g] = (f32x4){0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // state fragments in LDS

    // State term: O^T += S^T Phi(Q)^T (bf16 operands).
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        PhiQ p;
        phi_setup(p, u[g], G);
#pragma unroll
        for (int kc = 0; kc < NFC; ++kc) {
            const bf16x8 pf = phi_frag(p, kc, G, a.scale);
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
                acc[cb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, s.sfrag[cb][kc][lane]), pf, acc[cb][g], 0, 0, 0);
        }
    }

    // Causal sum over the segment's keys up to this workgroup's last query.
    constexpr int VCH = DV / 8;
    constexpr int VLOADS = (BS * VCH + NT - 1) / NT;
    u32x4 kreg = {0u, 0u, 0u, 0u};
    u32x4 vreg[VLOADS];
    auto load_stage = [&](int st) __attribute__((always_inline)) {
        const int t0 = seg_begin + st * BS;
        if (tid < 2 * BS) {
            const int t = t0 + (tid >> 1);
            kreg = t < a.L ? *reinterpret_cast<const u32x4 *>(kb + (int64_t)t * a.k_l + 8 * (tid & 1))
                           : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int w = 0; w < VLOADS; ++w) {
            const int idx = tid + w * NT;
            vreg[w] = (u32x4){0u, 0u, 0u, 0u};
            if (idx < BS * VCH) {
                const int t = t0 + idx / VCH;
                if (t < a.L)
                    vreg[w] = *reinterpret_cast<const u32x4 *>(vb + (int64_t)t * a.v_l +
                                                               8 * (idx % VCH));
            }
        }
    };
    auto store_stage = [&]() __attribute__((always_inline)) {
        if (tid < 2 * BS)
            *reinterpret_cast<u32x4 *>(&s.k[tid >> 1][8 * (tid & 1)]) = kreg;
#pragma unroll
        for (int w = 0; w < VLOADS; ++w) {
            const int idx = tid + w * NT;
            if (idx < BS * VCH) {
                const int j = idx / VCH, c0 = 8 * (idx % VCH), p = tok_pos(j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f16x2 hv = cvt_f16x2(bf16_lo(vreg[w][e]), bf16_hi(vreg[w][e]));
                    s.vt[vslot(c0 + 2 * e, p >> 3) * 8 + (p & 7)] =
                        __builtin_bit_cast(uint32_t, hv) & 0xffffu;
                    s.vt[vslot(c0 + 2 * e + 1, p >> 3) * 8 + (p & 7)] =
                        __builtin_bit_cast(uint32_t, hv) >> 16;
                }
            }
        }
    };

    const int q_last = min(q0 + QT, a.L) - 1;           // last query of the workgroup
    const int n_st = (q_last - seg_begin) / BS + 1;
    const int w_last = min(wq0 + QW, a.L) - 1;          // last query of the wavefront
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    const float xs = a.scale;

    load_stage(0);
    for (int st = 0; st < n_st; ++st) {
        __syncthreads();  // the previous stage has been read
        store_stage();
        __syncthreads();
        if (st + 1 < n_st)
            load_stage(st + 1);
        const int t0 = seg_begin + st * BS;
        if (t0 > w_last)
            continue;  // every key of this stage is after this wavefront's queries
        bf16x4 kf[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
            kf[kt] = *reinterpret_cast<const bf16x4 *>(&s.k[16 * kt + l16][4 * G]);
        f16x8 vf[C::VB];
#pragma unroll
        for (int cb = 0; cb < C::VB; ++cb)
            vf[cb] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                   &s.vt[vslot(16 * cb + l16, G) * 8]));
        const bool diag = t0 + BS - 1 > wq0;  // some key may follow some query
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            // S^T tile kt: lane holds keys t0 + 16 kt + 4G + e of query
            // wq0 + 16 g + l16.
            const int qrow = wq0 + 16 * g + l16;
            f16x8 w;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const f32x4 sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(s16x4, kf[kt]), __builtin_bit_cast(s16x4, qfrag[g]),
                    (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = xs * sc[e];
                    float wt = __builtin_fmaf(0.5f * x, x, x + 1.f);
                    if (diag && t0 + 16 * kt + 4 * G + e > qrow)
                        wt = 0.f;
                    w[4 * kt + e] = (_Float16)wt;
                }
            }
#pragma unroll
            for (int cb = 0; cb < C::VB; ++cb)
                acc[cb][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[cb], w, acc[cb][g], 0, 0, 0);
            acc[C::VB][g] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, w, acc[C::VB][g], 0, 0, 0);
        }
    }

    // o = numerator / normaliser: lane holds columns 16 cb + 4G .. +3 of
    // query wq0 + 16 g + l16; every element of the normaliser block is the
    // query's normaliser.
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int row = wq0 + 16 * g + l16;
        if (row >= a.L)
            continue;
        const float inv = 1.0f / acc[C::VB][g][0];
        float *orow = a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)row * a.o_l;
#pragma unroll
        for (int cb = 0; cb < C::VB; ++cb) {
            f32x4 r = acc[cb][g];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] *= inv;
            *reinterpret_cast<f32x4 *>(orow + 16 * cb + 4 * G) = r;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: one token per (batch, head).  Thread (fg, c) handles column c of
// features fg, fg + 4, ...: it adds phi_f(k) [v | 1]_c to the state and sums
// phi_f(q) S_fc; the four partial sums of a column meet in LDS.

template <int DV>
__global__ __launch_bounds__(4 * BCfg<DV>::NC) void parallax_based_decode_kernel(BasedArgs a) {
    using C = BCfg<DV>;
    __shared__ float phq[NF], phk[NF], qv[BK], kv[BK], vv[DV];
    __shared__ float part[4][C::NC];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *qr = a.q + (int64_t)bh * BK;
    const uint16_t *kr = a.k + (int64_t)bh * BK;
    const uint16_t *vr = a.v + (int64_t)bh * DV;
    if (tid < BK) {
        qv[tid] = __uint_as_float((uint32_t)qr[tid] << 16);
        kv[tid] = __uint_as_float((uint32_t)kr[tid] << 16);
    }
    if (tid < DV)
        vv[tid] = __uint_as_float((uint32_t)vr[tid] << 16);
    __syncthreads();
    if (tid < NF) {
        const FeatAB fa = feat_ab(tid, a.scale);
        // The prefill feeds bf16 / f16 features to the matrix cores; the
        // decode keeps them in fp32.
        phq[tid] = feat_val(fa, qv[fa.a], qv[fa.b]);
        phk[tid] = feat_val(fa, kv[fa.a], kv[fa.b]);
    }
    __syncthreads();
    const int fg = tid / C::NC, c = tid - fg * C::NC;
    const float vc = c < DV ? vv[c] : 1.f;
    float *st = a.state + (int64_t)bh * (NF * C::NC) + c;
    float sum = 0.f;
    for (int f = fg; f < NF; f += 4) {
        const float sv = st[f * C::NC] + phk[f] * vc;
        st[f * C::NC] = sv;
        sum += phq[f] * sv;
    }
    part[fg][c] = sum;
    __syncthreads();
    if (tid < DV) {
        const float num = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
        const float den = part[0][DV] + part[1][DV] + part[2][DV] + part[3][DV];
        a.o[(int64_t)bh * DV + tid] = num / den;
    }
}

template <int DV>
hipError_t launch_based_fwd_t(const BasedArgs &a, hipStream_t stream) {
    BasedArgs args = a;
    void *params[] = {&args};
    using C = BCfg<DV>;
    const unsigned bhn = (unsigned)(a.B * a.H);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_based_state_kernel<DV>),
                                   dim3(bhn * a.n_seg), dim3(64 * C::CB), params, 0, stream);
    if (e != hipSuccess)
        return e;
    const int64_t scan_threads = (int64_t)bhn * C::CB * NFC * 64;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_based_scan_kernel<DV>),
                        dim3((unsigned)((scan_threads + 255) / 256)), dim3(256), params, 0, stream);
    if (e != hipSuccess)
        return e;
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_based_out_kernel<DV>),
                           dim3(bhn * a.n_qt), dim3(64 * OW), params, 0, stream);
}

template <int DV>
hipError_t launch_based_decode_t(const BasedArgs &a, hipStream_t stream) {
    BasedArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_based_decode_kernel<DV>),
                           dim3((unsigned)(a.B * a.H)), dim3(4 * BCfg<DV>::NC), params, 0, stream);
}

}  // namespace

size_t based_state_floats(int dv) { return (size_t)NF * 16 * (dv / 16 + 1); }

size_t based_workspace_bytes(int64_t B, int64_t H, int64_t L, int dv) {
    const int64_t n_seg = (L + TS - 1) / TS;
    const size_t per_seg = based_state_floats(dv) * 4 + (size_t)(dv / 16 + 1) * NFC * 512 * 2;
    return (size_t)(B * H * n_seg) * per_seg;
}

hipError_t launch_based_fwd(const BasedArgs &a, int dv, hipStream_t stream) {
    return dv == 64 ? launch_based_fwd_t<64>(a, stream) : launch_based_fwd_t<128>(a, stream);
}

hipError_t launch_based_decode(const BasedArgs &a, int dv, hipStream_t stream) {
    return dv == 64 ? launch_based_decode_t<64>(a, stream) : launch_based_decode_t<128>(a, stream);
}

}  // namespace plx
