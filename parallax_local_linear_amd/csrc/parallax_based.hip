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
// the chip inside a segment).  Keys and values stream through LDS in
// super-stages of 128 tokens: one round of loads and barriers per four
// 32-token MFMA stages, loads of the next super-stage in flight meanwhile.
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
constexpr int BS = 32;     // tokens per MFMA stage
constexpr int SUB = 4;     // stages per super-stage (one round of loads and barriers)
constexpr int SST = SUB * BS;
constexpr int KTS = BS + 4;  // padded K^T row (floats): conflict-free 16-byte reads
constexpr int QT = kBasedQueryTile;  // queries per output workgroup
constexpr int QW = 32;     // queries per output wavefront
constexpr int OW = QT / QW;
static_assert(TS % QT == 0 && TS % SST == 0, "segment tiling");

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

// V^T stages in LDS: row r (a value column) holds the stage's 32 positions
// as f16, padded to VTS halves (80 bytes), so the 16-byte fragment reads of
// 16 consecutive rows fall on distinct banks and a thread's 8 column writes
// are one base address plus constant offsets.
constexpr int VTS = BS + 8;

// Feature f as coef * u_a * u_b, where u_16 is 1 (0 for tokens past the
// sequence end, which zeroes every feature of such tokens).
struct FeatAB {
    int a, b;
    float coef;
};
__device__ __forceinline__ FeatAB feat_ab(int f, float scale) {
    FeatAB r;
    if (f < 128) {
        const int delta = f >> 4;
        r.a = f & 15;
        r.b = (r.a + delta) & 15;
        r.coef = delta == 0 ? scale * 0.70710678118654752f : scale;
    } else if (f < 136) {
        r.a = f - 128;
        r.b = r.a + 8;
        r.coef = scale;
    } else if (f < 152) {
        r.a = f - 136;
        r.b = BK;
        r.coef = __builtin_sqrtf(scale);
    } else {
        r.a = r.b = BK;
        r.coef = f == 152 ? 1.f : 0.f;
    }
    return r;
}

// ---------------------------------------------------------------------------
// 1. Segment states.

template <int DV>
struct StateLds {
    float kt[SUB][BK + 1][KTS];             // K^T per stage (+ the ones row), MFMA order
    uint16_t vt[SUB][DV * VTS + 32];        // V^T per stage, f16, padded rows and stages
    u32x4 phi[SUB][NF / 16][64];            // Phi(K) B fragments per stage
};

// Loads of one super-stage (128 tokens) into registers and their stores
// into LDS, shared by the state and output kernels.
//   V: task t < VT (G = t % 4, stage = t / 4 % 4, column chunk m = t / 16)
//      loads the 8 tokens at reduction positions 8G .. 8G+7 of the stage,
//      8 columns each, and writes them transposed as 8 rows of 16 bytes;
//      lanes of a 16-lane phase differ in G and stage, which the 64-byte
//      stage padding puts on distinct banks.
//   K: chunk c < 256 (token c / 2, features 8 (c % 2) ..) by thread c.
// Tokens past L read zeros.
template <int DV>
struct StageIO {
    static constexpr int VT = SUB * 4 * (DV / 8);
    static constexpr int VSTAGE = DV * VTS + 32;
    u32x4 v[8];
    u32x4 k;

    __device__ __forceinline__ void load(const uint16_t *kb, const uint16_t *vb, int64_t k_l,
                                         int64_t v_l, int t0, int L, int tid) {
        if (tid < VT) {
            const int G = tid & 3, sub = (tid >> 2) & 3, m = tid >> 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + sub * BS + pos_tok(8 * G + e);
                v[e] = t < L ? *reinterpret_cast<const u32x4 *>(vb + (int64_t)t * v_l + 8 * m)
                             : (u32x4){0u, 0u, 0u, 0u};
            }
        }
        if (tid < 2 * SST) {
            const int t = t0 + (tid >> 1);
            k = t < L ? *reinterpret_cast<const u32x4 *>(kb + (int64_t)t * k_l + 8 * (tid & 1))
                      : (u32x4){0u, 0u, 0u, 0u};
        }
    }

    // V^T of stage s at vt[s * VSTAGE + col * VTS + pos], f16.
    __device__ __forceinline__ void store_v(uint16_t *vt, int tid) const {
        if (tid >= VT)
            return;
        const int G = tid & 3, sub = (tid >> 2) & 3, m = tid >> 4;
        uint32_t h[8][4];  // [token e][column pair]: f16x2
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                h[e][w] = __builtin_bit_cast(uint32_t, cvt_f16x2(bf16_lo(v[e][w]), bf16_hi(v[e][w])));
        uint16_t *dst = vt + sub * VSTAGE + 8 * m * VTS + 8 * G;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u32x4 out;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const uint32_t lo = h[2 * pp][i / 2], hi = h[2 * pp + 1][i / 2];
                out[pp] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4 *>(dst + i * VTS) = out;
        }
    }
};

template <int DV>
__global__ __launch_bounds__(64 * BCfg<DV>::CB) void parallax_based_state_kernel(BasedArgs a) {
    using C = BCfg<DV>;
    constexpr int NT = 64 * C::CB;
    using IO = StageIO<DV>;
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
    const int n_sst = (min(a.L - t_begin, TS) + SST - 1) / SST;

    IO io;
    f32x4 acc[NF / 16];
#pragma unroll
    for (int fb = 0; fb < NF / 16; ++fb)
        acc[fb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};

    io.load(kb, vb, a.k_l, a.v_l, t_begin, a.L, tid);
    for (int ss = 0; ss < n_sst; ++ss) {
        const int t0 = t_begin + ss * SST;
        __syncthreads();  // the previous super-stage has been read
        io.store_v(&s.vt[0][0], tid);
        if (tid < 2 * SST) {
            const int j = tid >> 1, p = tok_pos(j & (BS - 1));
            float *col = &s.kt[j / BS][8 * (tid & 1)][p];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                col[(2 * e) * KTS] = bf16_lo(io.k[e]);
                col[(2 * e + 1) * KTS] = bf16_hi(io.k[e]);
            }
            if (!(tid & 1))
                s.kt[j / BS][BK][p] = t0 + j < a.L ? 1.f : 0.f;
        }
        __syncthreads();
        if (ss + 1 < n_sst)
            io.load(kb, vb, a.k_l, a.v_l, t0 + SST, a.L, tid);
        // Phi(K) fragments: fragment-lane (stage, fb, l) holds feature
        // 16 fb + l%16 at positions 8 (l/16) .. +7.
        for (int fl = tid; fl < SUB * (NF / 16) * 64; fl += NT) {
            const int sub = fl / ((NF / 16) * 64);
            const int fb = (fl >> 6) % (NF / 16), fl16 = fl & 15, fG = (fl >> 4) & 3;
            const FeatAB fa = feat_ab(16 * fb + fl16, a.scale);
            const float *ra = &s.kt[sub][fa.a][8 * fG];
            const float *rb = &s.kt[sub][fa.b][8 * fG];
            const f32x4 ua0 = *reinterpret_cast<const f32x4 *>(ra);
            const f32x4 ua1 = *reinterpret_cast<const f32x4 *>(ra + 4);
            const f32x4 ub0 = *reinterpret_cast<const f32x4 *>(rb);
            const f32x4 ub1 = *reinterpret_cast<const f32x4 *>(rb + 4);
            f16x8 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[e] = (_Float16)(fa.coef * ua0[e] * ub0[e]);
                out[4 + e] = (_Float16)(fa.coef * ua1[e] * ub1[e]);
            }
            s.phi[sub][fb][fl & 63] = __builtin_bit_cast(u32x4, out);
        }
        __syncthreads();
        // Phi(K)^T times this wavefront's 16 columns of [V | 1], per stage:
        // rows are features, columns value columns.
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            const f16x8 vb16 =
                wave < C::VB ? __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                             &s.vt[sub][(16 * wave + l16) * VTS + 8 * G]))
                             : ones;
#pragma unroll
            for (int fb = 0; fb < NF / 16; ++fb)
                acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(f16x8, s.phi[sub][fb][lane]), vb16, acc[fb], 0, 0, 0);
        }
    }

    // dS [column][feature], fp32: lane holds features 16 fb + 4G .. +3 of
    // column 16 wave + l16.
    float *dst = a.dstate + ((int64_t)bh * a.n_seg + seg) * (NF * C::NC);
#pragma unroll
    for (int fb = 0; fb < NF / 16; ++fb)
        *reinterpret_cast<f32x4 *>(dst + (16 * wave + l16) * NF + 16 * fb + 4 * G) = acc[fb];
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
    // Four segments' loads in flight at a time.
    for (int seg0 = 0; seg0 < a.n_seg; seg0 += 4) {
        float val[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int seg = seg0 + u;
            const float *ds = a.dstate + ((int64_t)bh * a.n_seg + min(seg, a.n_seg - 1)) * (NF * C::NC) +
                              col * NF + f0;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(ds);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(ds + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                val[u][e] = lo[e];
                val[u][4 + e] = hi[e];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int seg = seg0 + u;
            if (seg >= a.n_seg)
                break;
            const int64_t sidx = (int64_t)bh * a.n_seg + seg;
            bf16x8 frag;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                frag[e] = (__bf16)run[e];
            *reinterpret_cast<bf16x8 *>(a.sfrag + ((sidx * C::CB + cb) * NFC + kc) * 512 +
                                        lane * 8) = frag;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                run[e] += val[u][e];
        }
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
    uint16_t k[SST][BK];                    // K of the super-stage, bf16, row-major
    uint16_t vt[SUB][DV * VTS + 32];        // V^T per stage, f16, padded rows and stages
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // The prefix state's fragments of this segment, 1 KiB blocks copied
    // straight into LDS, all in flight at once with the query loads below.
    // Wave w copies blocks w, w + OW, ...; a spare slot copies the last block
    // again (the same bytes to the same place).
    {
        constexpr int NBLK = C::CB * NFC;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(a.sfrag + ((int64_t)bh * a.n_seg + seg) * (NBLK * 512), NBLK * 1024);
#pragma unroll
        for (int c = 0; c < (NBLK + OW - 1) / OW; ++c) {
            const int blk = min(OW * c + wave, NBLK - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)(&s.sfrag[0][0][0] + blk * 64), 16,
                lane * 16, blk * 1024, 0, 0);
        }
    }

    // This wavefront's queries: 16 g + l16 of rows q0 + 32 wave .. +31.
    const int wq0 = q0 + QW * wave;
    u32x4 xq[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int row = min(wq0 + 16 * g + l16, a.L - 1);
        xq[g][0] = *reinterpret_cast<const u32x4 *>(qb + (int64_t)row * a.q_l);
        xq[g][1] = *reinterpret_cast<const u32x4 *>(qb + (int64_t)row * a.q_l + 8);
    }
    f32x4 acc[C::CB][2];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 2; ++g)
            acc[cb][g] = (f32x4){0.f, 0.f, 0.f, 0.f};

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
    __syncthreads();                     // and every other wave's

    // The first key/value super-stage, in flight during the state term.
    using IO = StageIO<DV>;
    IO io;
    io.load(kb, vb, a.k_l, a.v_l, seg_begin, a.L, tid);

    // State term: O^T += S^T Phi(Q)^T (bf16 operands); also the score B
    // fragments (features 4G .. 4G+3 of each query).
    bf16x4 qfrag[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const u32x4 x0 = xq[g][0], x1 = xq[g][1];
        float u[BK];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[2 * e] = bf16_lo(x0[e]);
            u[2 * e + 1] = bf16_hi(x0[e]);
            u[8 + 2 * e] = bf16_lo(x1[e]);
            u[8 + 2 * e + 1] = bf16_hi(x1[e]);
        }
        const uint32_t w0 = (G < 2 ? x0 : x1)[2 * (G & 1)];
        const uint32_t w1 = (G < 2 ? x0 : x1)[2 * (G & 1) + 1];
        qfrag[g] = __builtin_bit_cast(bf16x4, (u32x2){w0, w1});
        PhiQ p;
        phi_setup(p, u, G);
#pragma unroll
        for (int kc = 0; kc < NFC; ++kc) {
            const bf16x8 pf = phi_frag(p, kc, G, a.scale);
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
                acc[cb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, s.sfrag[cb][kc][lane]), pf, acc[cb][g], 0, 0, 0);
            // Keeps one chunk's fragment reads in flight at a time (registers).
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Causal sum over the segment's keys up to this workgroup's last query,
    // in super-stages of 128 keys (4 MFMA stages of 32).
    const int q_last = min(q0 + QT, a.L) - 1;           // last query of the workgroup
    const int n_sst = (q_last - seg_begin) / SST + 1;
    const int w_last = min(wq0 + QW, a.L) - 1;          // last query of the wavefront
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    const float xs = a.scale;
    const float c2 = 0.5f * xs * xs;

    for (int ss = 0; ss < n_sst; ++ss) {
        __syncthreads();  // the previous super-stage has been read
        io.store_v(&s.vt[0][0], tid);
        if (tid < 2 * SST)
            *reinterpret_cast<u32x4 *>(&s.k[tid >> 1][8 * (tid & 1)]) = io.k;
        __syncthreads();
        if (ss + 1 < n_sst)
            io.load(kb, vb, a.k_l, a.v_l, seg_begin + (ss + 1) * SST, a.L, tid);
        // Unrolled: the next stage's fragment reads can overlap this one's products.
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            const int t0 = seg_begin + ss * SST + sub * BS;
            if (t0 > w_last)
                break;  // every later key follows this wavefront's queries
            bf16x4 kf[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                kf[kt] = *reinterpret_cast<const bf16x4 *>(&s.k[sub * BS + 16 * kt + l16][4 * G]);
            f16x8 vf[C::VB];
#pragma unroll
            for (int cb = 0; cb < C::VB; ++cb)
                vf[cb] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                       &s.vt[sub][(16 * cb + l16) * VTS + 8 * G]));
            // Some key may follow some query only where the stage reaches
            // the wavefront's first query; elsewhere the threshold keeps all.
            const bool diag = t0 + BS - 1 > wq0;
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
                    // key t0 + 16 kt + 4G + e is visible iff e <= lim
                    const int lim = diag ? qrow - (t0 + 16 * kt + 4 * G) : 3;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // 1 + x + x^2 / 2 at x = scale s, as (c2 s + scale) s + 1
                        const float wt = __builtin_fmaf(__builtin_fmaf(c2, sc[e], xs), sc[e], 1.f);
                        w[4 * kt + e] = (_Float16)(e <= lim ? wt : 0.f);
                    }
                }
#pragma unroll
                for (int cb = 0; cb < C::VB; ++cb)
                    acc[cb][g] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[cb], w, acc[cb][g], 0, 0, 0);
                acc[C::VB][g] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, w, acc[C::VB][g], 0, 0, 0);
            }
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
    // Thread (fg, cq) owns state columns 4 cq .. 4 cq + 3 of features
    // fg, fg + FGN, ...: 16-byte accesses, all of a thread's loads issued
    // before its stores.
    constexpr int NQ = C::NC / 4;             // column quads
    constexpr int FGN = 4 * C::NC / NQ;       // feature groups (16)
    constexpr int NI = NF / FGN;              // features per thread
    static_assert(C::NC % 4 == 0 && FGN * NQ == 4 * C::NC && NI * FGN == NF, "decode split");
    __shared__ float phq[NF], phk[NF], qv[BK + 1], kv[BK + 1], vv[DV];
    __shared__ float part[FGN][C::NC];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *qr = a.q + (int64_t)bh * BK;
    const uint16_t *kr = a.k + (int64_t)bh * BK;
    const uint16_t *vr = a.v + (int64_t)bh * DV;
    if (tid < BK) {
        qv[tid] = __uint_as_float((uint32_t)qr[tid] << 16);
        kv[tid] = __uint_as_float((uint32_t)kr[tid] << 16);
    } else if (tid == BK) {
        qv[BK] = kv[BK] = 1.f;
    }
    if (tid < DV)
        vv[tid] = __uint_as_float((uint32_t)vr[tid] << 16);
    __syncthreads();
    if (tid < NF) {
        // The prefill feeds bf16 / f16 features to the matrix cores; the
        // decode keeps them in fp32.
        const FeatAB fa = feat_ab(tid, a.scale);
        phq[tid] = fa.coef * qv[fa.a] * qv[fa.b];
        phk[tid] = fa.coef * kv[fa.a] * kv[fa.b];
    }
    __syncthreads();
    const int fg = tid / NQ, cq = tid - fg * NQ;
    float vc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        vc[j] = 4 * cq + j < DV ? vv[4 * cq + j] : 1.f;
    float4 *st = reinterpret_cast<float4 *>(a.state + (int64_t)bh * (NF * C::NC)) + cq;
    float4 sv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
        sv[i] = st[(fg + FGN * i) * NQ];
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int f = fg + FGN * i;
        const float pk = phk[f], pq = phq[f];
        sv[i].x += pk * vc[0];
        sv[i].y += pk * vc[1];
        sv[i].z += pk * vc[2];
        sv[i].w += pk * vc[3];
        st[f * NQ] = sv[i];
        sum[0] += pq * sv[i].x;
        sum[1] += pq * sv[i].y;
        sum[2] += pq * sv[i].z;
        sum[3] += pq * sv[i].w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        part[fg][4 * cq + j] = sum[j];
    __syncthreads();
    if (tid < DV) {
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int g = 0; g < FGN; ++g) {
            num += part[g][tid];
            den += part[g][DV];
        }
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
