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
//   * A workgroup = 8 wavefronts x 16 query rows = 128 rows, one workgroup
//     per CU, two wavefronts per SIMD.  The wavefronts form two groups of
//     four (waves 0-3 and 4-7, one of each on every SIMD) that run half a
//     stage apart ("ping-pong"): while one group issues its matrix-core
//     work, the other does its exponentials and LDS traffic, and a
//     workgroup barrier after every phase swaps the roles.  Each wave
//     alternates
//        M phase: score MFMAs of stage t, value and row-sum MFMAs of stage
//                 t-1 with the LDS reads of stage t+1's K fragments
//                 between them;
//        V phase: LDS reads of the V fragments of stage t, weights of
//                 stage t, and the copy of its group's half of stage t+5
//                 from global memory to LDS.
//   * Keys stream through LDS in stages of 32 keys with six buffers.  The
//     copies go straight from global memory into LDS (buffer loads with
//     the LDS destination, which puts lane i's 16 bytes at 16 i), five
//     stages ahead of use, and each wave waits for its own copies of three
//     stages back at the end of its V phase.  K comes from the K tensor
//     through a buffer resource that ends at the last valid row, so rows
//     past the sequence end arrive as zeros.  V comes from a workspace
//     image that a small first kernel writes once per key: float16,
//     transposed, with the keys of each stage permuted so that one 16-byte
//     LDS read gives each lane the 8 keys the value MFMA needs.
//   * LDS layouts have no padding; an XOR swizzle of the 16-byte chunks of
//     each row (K: chunk ^ row, V^T: chunk ^ (row / 4)) keeps the 16-row
//     fragment reads free of bank conflicts, and the copy of each lane
//     fetches the chunk that belongs to its LDS slot.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_bf16.  In that accumulator layout each lane holds
//     one query row (4 lanes, l ^ 16 and l ^ 32 apart, share a row), so the
//     row max is an in-lane reduction plus two exchanges, and the
//     f16-rounded weights are already in the B-operand layout of
//     O^T = V^T P~^T (v_mfma_f32_16x16x32_f16): no LDS round trip for P.
//   * ell and S come from two more MFMAs of the same f16 weights against an
//     all-ones operand, so A, C, ell and S are sums of the same values, and
//     no VALU time goes to the sums.
//   * Each row's offset m is fixed at its first visible stage (that stage's
//     max + kMargin), so the accumulators are never rescaled inside the
//     loop.  Rows whose scores later exceed m + kTauHi make the workgroup
//     recompute once with the exact row max as offset; weights stay
//     <= 2^kTauHi in the first pass and <= 1 in the second.
//   * Causal, sliding-window and sink masks ("Sliding-window beats linear
//     attention" review, sec. 1) skip whole stages per workgroup.  Stages
//     visible to every row of the workgroup run first and mask-free; the
//     others apply per-element masks.
//   * Workgroups are issued heaviest query tile first; the block index keeps
//     all tiles of one (batch, head) on one XCD when B*H is a multiple of 8,
//     so their K/V reuse stays in that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

constexpr int ROWS = 16;                  // query rows per wavefront
constexpr int NWAVES = 8;                 // two groups of four wavefronts
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BM = ROWS * NWAVES;         // query rows per workgroup
constexpr int BN = 32;                    // keys per stage
constexpr int NBUF = 6;                   // LDS stage buffers
constexpr int AHEAD = 5;                  // stages between a copy and its use
constexpr int IN_FLIGHT = 2;              // stages a wave's copies may still be in flight
// Softmax offsets, log2 units (see above).
constexpr float kMargin = 3.0f;
constexpr float kTauHi = 5.0f;

static_assert(BM == fwd_block_rows(64) && BM == fwd_block_rows(128),
              "host and kernel must agree on the query tile");
static_assert(NBUF >= AHEAD + 1, "a buffer is refilled only after its last read");
static_assert(AHEAD - IN_FLIGHT >= 3, "K of stage t+1 is read in the M phase of stage t");

template <int D>
struct Cfg {
    static constexpr int KC = D / 32;     // reduction chunks of the score MFMA
    static constexpr int DT = D / 16;     // output tiles of the value MFMA
    static constexpr int CPR = D / 8;     // 16-byte chunks per K row
    static constexpr int K_ELEMS = BN * D;
    static constexpr int V_ELEMS = D * BN;
    // 16-byte copies of a half stage (one group's share) of K and of V^T.
    // At d = 128 every wave of the group copies one K and one V^T chunk per
    // lane; at d = 64 the group's first two waves copy K, the others V^T.
    static constexpr int HALF_K = BN / 2 * CPR;
    static constexpr int HALF_V = D / 2 * (BN / 8);
    static constexpr bool SPLIT = HALF_K < 256;
    static constexpr int COPIES = SPLIT ? 1 : 2;  // copy instructions per wave per stage
    static_assert(HALF_K == HALF_V && (HALF_K == 256 || HALF_K == 128), "copy split");
};

// Row swizzle of the K layout: chunk c of row r sits in slot
// r * CPR + (c ^ kswz(r)).  With 256-byte rows (d = 128) every row spans all
// banks, so the 16 rows of a fragment read need 16 distinct chunk
// positions; with 128-byte rows (d = 64) rows r and r+1 share the banks and
// rows of equal parity need 8 distinct positions.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Slot of chunk q (positions 8q .. 8q+7) of V^T row f in a V^T stage: four
// 64-byte rows share the banks, so the chunk index is rotated by f / 4.
__device__ __forceinline__ int vswz_slot(int f, int q) { return 4 * f + (q ^ ((f >> 2) & 3)); }

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

// Exchanges between 16-lane rows done on the VALU (v_permlane16_swap):
// no LDS instruction, so they never wait behind outstanding LDS reads.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reductions over the four lanes that share a query row (l, l^16, l^32, l^48).
__device__ __forceinline__ float row_max4(float x) { return xor32_max(xor16_max(x)); }

// Marks x as needed here: code that computes it cannot be moved past this
// point (neither by IR passes nor by the scheduler), which keeps each
// ping-pong phase's work inside its phase.  The statement only reads x (it
// emits nothing), so the compiler still sees the real producer of x, for
// instance an MFMA, and keeps the wait states later readers need.
template <typename T>
__device__ __forceinline__ void pin(const T &x) {
    asm volatile("" ::"v"(x));
}

// Workgroup barrier between ping-pong phases.  With WAIT_LDS, this wave's
// LDS reads complete first (needed where another wave's next copy reuses
// the buffer just read).  The scheduler may not move anything across it.
// No memory fence: a fence would also wait for the copies into LDS that
// are meant to stay in flight across phases (their completion is waited
// for explicitly, see wait_copies).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
template <bool WAIT_LDS = true>
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (WAIT_LDS)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Waits until at most n of this wave's global -> LDS copies are in flight
// (s_waitcnt vmcnt(n); the LDS and export counters are left alone).
template <int N>
__device__ __forceinline__ void wait_copies() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// Floor and ceiling of a / BN for any sign of a.
__device__ __forceinline__ int floor_div_bn(int a) { return a >= 0 ? a / BN : -((-a + BN - 1) / BN); }
__device__ __forceinline__ int ceil_div_bn(int a) { return -floor_div_bn(-a); }

template <int D>
struct Ctx {
    bf16x8 qf[Cfg<D>::KC], rf[Cfg<D>::KC];
    f32x4 accA[Cfg<D>::DT], accC[Cfg<D>::DT];
    float m_ref;  // this row's softmax offset (scaled log2 units), -inf until set
    float msub;   // m_ref, or 0 while it is unset (all scores so far are -inf)
    float xlane;  // running max of this lane's raw scores of the row
    // Row sums ell and S on the matrix core: (ones x P~^T) puts each row's
    // sum in every element of its column, so element 0 of the lane's
    // accumulator is its row's sum.
    f32x4 accL, accS;
};

// K fragments of one stage (A operand of the score MFMAs): key 16 kt + l16,
// features 32 kc + 8G .. +7.
template <int D>
struct KFrags {
    bf16x8 f[2][Cfg<D>::KC];
};

// V^T fragments of one stage (A operand of the value MFMAs): V^T row
// 16 dt + l16, reduction positions 8G .. 8G+7.
template <int D>
struct VFrags {
    f16x8 f[Cfg<D>::DT];
};

// Scores of one stage: S^T tiles (16 keys x 16 rows) for keys 0-15 and 16-31.
struct Scores {
    f32x4 q[2], r[2];
};

// f16 weights of one stage in the value MFMA's B-operand order: p~ and p~ s.
struct Weights {
    f16x8 p, w;
};

// LDS stage buffer: K [32 keys][d] and V^T [d][32 positions], both in the
// swizzled 16-byte-chunk layouts above.
template <int D>
struct __attribute__((aligned(16))) StageBuf {
    uint16_t k[Cfg<D>::K_ELEMS];
    uint16_t v[Cfg<D>::V_ELEMS];
};

// Compile-time stage buffer number.
template <int I>
using Buf = std::integral_constant<int, I % NBUF>;

// Per-lane byte offsets of the fragment reads inside a K and a V^T stage:
// ka[kc] for key tile 0 (tile 1 is 16 rows further), va for V^T tile 0
// (tile dt is 16 dt rows further).
template <int D>
struct FragAddr {
    uint32_t ka[Cfg<D>::KC];
    uint32_t va;
};

template <int D>
__device__ __forceinline__ FragAddr<D> frag_addr(int l16, int G) {
    using C = Cfg<D>;
    FragAddr<D> f;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
        f.ka[kc] = (uint32_t)(l16 * C::CPR + ((4 * kc + G) ^ kswz<D>(l16))) * 16u;
    f.va = (uint32_t)vswz_slot(l16, G) * 16u;
    return f;
}

template <int D>
__device__ __forceinline__ void read_kfrags(KFrags<D> &kf, const uint16_t *sk,
                                            const FragAddr<D> &fa) {
    const char *base = reinterpret_cast<const char *>(sk);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kc = 0; kc < Cfg<D>::KC; ++kc)
            kf.f[kt][kc] = *reinterpret_cast<const bf16x8 *>(base + fa.ka[kc] +
                                                             kt * 16 * Cfg<D>::CPR * 16);
}

template <int D>
__device__ __forceinline__ void read_vfrags(VFrags<D> &vf, const uint16_t *sv,
                                            const FragAddr<D> &fa) {
    const char *base = reinterpret_cast<const char *>(sv);
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt)
        vf.f[dt] = *reinterpret_cast<const f16x8 *>(base + fa.va + dt * 16 * 4 * 16);
}

// S^T = K Q^T and R K^T for one stage: 2 key tiles x KC chunks x 2 MFMAs,
// four independent accumulation chains, each K fragment shared by the Q and
// the R product.
template <int D>
__device__ __forceinline__ void score_mfmas(const Ctx<D> &cx, const KFrags<D> &kf, Scores &s) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        s.q[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[kt][0], cx.qf[0], z, 0, 0, 0);
        s.r[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[kt][0], cx.rf[0], z, 0, 0, 0);
    }
#pragma unroll
    for (int kc = 1; kc < Cfg<D>::KC; ++kc)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s.q[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[kt][kc], cx.qf[kc], s.q[kt], 0, 0, 0);
            s.r[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[kt][kc], cx.rf[kc], s.r[kt], 0, 0, 0);
        }
}

// O^T += V^T P~^T and V^T (P~ o S)^T for one stage, and the row sums
// ell += sum p~ and S += sum p~ s of the same f16 values.
template <int D>
__device__ __forceinline__ void value_mfmas(Ctx<D> &cx, const VFrags<D> &vf, const Weights &pw) {
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    cx.accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.p, cx.accL, 0, 0, 0);
    cx.accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.w, cx.accS, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt) {
        cx.accA[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.p, cx.accA[dt], 0, 0, 0);
        cx.accC[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.w, cx.accC[dt], 0, 0, 0);
    }
}

// Per-element mask of a stage: invisible scores become -inf.
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

// Sets the softmax offset of rows that have none yet from this stage's row
// max (+ kMargin); rows whose scores so far are all -inf stay unset.
// Returns whether every row of the wavefront now has its offset.
template <int D>
__device__ __forceinline__ bool init_offsets(Ctx<D> &cx, const Scores &s, float c) {
    float mt = fmaxf(fmaxf(fmaxf(s.q[0][0], s.q[0][1]), s.q[0][2]),
                     fmaxf(fmaxf(s.q[0][3], s.q[1][0]), s.q[1][1]));
    mt = fmaxf(fmaxf(mt, s.q[1][2]), s.q[1][3]);
    mt = row_max4(mt);
    cx.m_ref = (cx.m_ref == kNegInf) ? fmaf(mt, c, kMargin) : cx.m_ref;
    cx.msub = (cx.m_ref == kNegInf) ? 0.f : cx.m_ref;
    return __builtin_amdgcn_ballot_w64(cx.m_ref == kNegInf) == 0;
}

// Weights of one stage: the per-lane running max of the raw scores, and the
// f16 weights p~ and p~ s in the value MFMA's B-operand order (p~ s is
// rounded once, from the f32 product).
template <int D>
__device__ __forceinline__ void weights(Ctx<D> &cx, const Scores &s, Weights &pw, float c) {
    cx.xlane = fmaxf(fmaxf(fmaxf(cx.xlane, s.q[0][0]), s.q[0][1]),
                     fmaxf(fmaxf(s.q[0][2], s.q[0][3]), s.q[1][0]));
    cx.xlane = fmaxf(fmaxf(fmaxf(cx.xlane, s.q[1][1]), s.q[1][2]), s.q[1][3]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * e2;
            const float p0 = exp2_fast(fmaf(s.q[kt][e], c, -cx.msub));
            const float p1 = exp2_fast(fmaf(s.q[kt][e + 1], c, -cx.msub));
            const f16x2 ph = cvt_f16x2(p0, p1);
            const f16x2 wh = cvt_f16x2(p0 * s.r[kt][e], p1 * s.r[kt][e + 1]);
            pw.p[4 * kt + e] = ph[0];
            pw.p[4 * kt + e + 1] = ph[1];
            pw.w[4 * kt + e] = wh[0];
            pw.w[4 * kt + e + 1] = wh[1];
        }
    }
}

// Workspace image of the values.  For each 32-key stage (keys 32s .. 32s+31,
// zeros past L) of each (batch, head): float16 values transposed to [d
// features][32 positions], key j at position vt_pos(j), each feature row's
// four 16-byte chunks in the prefill's swizzled LDS slot order, so that the
// prefill moves each stage into LDS with plain 16-byte copies.  The
// conversion and transposition happen once per key instead of once per
// query tile.
//
// A thread owns 8 keys x 8 features: the keys that fill positions 8G ..
// 8G+7 (4G..4G+3 and 16+4G..16+4G+3) and features 8fg .. 8fg+7.  It loads
// the 8 key rows' 16-byte pieces (adjacent fg on adjacent lanes, so each key
// row is read contiguously), converts, transposes the 8 x 8 block in
// registers and stores 8 feature rows' chunk G.  No LDS, no barrier.
template <int D>
__global__ __launch_bounds__(256) void parallax_vprep_kernel(FwdArgs a) {
    constexpr int FG = D / 8;          // feature groups
    constexpr int TPS = 4 * FG;        // threads per stage
    constexpr int SPB = 256 / TPS;     // stages per block
    constexpr int SPW = 64 / TPS;      // stages per wavefront (1 or 2)
    const int li = threadIdx.x % TPS;
    const int G = li / FG;
    const int fg = li % FG;
    const int s = blockIdx.x * SPB + threadIdx.x / TPS;
    // First stage of this wavefront: the buffer resource starts there, so
    // it is uniform and offsets stay small for any row stride.
    const int s_wave = blockIdx.x * SPB + (threadIdx.x / 64) * SPW;
    if (s_wave >= a.n_st)
        return;
    const int j0 = s * BN;
    const int jw = s_wave * BN;
    for (int bh = blockIdx.y; bh < a.B * a.H; bh += gridDim.y) {
        const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
        const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;
        const __amdgpu_buffer_rsrc_t rv =
            make_rsrc(vb + (int64_t)jw * a.v_l, rows_bytes(jw, a.L, a.v_l, D));
        uint32_t hv[8][4];  // [key k][feature pair]: f16x2 bits
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int key = j0 - jw + (k < 4 ? 4 * G + k : 16 + 4 * G + (k - 4));
            const u32x4 x = bufld16(rv, (uint32_t)(key * a.v_l * 2 + 16 * fg));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hv[k][i] = __builtin_bit_cast(uint32_t, cvt_f16x2(bf16_lo(x[i]), bf16_hi(x[i])));
        }
        if (s >= a.n_st)
            continue;
        uint16_t *dst = a.vt + ((int64_t)bh * a.n_st + s) * (D * BN);
#pragma unroll
        for (int cf = 0; cf < 8; ++cf) {
            // Feature 8fg+cf at positions 8G .. 8G+7: half cf%2 of word cf/2
            // of keys k = 0..7.
            u32x4 out;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const uint32_t lo = hv[2 * pp][cf / 2], hi = hv[2 * pp + 1][cf / 2];
                out[pp] = (cf & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                   : ((lo & 0xffffu) | (hi << 16));
            }
            const int f = 8 * fg + cf;
            *reinterpret_cast<u32x4 *>(dst + vswz_slot(f, G) * 8) = out;
        }
    }
}

// WHOLE: the K slice and the V^T images of one (batch, head) each span
// fewer than 2^31 bytes, so one buffer resource per tensor covers every
// stage and a stage needs only an offset; otherwise every stage builds its
// own resources.
template <int D, bool WHOLE, bool STATS>
__global__ __launch_bounds__(NTHREADS, 2) void parallax_fwd_kernel(FwdArgs a) {
    using C = Cfg<D>;
    // One LDS variable per stage buffer, each indexed only by compile-time
    // buffer numbers: the compiler then tells the buffers apart and waits
    // before a fragment read only for the copies into that buffer.
    __shared__ StageBuf<D> sb0, sb1, sb2, sb3, sb4, sb5;
    auto sbuf = [&](auto b) -> StageBuf<D> & {
        if constexpr (std::is_same_v<decltype(b), int>) {
            const int i = b % NBUF;
            return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : i == 3 ? sb3 : i == 4 ? sb4 : sb5;
        } else {
            constexpr int i = decltype(b)::value % NBUF;
            if constexpr (i == 0)
                return sb0;
            else if constexpr (i == 1)
                return sb1;
            else if constexpr (i == 2)
                return sb2;
            else if constexpr (i == 3)
                return sb3;
            else if constexpr (i == 4)
                return sb4;
            else
                return sb5;
        }
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // ping-pong group
    const int wg = wave & 3;    // wave inside the group
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
    const uint16_t *vtb = a.vt + (int64_t)bh * a.n_st * (D * BN);  // this slice's V^T images

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
        cx.msub = 0.f;
        cx.xlane = kNegInf;
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
    // Key offset of stage u of that list.
    auto list_j0 = [&](int u) { return (u < n_ss ? u : st_lo + (u - n_ss)) * BN; };

    // Stages of the window/causal run that every row of the workgroup sees
    // in full: [f_lo, f_hi).  A stage starting at key j0 qualifies when its
    // last key is causal for the first row and inside the sequence
    // (j0 <= jmax) and, with a window, its first key is inside the last
    // row's window (j0 >= jmin).  Sink stages and stages that are full only
    // through the sinks are left to the masked path, which is exact for
    // every stage.
    int f_lo = n, f_hi = n;
    {
        const int jmax = min(i0 - (BN - 1), L - BN);
        const int jmin = window > 0 ? i1 - window + 1 : 0;
        const int lo = n_ss + max(0, ceil_div_bn(jmin) - st_lo);
        const int hi = min(n, n_ss + floor_div_bn(jmax) - st_lo + 1);
        if (jmax >= 0 && lo < hi) {
            f_lo = lo;
            f_hi = hi;
        }
    }
    // Processing order: the full stages first (so that the first stage
    // fixes every row's softmax offset from 32 visible keys and the main
    // loop needs neither masks nor offset logic), then the masked ones.
    const int n_full = f_hi - f_lo;
    auto stage_j0 = [&](int t) {
        const int m = t - n_full;
        return list_j0(t < n_full ? f_lo + t : (m < f_lo ? m : f_hi + (m - f_lo)));
    };

    // Copies of this wave's share of a stage, global -> LDS.  The LDS
    // destination of lane i is slot base + i of the stage (16-byte slots),
    // so each lane fetches the chunk that the swizzled layout puts there.
    // Copies past the last stage reload the last stage (into a buffer
    // nobody reads again), which keeps the loop branch-free.
    const bool k_role = !C::SPLIT || wg < 2;  // d = 64: waves copying K
    const int kslot0 = grp * C::HALF_K + wg * 64;                       // K slots of this wave
    const int vslot0 = grp * C::HALF_V + (C::SPLIT ? wg - 2 : wg) * 64;  // V^T slots of this wave
    uint32_t kgoff;  // byte offset of this lane's K chunk from the stage's first row
    {
        const int s = kslot0 + lane;
        const int r = s / C::CPR;
        const int ch = (s % C::CPR) ^ kswz<D>(r);
        kgoff = (uint32_t)(r * a.k_l * 2 + ch * 16);
    }
    const uint32_t vgoff = (uint32_t)(vslot0 + lane) * 16u;
    constexpr uint32_t kImage = D * BN * 2;  // bytes of one stage's V^T image
    const __amdgpu_buffer_rsrc_t rk_all = make_rsrc(kb, WHOLE ? rows_bytes(0, L, a.k_l, D) : 0u);
    const __amdgpu_buffer_rsrc_t rv_all = make_rsrc(vtb, WHOLE ? (uint32_t)a.n_st * kImage : 0u);
    typedef __attribute__((address_space(3))) void lds_void;
    auto copy = [&](int t, auto buf) __attribute__((always_inline)) {
        const int j0 = __builtin_amdgcn_readfirstlane(stage_j0(min(t, n - 1)));
        const int si = j0 / BN;
        lds_void *kdst = (lds_void *)&sbuf(buf).k[kslot0 * 8];
        lds_void *vdst = (lds_void *)&sbuf(buf).v[vslot0 * 8];
        if constexpr (WHOLE) {
            // Offsets stay below 2^32: the K slice is < 2^31 bytes and a
            // stage reaches at most 31 rows (< 2^30 bytes) past its end; the
            // V^T images of the slice span < 2^31 bytes.
            const uint32_t ko = (uint32_t)j0 * (uint32_t)a.k_l * 2u;
            const uint32_t vo = (uint32_t)si * kImage;
            if (k_role)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk_all, kdst, 16, (int)(kgoff + ko), 0, 0, 0);
            if (!C::SPLIT || !k_role)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv_all, vdst, 16, (int)(vgoff + vo), 0, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc(kb + (int64_t)j0 * a.k_l, rows_bytes(j0, L, a.k_l, D));
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vtb + (int64_t)si * (D * BN), kImage);
            if (k_role)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kdst, 16, (int)kgoff, 0, 0, 0);
            if (!C::SPLIT || !k_role)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, vdst, 16, (int)vgoff, 0, 0, 0);
        }
    };

    const FragAddr<D> fa = frag_addr<D>(l16, G);
    KFrags<D> kf;
    VFrags<D> vf;
    Scores sc;
    Weights pw;

    // End of the M phase, when the score MFMAs are done.  Masked stages: the
    // mask of stage t's scores and the softmax offsets of rows that still
    // have none.  Full stages come first and stage 0 sets every offset, so
    // the other full stages need neither.  `masked` is kFull (0), kMasked (1)
    // or kCausal (2): a causal-only mask (no window; then the sinks are
    // inside the causal span) once every offset is set.
    bool offsets_set = false;  // wave-uniform
    auto finish_scores = [&](auto masked, int t) __attribute__((always_inline)) {
        if constexpr (decltype(masked)::value == 2) {
            const int dlim = min(row, L - 1) - stage_j0(t) - 4 * G;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sc.q[kt][e] = (16 * kt + e <= dlim) ? sc.q[kt][e] : kNegInf;
        } else if constexpr (decltype(masked)::value) {
            mask_scores(sc, stage_j0(t), row, G, L, window, n_sink);
            if (!offsets_set)
                offsets_set = init_offsets<D>(cx, sc, c);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            pin(sc.q[kt]);
            pin(sc.r[kt]);
        }
        pin(cx.msub);
    };
    // M phase of step t (b0 = t % NBUF, always a compile-time constant):
    // the score MFMAs of stage t, then the value MFMAs of stage t-1 with the
    // reads of stage t+1's K fragments between them (the K registers are
    // free once the score MFMAs have issued).  An M-phase wave has idle
    // issue slots between its MFMAs, while a V-phase wave stalls on each
    // LDS read that the busy LDS cannot take yet.
    auto mphase = [&](auto masked, auto b0, int t, bool values) __attribute__((always_inline)) {
        score_mfmas<D>(cx, kf, sc);
        __builtin_amdgcn_sched_barrier(0);
        if (values)
            value_mfmas<D>(cx, vf, pw);
        read_kfrags<D>(kf, sbuf(b0 + 1).k, fa);
#pragma unroll
        for (int i = 0; i < 2 * C::KC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, C::DT / C::KC, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        finish_scores(masked, t);
    };
    // V phase of step t: V fragment reads first, weights, the copy of stage
    // t+5, then the wait for this wave's copies of stage t+3, which the
    // barrier then publishes to both groups before their M phases read its
    // K.  Stage s lives in buffer s % 6 from its copy (step s-5) to its last
    // read (V phase of step s).
    auto vphase = [&](auto b0, int t) __attribute__((always_inline)) {
        read_vfrags<D>(vf, sbuf(b0).v, fa);
        __builtin_amdgcn_sched_barrier(0);
        weights<D>(cx, sc, pw, c);
        pin(pw.p);
        pin(pw.w);
        copy(t + AHEAD, b0 + AHEAD);
        wait_copies<IN_FLIGHT * C::COPIES>();
    };
    // One step: M phase, barrier, V phase, barrier.  The M phase's K reads
    // need no wait at its barrier: they feed this wave's next M phase, and
    // their buffer is refilled two phases after that.  The V phase's reads
    // do: the other group's next copy reuses that buffer.
    auto step = [&](auto masked, auto b0, int t) __attribute__((always_inline)) {
        mphase(masked, b0, t, true);
        phase_barrier<false>();
        vphase(b0, t);
        phase_barrier();
    };
    const std::integral_constant<bool, true> kMasked;
    const std::integral_constant<bool, false> kFull;
    const Buf<0> kB0;
    const Buf<1> kB1;
    const Buf<2> kB2;
    const Buf<3> kB3;
    const Buf<4> kB4;
    const Buf<5> kB5;

    // Pass 0 uses offsets fixed at each row's first visible stage; if any
    // row's scores later rose more than kTauHi above its offset, pass 1
    // recomputes the workgroup with the exact row max as offset.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            cx.accA[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
            cx.accC[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        cx.accL = (f32x4){0.f, 0.f, 0.f, 0.f};
        cx.accS = (f32x4){0.f, 0.f, 0.f, 0.f};

        // Stages 0 .. AHEAD-1 into LDS.
        copy(0, kB0);
        copy(1, kB1);
        copy(2, kB2);
        copy(3, kB3);
        copy(4, kB4);
        wait_copies<0>();
        __syncthreads();
        read_kfrags<D>(kf, sb0.k, fa);
        // The second group starts one phase later.
        if (grp == 1)
            phase_barrier();
        // Step 0 has no value MFMAs; it sets the offsets of all rows that
        // see any of its keys (all rows when it is a full stage).
        if (n_full == 0) {
            mphase(kMasked, kB0, 0, false);
        } else {
            mphase(kFull, kB0, 0, false);
            if (!offsets_set)
                offsets_set = init_offsets<D>(cx, sc, c);
        }
        phase_barrier<false>();
        vphase(kB0, 0);
        phase_barrier();
        // The main loop runs NBUF steps per iteration (t = 1 mod 6), which
        // fixes the LDS buffers of every step.
        int t = 1;
        const int t_mask = max(1, n_full);
        for (; t + 5 < t_mask; t += 6) {
            step(kFull, kB1, t);
            step(kFull, kB2, t + 1);
            step(kFull, kB3, t + 2);
            step(kFull, kB4, t + 3);
            step(kFull, kB5, t + 4);
            step(kFull, kB0, t + 5);
        }
        // Causal tiles whose offsets are all set (the common case): the
        // remaining full stages and the diagonal ones go through a lean
        // causal step, unrolled like the main loop so that every LDS buffer
        // number stays a compile-time constant; the last partial group uses
        // nested guards (a loop with early exits makes the register
        // allocator spill heavily).  Otherwise: steps with a runtime buffer
        // number, before whose LDS reads the compiler waits for every copy
        // in flight.
        if (n_full > 0 && window <= 0) {
            const std::integral_constant<int, 2> kCausal;
            for (; t + 5 < n; t += 6) {
                step(kCausal, kB1, t);
                step(kCausal, kB2, t + 1);
                step(kCausal, kB3, t + 2);
                step(kCausal, kB4, t + 3);
                step(kCausal, kB5, t + 4);
                step(kCausal, kB0, t + 5);
            }
            if (t < n) {
                step(kCausal, kB1, t);
                if (t + 1 < n) {
                    step(kCausal, kB2, t + 1);
                    if (t + 2 < n) {
                        step(kCausal, kB3, t + 2);
                        if (t + 3 < n) {
                            step(kCausal, kB4, t + 3);
                            if (t + 4 < n)
                                step(kCausal, kB5, t + 4);
                        }
                    }
                }
            }
            t = n;
        }
        for (; t < t_mask; ++t)
            step(kFull, t, t);
        for (; t < n; ++t)
            step(kMasked, t, t);
        // Value MFMAs of the last stage; the first group catches up with the
        // second group's extra barrier.
        value_mfmas<D>(cx, vf, pw);
        if (grp == 0)
            phase_barrier();

        const float xmax = row_max4(cx.xlane);
        const bool overflow = pass == 0 && xmax * c > cx.m_ref + kTauHi;
        // Copies still in flight (stages past the end) land before LDS is
        // reused by the next pass.
        wait_copies<0>();
        if (!__syncthreads_or(overflow))
            break;
        // Exact offsets for the recomputation: each row's true max.
        cx.m_ref = xmax * c;
        cx.msub = cx.m_ref == kNegInf ? 0.f : cx.m_ref;
        offsets_set = true;
    }

    // Epilogue.
    const float ell_t = cx.accL[0];
    const float s_t = cx.accS[0];
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
        // Saved for the backward: sbar = S / ell and pv = A / ell.
        if constexpr (STATS) {
            float *pb = a.pv + ((int64_t)bh * L + row) * D;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                f32x4 out;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    out[u] = cx.accA[dt][u] * inv;
                *reinterpret_cast<f32x4 *>(pb + 16 * dt + 4 * G) = out;
            }
            if (G == 0)
                a.sbar[(int64_t)bh * L + row] = s_t * inv;
        }
    }
}

// Bytes from the first element of a [L, d] slice with row stride ld
// (2-byte elements) through its last element.
int64_t slice_bytes(int64_t L, int64_t ld, int d) { return (L - 1) * ld * 2 + (int64_t)d * 2; }

template <int D>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
    FwdArgs args = a;
    void *params[] = {&args};
    constexpr int SPB = 256 / (4 * (D / 8));  // stages per prepass block
    const dim3 pgrid((unsigned)((a.n_st + SPB - 1) / SPB), (unsigned)min(a.B * a.H, 65535));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_vprep_kernel<D>),
                                   pgrid, dim3(256), params, 0, stream);
    if (e != hipSuccess)
        return e;
    const dim3 grid((unsigned)(a.B * a.H * a.n_qtiles));
    const dim3 block(NTHREADS);
    const bool whole = slice_bytes(a.L, a.k_l, D) <= INT32_MAX &&
                       (int64_t)a.n_st * D * BN * 2 <= INT32_MAX;
    const void *fn;
    if (a.pv)
        fn = whole ? reinterpret_cast<const void *>(&parallax_fwd_kernel<D, true, true>)
                   : reinterpret_cast<const void *>(&parallax_fwd_kernel<D, false, true>);
    else
        fn = whole ? reinterpret_cast<const void *>(&parallax_fwd_kernel<D, true, false>)
                   : reinterpret_cast<const void *>(&parallax_fwd_kernel<D, false, false>);
    return hipLaunchKernel(fn, grid, block, params, 0, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int d, hipStream_t stream) {
    return d == 64 ? launch_fwd_t<64>(a, stream) : launch_fwd_t<128>(a, stream);
}

}  // namespace plx
