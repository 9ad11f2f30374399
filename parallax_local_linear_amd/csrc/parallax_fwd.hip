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
//   * Keys stream through LDS in stages of 32 keys (64 at d = 64: two
//     32-key halves, so that a step carries about the same matrix-core
//     work per barrier at either d) with six buffers.  The copies go
//     straight from global memory into LDS (buffer loads with the LDS
//     destination, which puts lane i's 16 bytes at 16 i), five
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

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace plx {

// The prefill's workspace for callers that cannot allocate: a file-scope
// device array, one copy per GPU, kept until the process ends.  Host code
// never uses its name as an address (on the host it is only a stand-in for
// the symbol): fwd_scratch() looks up each device's address once, with that
// device current, and every launch takes that address.
static __device__ __align__(256) unsigned char scratch[kFwdScratchBytes];

hipError_t fwd_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

constexpr int ROWS = 16;                  // query rows per wavefront
constexpr int NWAVES = 8;                 // two groups of four wavefronts
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BM = ROWS * NWAVES;         // query rows per workgroup
constexpr int BN = 32;                    // keys per half stage (one V^T image, a score tile pair)
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
    // Keys per stage of the main kernel: 32 at d = 128, 64 at d = 64 (two
    // 32-key halves), so that a stage is 16 KB of K and V^T at either d and
    // a step at d = 64 carries as many score MFMAs as at d = 128 against
    // the same per-step costs (barriers, waits, copy issue, latencies).
    static constexpr int NVH = D == 64 ? 2 : 1;  // 32-key halves per stage
    static constexpr int SBN = BN * NVH;
    // 16-byte copies of a half stage (one group's share) of K and of V^T:
    // every wave of the group copies one K and one V^T chunk per lane.
    static constexpr int HALF_K = SBN / 2 * CPR;
    static constexpr int HALF_V = D / 2 * (SBN / 8);
    static constexpr int COPIES = 2;  // copy instructions per wave per stage
    static_assert(HALF_K == 256 && HALF_V == 256, "one K and one V^T chunk per lane");
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

// Stores a wavefront's 16 output rows non-temporally (no later work in the
// call reads them), each store instruction writing whole 128-byte lines.
// Lane (l16, G) holds features 16 dt + 4G .. +3 of row l16 in out[dt]; lanes
// l and l ^ 8 trade one 16-byte piece per pair of feature tiles, so that the
// first instruction of a pair writes rows 0-7 and the second rows 8-15, each
// row's 32 features by 8 lanes.  (Written from the accumulator layout, each
// instruction would write half of every row's lines, and non-temporal
// stores of half lines are not merged in L2.)  The outputs are
// o = (A keep + C) inv from the accumulators, formed a pair of tiles at a
// time.  Rows at or past `L` are not stored; o0 is row i0 of the wavefront,
// ld the row stride in elements.
template <int DT>
__device__ __forceinline__ void store_rows_nt(float *o0, int64_t ld, int i0, int L, int l16,
                                              int G, const f32x4 (&accA)[DT],
                                              const f32x4 (&accC)[DT], float keep, float inv) {
    static_assert(DT % 2 == 0, "pairs of feature tiles");
    const bool lo = l16 < 8;
    const int ra = lo ? l16 : l16 - 8;  // row of the first instruction of a pair
    const int rb = ra + 8;              // row of the second
    const int seg = (lo ? 0 : 4) + G;   // 16-byte piece of the row's 128-byte line
#pragma unroll
    for (int p = 0; p < DT / 2; ++p) {
        f32x4 out[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                out[q][u] = (accA[2 * p + q][u] * keep + accC[2 * p + q][u]) * inv;
        const f32x4 send = lo ? out[1] : out[0];
        f32x4 recv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            recv[i] = __shfl_xor(send[i], 8, 64);
        const f32x4 va = lo ? out[0] : recv;
        const f32x4 vb = lo ? recv : out[1];
        if (i0 + ra < L)
            __builtin_nontemporal_store(va, reinterpret_cast<f32x4 *>(o0 + ra * ld + 32 * p + 4 * seg));
        if (i0 + rb < L)
            __builtin_nontemporal_store(vb, reinterpret_cast<f32x4 *>(o0 + rb * ld + 32 * p + 4 * seg));
    }
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

// Floor and ceiling of a / S for any sign of a.
template <int S>
__device__ __forceinline__ int floor_div(int a) { return a >= 0 ? a / S : -((-a + S - 1) / S); }
template <int S>
__device__ __forceinline__ int ceil_div(int a) { return -floor_div<S>(-a); }

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
// PRECISE adds their rounding residuals, p~ - f16(p~) and p~ s - f16(p~ s),
// rounded to f16 again: each weight then reaches the matrix core as the sum
// of two f16 values (about 22 significant bits instead of 11).
template <bool PRECISE>
struct Weights {
    f16x8 p, w;
};
template <>
struct Weights<true> {
    f16x8 p, w, plo, wlo;
};

// LDS stage buffer of SK keys: K [SK keys][d] and V^T as SK / 32 images of
// [d][32 positions] (one per 32-key half), both in the swizzled
// 16-byte-chunk layouts above.
template <int D, int SK = BN>
struct __attribute__((aligned(16))) StageBuf {
    uint16_t k[SK * D];
    uint16_t v[D * SK];
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
// ell += sum p~ and S += sum p~ s of the same f16 values (with PRECISE, the
// residual parts go into the same accumulators).
template <int D, bool PRECISE>
__device__ __forceinline__ void value_mfmas(Ctx<D> &cx, const VFrags<D> &vf,
                                            const Weights<PRECISE> &pw) {
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    cx.accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.p, cx.accL, 0, 0, 0);
    cx.accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.w, cx.accS, 0, 0, 0);
    if constexpr (PRECISE) {
        cx.accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.plo, cx.accL, 0, 0, 0);
        cx.accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw.wlo, cx.accS, 0, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt) {
        cx.accA[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.p, cx.accA[dt], 0, 0, 0);
        cx.accC[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.w, cx.accC[dt], 0, 0, 0);
        if constexpr (PRECISE) {
            cx.accA[dt] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.plo, cx.accA[dt], 0, 0, 0);
            cx.accC[dt] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f[dt], pw.wlo, cx.accC[dt], 0, 0, 0);
        }
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

// Mask of a stage by a per-lane range of key offsets: element (kt, e), key
// j0 + 4G + 16 kt + e, stays visible iff lo <= 16 kt + e <= hi.
__device__ __forceinline__ void mask_range(Scores &s, int lo, int hi) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s.q[kt][e] = (16 * kt + e >= lo && 16 * kt + e <= hi) ? s.q[kt][e] : kNegInf;
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
// rounded once, from the f32 product; with PRECISE, also the f16 residuals).
template <int D, bool PRECISE>
__device__ __forceinline__ void weights(Ctx<D> &cx, const Scores &s, Weights<PRECISE> &pw,
                                        float c) {
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
            pw.p[4 * kt + e] = ph[0];
            pw.p[4 * kt + e + 1] = ph[1];
            if constexpr (PRECISE) {
                // The residuals are exact in f32 (the f16 values carry 11 of
                // the 24 significant bits), then rounded to f16.
                const float w0 = p0 * s.r[kt][e];
                const float w1 = p1 * s.r[kt][e + 1];
                const f16x2 wh = cvt_f16x2(w0, w1);
                const f16x2 pl = cvt_f16x2(p0 - (float)ph[0], p1 - (float)ph[1]);
                const f16x2 wl = cvt_f16x2(w0 - (float)wh[0], w1 - (float)wh[1]);
                pw.w[4 * kt + e] = wh[0];
                pw.w[4 * kt + e + 1] = wh[1];
                pw.plo[4 * kt + e] = pl[0];
                pw.plo[4 * kt + e + 1] = pl[1];
                pw.wlo[4 * kt + e] = wl[0];
                pw.wlo[4 * kt + e + 1] = wl[1];
            } else {
                const f16x2 wh = cvt_f16x2(p0 * s.r[kt][e], p1 * s.r[kt][e + 1]);
                pw.w[4 * kt + e] = wh[0];
                pw.w[4 * kt + e + 1] = wh[1];
            }
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
    // The main kernel, which runs after this one, counts recomputed tiles.
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        a.counters[0] = 0u;
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
        u32x4 out[8];
#pragma unroll
        for (int cf = 0; cf < 8; ++cf) {
            // Feature 8fg+cf at positions 8G .. 8G+7: half cf%2 of word cf/2
            // of keys k = 0..7.
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const uint32_t lo = hv[2 * pp][cf / 2], hi = hv[2 * pp + 1][cf / 2];
                out[cf][pp] = (cf & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                       : ((lo & 0xffffu) | (hi << 16));
            }
        }
        // Feature rows 2m and 2m+1 (64 bytes each) share a 128-byte line.
        // Lanes fg and fg ^ 1 (adjacent lanes) trade one chunk per row pair,
        // so that each store instruction writes whole lines: the first of a
        // pair writes rows 8F + c and 8F + c + 1 of even F (lane F its own
        // row, lane F + 1 the one it received), the second those of odd F.
        const int e = fg & 1;
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
            const u32x4 send = e ? out[c] : out[c + 1];
            u32x4 recv;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                recv[i] = (uint32_t)__shfl_xor((int)send[i], 1, 64);
            const int fa = e ? 8 * (fg - 1) + c + 1 : 8 * fg + c;
            const int fb = e ? 8 * fg + c + 1 : 8 * (fg + 1) + c;
            *reinterpret_cast<u32x4 *>(dst + vswz_slot(fa, G) * 8) = e ? recv : out[c];
            *reinterpret_cast<u32x4 *>(dst + vswz_slot(fb, G) * 8) = e ? out[c + 1] : recv;
        }
    }
}

// WHOLE: the K slice and the V^T images of one (batch, head) each span
// fewer than 2^31 bytes, so one buffer resource per tensor covers every
// stage and a stage needs only an offset; otherwise every stage builds its
// own resources.  STATS: also store sbar and pv for the backward.
// PRECISE: weights as two f16 parts each (see Weights).
template <int D, bool WHOLE, bool STATS, bool PRECISE>
__global__ __launch_bounds__(NTHREADS, 2) void parallax_fwd_kernel(FwdArgs a) {
    using C = Cfg<D>;
    constexpr int NVH = C::NVH;  // 32-key halves per stage
    constexpr int SBN = C::SBN;  // keys per stage
    using SBuf = StageBuf<D, SBN>;
    // One LDS variable per stage buffer, each indexed only by compile-time
    // buffer numbers: the compiler then tells the buffers apart and waits
    // before a fragment read only for the copies into that buffer.
    __shared__ SBuf sb0, sb1, sb2, sb3, sb4, sb5;
    auto sbuf = [&](auto b) -> SBuf & {
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
    const int st_hi = i1 / SBN;
    int st_lo = 0, n_ss = 0;
    if (window > 0) {
        const int lo = i0 - window + 1;
        st_lo = lo > 0 ? lo / SBN : 0;
        n_ss = min((n_sink + SBN - 1) / SBN, st_lo);
    }
    const int n = n_ss + (st_hi - st_lo + 1);
    // Key offset of stage u of that list.
    auto list_j0 = [&](int u) { return (u < n_ss ? u : st_lo + (u - n_ss)) * SBN; };

    // Stages of the window/causal run that every row of the workgroup sees
    // in full: [f_lo, f_hi).  A stage starting at key j0 qualifies when its
    // last key is causal for the first row and inside the sequence
    // (j0 <= jmax) and, with a window, its first key is inside the last
    // row's window (j0 >= jmin).  Sink stages and stages that are full only
    // through the sinks are left to the masked path, which is exact for
    // every stage.
    int f_lo = n, f_hi = n;
    {
        const int jmax = min(i0 - (SBN - 1), L - SBN);
        const int jmin = window > 0 ? i1 - window + 1 : 0;
        const int lo = n_ss + max(0, ceil_div<SBN>(jmin) - st_lo);
        const int hi = min(n, n_ss + floor_div<SBN>(jmax) - st_lo + 1);
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
    const int kslot0 = grp * C::HALF_K + wg * 64;  // K slots of this wave
    const int vslot0 = grp * C::HALF_V + wg * 64;  // V^T slots of this wave
    uint32_t kgoff;  // byte offset of this lane's K chunk from the stage's first row
    {
        const int s = kslot0 + lane;
        const int r = s / C::CPR;
        const int ch = (s % C::CPR) ^ kswz<D>(r);
        kgoff = (uint32_t)(r * a.k_l * 2 + ch * 16);
    }
    // A stage's V^T is NVH consecutive 32-key images of the workspace, so
    // this lane's chunk lies vgoff bytes past the stage's first image.
    const uint32_t vgoff = (uint32_t)(vslot0 + lane) * 16u;
    constexpr uint32_t kImage = D * BN * 2;  // bytes of one 32-key V^T image
    const __amdgpu_buffer_rsrc_t rk_all = make_rsrc(kb, WHOLE ? rows_bytes(0, L, a.k_l, D) : 0u);
    const __amdgpu_buffer_rsrc_t rv_all = make_rsrc(vtb, WHOLE ? (uint32_t)a.n_st * kImage : 0u);
    typedef __attribute__((address_space(3))) void lds_void;
    auto copy = [&](int t, auto buf) __attribute__((always_inline)) {
        const int j0 = __builtin_amdgcn_readfirstlane(stage_j0(min(t, n - 1)));
        const int si = j0 / BN;  // first 32-key image of the stage
        lds_void *kdst = (lds_void *)&sbuf(buf).k[kslot0 * 8];
        lds_void *vdst = (lds_void *)&sbuf(buf).v[vslot0 * 8];
        if constexpr (WHOLE) {
            // Offsets stay below 2^32: the K slice is < 2^31 bytes and a
            // stage reaches at most SBN - 1 rows (< 2^31 bytes at row
            // strides below 2^24 elements) past its end; the V^T images of
            // the slice span < 2^31 bytes, and images past the last one
            // (the second half of a last 64-key stage) read as zeros.
            const uint32_t ko = (uint32_t)j0 * (uint32_t)a.k_l * 2u;
            const uint32_t vo = (uint32_t)si * kImage;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk_all, kdst, 16, (int)(kgoff + ko), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv_all, vdst, 16, (int)(vgoff + vo), 0, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc(kb + (int64_t)j0 * a.k_l, rows_bytes(j0, L, a.k_l, D));
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(
                vtb + (int64_t)si * (D * BN), (uint32_t)min(NVH, a.n_st - si) * kImage);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kdst, 16, (int)kgoff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, vdst, 16, (int)vgoff, 0, 0, 0);
        }
    };

    // Fragments, scores and weights of a stage, one set per 32-key half
    // (half h: keys 32 h .. 32 h + 31 of the stage).
    const FragAddr<D> fa = frag_addr<D>(l16, G);
    KFrags<D> kf[NVH];
    VFrags<D> vf[NVH];
    Scores sc[NVH];
    Weights<PRECISE> pw[NVH];
    auto read_k = [&](auto b) __attribute__((always_inline)) {
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
            read_kfrags<D>(kf[hv], sbuf(b).k + hv * BN * D, fa);
    };
    auto all_offsets = [&]() __attribute__((always_inline)) {
        bool set = false;
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
            set = init_offsets<D>(cx, sc[hv], c);
        return set;
    };

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
            for (int hv = 0; hv < NVH; ++hv)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sc[hv].q[kt][e] = (BN * hv + 16 * kt + e <= dlim) ? sc[hv].q[kt][e] : kNegInf;
        } else if constexpr (decltype(masked)::value) {
#pragma unroll
            for (int hv = 0; hv < NVH; ++hv)
                mask_scores(sc[hv], stage_j0(t) + BN * hv, row, G, L, window, n_sink);
            if (!offsets_set)
                offsets_set = all_offsets();
        }
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                pin(sc[hv].q[kt]);
                pin(sc[hv].r[kt]);
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
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
            score_mfmas<D>(cx, kf[hv], sc[hv]);
        __builtin_amdgcn_sched_barrier(0);
        if (values) {
#pragma unroll
            for (int hv = 0; hv < NVH; ++hv)
                value_mfmas<D, PRECISE>(cx, vf[hv], pw[hv]);
        }
        read_k(b0 + 1);
#pragma unroll
        for (int i = 0; i < NVH * 2 * C::KC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, (PRECISE ? 2 : 1) * C::DT / C::KC, 0);
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
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
            read_vfrags<D>(vf[hv], sbuf(b0).v + hv * D * BN, fa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv) {
            weights<D, PRECISE>(cx, sc[hv], pw[hv], c);
            pin(pw[hv].p);
            pin(pw[hv].w);
            if constexpr (PRECISE) {
                pin(pw[hv].plo);
                pin(pw[hv].wlo);
            }
        }
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
        // Wait for this wave's Q and R loads and its copies of stages 0-2
        // (issued first), then publish them.  The first group's first two
        // M phases read K of stages 0-2; each wave's copies of stage s+3
        // are waited for at the end of its V phase of step s, but the
        // second group runs a phase behind and has had no V phase when the
        // first group reads stage 2, so stage 2 is waited for here.
        wait_copies<(AHEAD - 3) * C::COPIES>();
        __syncthreads();
        read_k(kB0);
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
                offsets_set = all_offsets();
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
#pragma unroll
        for (int hv = 0; hv < NVH; ++hv)
            value_mfmas<D, PRECISE>(cx, vf[hv], pw[hv]);
        if (grp == 0)
            phase_barrier();

        const float xmax = row_max4(cx.xlane);
        const bool overflow = pass == 0 && xmax * c > cx.m_ref + kTauHi;
        // Copies still in flight (stages past the end) land before LDS is
        // reused by the next pass.
        wait_copies<0>();
        if (!__syncthreads_or(overflow))
            break;
        if (tid == 0)
            atomicAdd(a.counters, 1u);
        // Exact offsets for the recomputation: each row's true max.
        cx.m_ref = xmax * c;
        cx.msub = cx.m_ref == kNegInf ? 0.f : cx.m_ref;
        offsets_set = true;
    }

    // Epilogue.  O is stored non-temporally, in whole lines (store_rows_nt;
    // rows past L compute values nobody stores); the precise instantiation,
    // one register short for the line exchange, stores each lane's pieces.
    const float ell_t = cx.accL[0];
    const float s_t = cx.accS[0];
    const float inv = 1.f / ell_t;
    const float keep = 1.f - s_t * inv;
    if constexpr (!PRECISE) {
        const int iw = i0 + ROWS * wave;  // the wavefront's first row
        store_rows_nt<C::DT>(a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)iw * a.o_l,
                             a.o_l, iw, L, l16, G, cx.accA, cx.accC, keep, inv);
    } else if (row < L) {
        float *ob = a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)row * a.o_l;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            f32x4 out;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                out[u] = (cx.accA[dt][u] * keep + cx.accC[dt][u]) * inv;
            __builtin_nontemporal_store(out, reinterpret_cast<f32x4 *>(ob + 16 * dt + 4 * G));
        }
    }
    if (row < L) {
        if (G == 0)
            __builtin_nontemporal_store((cx.m_ref + log2f(ell_t)) * kLn2, a.lse + (int64_t)bh * L + row);
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

// ---------------------------------------------------------------------------
// Windowed prefill: sliding windows of at most kWinMax keys with at most BN
// sink keys ("Sliding-window beats linear attention" review, sec. 1 and
// sec. 3: a 128-key window plus 4 sinks).  Such a row sees at most
// kWinMax + BN keys, so the work is bound by reading q, k, v, r and writing
// o, not by the matrix cores, and the kernel is shaped for streaming:
//   * a tile is 64 query rows (4 wavefronts x 16 rows); a workgroup walks a
//     run of consecutive tiles of one (batch, head), so K and V pass
//     through its LDS once, and runs of one head are placed on one XCD so
//     the key overlap between neighbouring runs is served by its L2;
//   * keys live in an LDS ring of 32-key stages (stage s in slot s % 8): a
//     tile spans at most 6 stages and adds 2 to the previous tile's, which
//     are loaded into registers while the current tile is computed and
//     written to their slots after it; the sink stage has its own buffer;
//   * V is converted to float16 and transposed here, 8 keys x 8 features
//     per thread in registers, into the same swizzled V^T layout the main
//     prefill kernel reads from its workspace: no prepass, no workspace;
//   * each wavefront takes only the stages its 16 rows see, the diagonal
//     stage first (every row sees its own key there, so that stage sets all
//     offsets), then the older window stages, then the sinks; a wavefront
//     whose scores outgrow its offsets recomputes its rows alone, since the
//     stages stay in LDS until the tile's closing barrier.
constexpr int WWAVES = 4;                 // wavefronts per workgroup
constexpr int WTHREADS = 64 * WWAVES;
constexpr int WROWS = ROWS * WWAVES;      // query rows per tile
constexpr int WRING = 8;                  // LDS stage slots
constexpr int WNEW = WROWS / BN;          // stages each tile adds to the previous one's
constexpr int kWinCUs = 256;              // compute units of the chip (MI355X)
constexpr int WPRO = 2 + (kFwdWinMax - 1 + BN - 1) / BN;  // most stages of one tile (6)
constexpr int kWinMax = kFwdWinMax;
// A tile spans 2 + ceil((W - 1) / BN) stages.
static_assert(2 + (kWinMax - 1 + BN - 1) / BN + WNEW <= WRING,
              "the ring holds a tile's stages and the next tile's new ones");
static_assert(kFwdWinSinkMax <= BN, "the sinks fit one stage");

// One thread's share of a stage's V^T image: the 8 keys x 4 features block
// (lane group G4 of positions, feature quad fq) of the stage starting at row
// `row0` of the resource, read from the bf16 values (8 x 8 bytes) ...
__device__ __forceinline__ void vblock_load(u32x2 (&raw)[8], __amdgpu_buffer_rsrc_t rv,
                                            int64_t v_l, int row0, int G4, int fq) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int key = row0 + (k < 4 ? 4 * G4 + k : 16 + 4 * G4 + (k - 4));
        raw[k] = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(key * v_l * 2 + 8 * fq), 0, 0);
    }
}

// ... and written to the stage as float16, transposed: feature 4 fq + cf,
// positions 8 G4 .. 8 G4 + 7 (the keys in the value MFMA's order), one
// 16-byte chunk per feature.
__device__ __forceinline__ void vblock_store(uint16_t *sv, const u32x2 (&raw)[8], int G4, int fq) {
    uint32_t hv[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            hv[k][i] = __builtin_bit_cast(uint32_t, cvt_f16x2(bf16_lo(raw[k][i]), bf16_hi(raw[k][i])));
#pragma unroll
    for (int cf = 0; cf < 4; ++cf) {
        u32x4 out;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            const uint32_t lo = hv[2 * pp][cf / 2], hi = hv[2 * pp + 1][cf / 2];
            out[pp] = (cf & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<u32x4 *>(sv + vswz_slot(4 * fq + cf, G4) * 8) = out;
    }
}

// Stages of which only one key tile (keys 16 h .. 16 h + 15) can be visible
// to the wavefront's rows take half the work: the score MFMAs, mask and
// weights of that tile only, and zero weights for the other one.
template <int D>
__device__ __forceinline__ void read_kfrags_half(KFrags<D> &kf, const uint16_t *sk,
                                                 const FragAddr<D> &fa, int h) {
    const char *base = reinterpret_cast<const char *>(sk);
#pragma unroll
    for (int kc = 0; kc < Cfg<D>::KC; ++kc)
        kf.f[h][kc] = *reinterpret_cast<const bf16x8 *>(base + fa.ka[kc] + h * 16 * Cfg<D>::CPR * 16);
}

template <int D>
__device__ __forceinline__ void score_mfmas_half(const Ctx<D> &cx, const KFrags<D> &kf, Scores &s,
                                                 int h) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    s.q[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[h][0], cx.qf[0], z, 0, 0, 0);
    s.r[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[h][0], cx.rf[0], z, 0, 0, 0);
#pragma unroll
    for (int kc = 1; kc < Cfg<D>::KC; ++kc) {
        s.q[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[h][kc], cx.qf[kc], s.q[h], 0, 0, 0);
        s.r[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[h][kc], cx.rf[kc], s.r[h], 0, 0, 0);
    }
}

__device__ __forceinline__ void mask_range_half(Scores &s, int lo, int hi, int h) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        s.q[h][e] = (16 * h + e >= lo && 16 * h + e <= hi) ? s.q[h][e] : kNegInf;
}

template <int D>
__device__ __forceinline__ void weights_half(Ctx<D> &cx, const Scores &s, Weights<false> &pw,
                                             float c, int h) {
    cx.xlane = fmaxf(fmaxf(cx.xlane, s.q[h][0]), fmaxf(fmaxf(s.q[h][1], s.q[h][2]), s.q[h][3]));
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
        const float p0 = exp2_fast(fmaf(s.q[h][e], c, -cx.msub));
        const float p1 = exp2_fast(fmaf(s.q[h][e + 1], c, -cx.msub));
        const f16x2 ph = cvt_f16x2(p0, p1);
        const f16x2 wh = cvt_f16x2(p0 * s.r[h][e], p1 * s.r[h][e + 1]);
        pw.p[4 * h + e] = ph[0];
        pw.p[4 * h + e + 1] = ph[1];
        pw.w[4 * h + e] = wh[0];
        pw.w[4 * h + e + 1] = wh[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pw.p[4 * (1 - h) + e] = (_Float16)0.f;
        pw.w[4 * (1 - h) + e] = (_Float16)0.f;
    }
}

// One pass over the stages of a wavefront in the common case of a window of
// NW stages: its 16 rows lie inside the sequence and past the window's start,
// so the stage list is always the diagonal stage (each row sees the keys up
// to itself), NW - 2 stages every row sees in full, the window's oldest
// stage (each row sees the keys from row - W + 1 on) and, with SINK, the
// sink stage (at most 16 sinks).  Every stage's kind and ring slot are then
// known at compile time: the pass is straight-line code (the same software
// pipeline as the general stage loop, without its branches, the register
// copies at their joins and the waits for loads a branch might have
// skipped), and a stage's mask is one per-lane threshold on the key offset
// 16 kt + e.  The sinks are keys 0-15, so the sink stage takes half the work.
template <int D, int NW, bool SINK>
__device__ __forceinline__ void window_pass(Ctx<D> &cx, VFrags<D> &vf, Weights<false> &pw,
                                            const StageBuf<D> *ring, const StageBuf<D> &sinkbuf,
                                            int hi_w, const FragAddr<D> &fa, int t_diag,
                                            int t_edge, int t_sink, float c) {
    static_assert(NW >= 3 && (WRING & (WRING - 1)) == 0, "window stages, ring slots");
    constexpr int NST = NW + (SINK ? 1 : 0);
    // Window stage hi_w - u (hi_w >= u here), or the sinks.
    auto buf = [&](int u) -> const StageBuf<D> & {
        return u < NW ? ring[(hi_w - u) & (WRING - 1)] : sinkbuf;
    };
    // The sink stage (u == NW) holds the sinks in keys 0-15: half the work.
    auto read_k = [&](KFrags<D> &kf, int u) {
        if (u == NW)
            read_kfrags_half<D>(kf, buf(u).k, fa, 0);
        else
            read_kfrags<D>(kf, buf(u).k, fa);
    };
    auto scores = [&](const KFrags<D> &kf, Scores &sc, int u) {
        if (u == NW)
            score_mfmas_half<D>(cx, kf, sc, 0);
        else
            score_mfmas<D>(cx, kf, sc);
    };
    KFrags<D> kf[2];
    Scores sc[2];
    read_k(kf[0], 0);
    read_k(kf[1], 1);
    scores(kf[0], sc[0], 0);
    read_k(kf[0], 2);
#pragma unroll
    for (int u = 0; u < NST; ++u) {
        Scores &cur = sc[u & 1];
        read_vfrags<D>(vf, buf(u).v, fa);
        // The V^T reads go first: the value MFMAs at the step's end wait
        // for them.
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < NST)
            scores(kf[(u + 1) & 1], sc[(u + 1) & 1], u + 1);
        if (u + 3 < NST)
            read_k(kf[(u + 1) & 1], u + 3);
        if (u == 0)
            mask_range(cur, INT32_MIN / 2, t_diag);
        else if (u == NW - 1)
            mask_range(cur, t_edge, INT32_MAX / 2);
        else if (u == NW)
            mask_range_half(cur, INT32_MIN / 2, t_sink, 0);
        // The diagonal stage sets the offsets: every row sees its own key.
        if (u == 0)
            init_offsets<D>(cx, cur, c);
        if (u == NW)
            weights_half<D>(cx, cur, pw, c, 0);
        else
            weights<D, false>(cx, cur, pw, c);
        value_mfmas<D, false>(cx, vf, pw);
        // Steps stay in order, so that later stages' reads are not hoisted
        // into this one (their registers would overlap the live ones).
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, bool STATS, bool PRECISE>
__global__ __launch_bounds__(WTHREADS, D == 64 ? 2 : 1) void parallax_fwd_window_kernel(FwdArgs a) {
    using C = Cfg<D>;
    constexpr int KCH = 32 * C::CPR / WTHREADS;  // K chunks per thread per stage
    constexpr int FG = D / 4;                    // feature quads of a V^T block
    constexpr int NVB = 4 * FG;                  // V^T blocks (8 keys x 4 features) per stage
    constexpr int BPW = WNEW * NVB / WWAVES;     // new-stage V^T blocks per wavefront
    constexpr int VPRO = ((WPRO + 1) * NVB + WTHREADS - 1) / WTHREADS;  // first-tile blocks per thread
    static_assert(KCH >= 1 && BPW <= 64 && WNEW * NVB % WWAVES == 0, "copy split");
    __shared__ StageBuf<D> ring[WRING];
    __shared__ StageBuf<D> sinkbuf;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;

    // Workgroup -> (batch, head, run): each XCD (block index mod 8) takes a
    // contiguous range of runs, in order.
    const int bid = blockIdx.x;
    const int lin = (bid % 8) * a.w_per_xcd + bid / 8;
    if (lin >= a.w_blocks)
        return;
    // The two workgroups on a CU run the same schedule: left in step, their
    // loads, stores and barriers fall together while the matrix cores idle,
    // and every workgroup of the chip loads its first tile at the same time.
    // Every other workgroup of an XCD therefore starts about 8000 cycles
    // (most of a tile) later when runs are long enough to amortise it.
    if (D == 64 && a.w_tpw >= 4 && ((bid / 8) & 1)) {
        __builtin_amdgcn_s_sleep(64);
        __builtin_amdgcn_s_sleep(64);
    }
    const int bh = lin / a.w_runs;
    const int run = lin - bh * a.w_runs;
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int L = a.L;
    const int window = a.window;
    const int n_sink = a.n_sink;
    const float c = a.scale_log2;
    const int m_first = run * a.w_tpw;
    const int m_end = min(m_first + a.w_tpw, a.w_tiles);

    const uint16_t *qb = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h;
    const uint16_t *rb = a.r + (int64_t)b * a.r_b + (int64_t)h * a.r_h;
    const uint16_t *kb = a.k + (int64_t)b * a.k_b + (int64_t)h * a.k_h;
    const uint16_t *vb = a.v + (int64_t)b * a.v_b + (int64_t)h * a.v_h;

    // Stages of tile m: from the first row's oldest window key to the last row.
    auto st_first = [&](int m) {
        const int lo = m * WROWS - window + 1;
        return lo > 0 ? lo / BN : 0;
    };
    auto st_last = [&](int m) { return (min(m * WROWS + WROWS, L) - 1) / BN; };

    // This thread's K chunks of a stage: slot s = tid + 256 ch holds chunk
    // (s % CPR) ^ kswz(row) of key row s / CPR.
    uint32_t koff[KCH];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch) {
        const int s = tid + WTHREADS * ch;
        const int r = s / C::CPR;
        koff[ch] = (uint32_t)(r * a.k_l * 2 + ((s % C::CPR) ^ kswz<D>(r)) * 16);
    }
    // Resource over the rows from stage st on (rows past L read as zeros);
    // row strides of at most 2^20 keep 6 stages of offsets within 32 bits.
    auto stage_rsrc = [&](const uint16_t *base, int64_t ld, int st) {
        const int j0 = st * BN;
        return make_rsrc(base + (int64_t)j0 * ld, rows_bytes(j0, L, ld, D));
    };

    // Q and R fragments of a tile (rows past L read as zeros).
    auto load_qr = [&](bf16x8 (&qf)[C::KC], bf16x8 (&rf)[C::KC], int m) {
        const int i0w = m * WROWS + ROWS * wave;
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(qb + (int64_t)i0w * a.q_l, rows_bytes(i0w, L, a.q_l, D));
        const __amdgpu_buffer_rsrc_t rr =
            make_rsrc(rb + (int64_t)i0w * a.r_l, rows_bytes(i0w, L, a.r_l, D));
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
            const uint32_t col = (32 * kc + 8 * G) * 2;
            qf[kc] = __builtin_bit_cast(bf16x8, bufld16(rq, (uint32_t)(l16 * a.q_l * 2) + col));
            rf[kc] = __builtin_bit_cast(bf16x8, bufld16(rr, (uint32_t)(l16 * a.r_l * 2) + col));
        }
    };
    Ctx<D> cx;
    load_qr(cx.qf, cx.rf, m_first);

    // The next tile's loads go through resources that move by a fixed number
    // of rows per tile (two K/V stages, 64 Q/R rows): a pointer and the bytes
    // left to the slice's last element, advanced by one addition each,
    // instead of 64-bit products of row indices and strides for five
    // resources at every tile.  A stream whose first row is past L has no
    // bytes, so its rows read as zeros, as with rows_bytes.
    struct RowStream {
        const char *p;
        int64_t rem;
    };
    auto stream_at = [&](const uint16_t *base, int64_t ld, int row) -> RowStream {
        return {reinterpret_cast<const char *>(base + (int64_t)row * ld),
                ((int64_t)L - 1 - row) * ld * 2 + 2 * D};
    };
    auto stream_rsrc = [&](const RowStream &st, int row) {
        const uint32_t n = row >= L || st.rem <= 0 ? 0u
                           : st.rem >= 0xffffffffll ? 0xffffffffu
                                                    : (uint32_t)st.rem;
        return make_rsrc(st.p, n);
    };
    const int kv_row0 = (st_last(m_first) + 1) * BN;
    const int qr_row0 = (m_first + 1) * WROWS + ROWS * wave;
    RowStream ks = stream_at(kb, a.k_l, kv_row0), vs = stream_at(vb, a.v_l, kv_row0);
    RowStream qs = stream_at(qb, a.q_l, qr_row0), rs = stream_at(rb, a.r_l, qr_row0);

    // The first tile's stages (at most WPRO) and the sink stage, every load
    // issued before the first LDS write.
    {
        const int s0 = st_first(m_first);
        const int n0 = st_last(m_first) - s0 + 1;
        const bool sink = n_sink > 0;
        const __amdgpu_buffer_rsrc_t rk = stage_rsrc(kb, a.k_l, s0);
        const __amdgpu_buffer_rsrc_t rv = stage_rsrc(vb, a.v_l, s0);
        const __amdgpu_buffer_rsrc_t rk0 = stage_rsrc(kb, a.k_l, 0);
        const __amdgpu_buffer_rsrc_t rv0 = stage_rsrc(vb, a.v_l, 0);
        u32x4 kraw[WPRO + 1][KCH];
        u32x2 vraw[VPRO][8];
#pragma unroll
        for (int p = 0; p <= WPRO; ++p)
#pragma unroll
            for (int ch = 0; ch < KCH; ++ch)
                if (p < n0)
                    kraw[p][ch] = bufld16(rk, koff[ch] + (uint32_t)(p * BN * a.k_l * 2));
                else if (p == WPRO && sink)
                    kraw[p][ch] = bufld16(rk0, koff[ch]);
#pragma unroll
        for (int i = 0; i < VPRO; ++i) {
            const int blk = tid + WTHREADS * i;
            const int p = blk / NVB;
            const int vb_ = blk % NVB;
            // Lanes of one wavefront may take blocks of two stages: the
            // resource is uniform, the stage is in each lane's offset.
            if (p < n0)
                vblock_load(vraw[i], rv, a.v_l, p * BN, vb_ / FG, vb_ % FG);
            else if (p == WPRO && sink)
                vblock_load(vraw[i], rv0, a.v_l, 0, vb_ / FG, vb_ % FG);
        }
#pragma unroll
        for (int p = 0; p <= WPRO; ++p)
#pragma unroll
            for (int ch = 0; ch < KCH; ++ch)
                if (p < n0 || (p == WPRO && sink)) {
                    StageBuf<D> &buf = p < WPRO ? ring[(s0 + p) % WRING] : sinkbuf;
                    *reinterpret_cast<u32x4 *>(&buf.k[(tid + WTHREADS * ch) * 8]) = kraw[p][ch];
                }
#pragma unroll
        for (int i = 0; i < VPRO; ++i) {
            const int blk = tid + WTHREADS * i;
            const int p = blk / NVB;
            const int vb_ = blk % NVB;
            if (p < n0 || (p == WPRO && sink)) {
                StageBuf<D> &buf = p < WPRO ? ring[(s0 + p) % WRING] : sinkbuf;
                vblock_store(buf.v, vraw[i], vb_ / FG, vb_ % FG);
            }
        }
    }

    // Every load so far has landed before the tile loop: the loop's wait
    // counts then only cover the loads each tile issues for the next one
    // (otherwise the first tile's Q/R loads would make every stage wait for
    // the whole prefetch).
    wait_copies<0>();
    __syncthreads();

    const FragAddr<D> fa = frag_addr<D>(l16, G);
    VFrags<D> vf;
    Weights<PRECISE> pw;
    // The next tile's new stages and Q/R, in flight during the current tile.
    u32x4 kpre[WNEW][KCH];
    u32x2 vpre[8];
    bf16x8 qn[C::KC], rn[C::KC];
    // The new stages' V^T blocks are spread evenly over the wavefronts:
    // lane < BPW of wavefront w converts block w * BPW + lane.
    const bool v_role = lane < BPW;
    const int vu = (wave * BPW + lane) / NVB;  // new stage of this lane's block
    const int vblk = (wave * BPW + lane) % NVB;

    for (int m = m_first; m < m_end; ++m) {
        const bool more = m + 1 < m_end;
        const int new_lo = st_last(m) + 1;
        const int n_new = more ? st_last(m + 1) - st_last(m) : 0;
        if (more) {
            // Stage new_lo + u is u * BN rows into the K stream (new_lo is
            // 2 (m + 1) here: tile m is not the sequence's last).
            const int kv_row = new_lo * BN;
            const __amdgpu_buffer_rsrc_t rk = stream_rsrc(ks, kv_row);
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(kb, 0u);
#pragma unroll
            for (int u = 0; u < WNEW; ++u)
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
                    kpre[u][ch] = __builtin_amdgcn_raw_buffer_load_b128(
                        u < n_new ? rk : rz, (int)koff[ch], (int)(u * BN * a.k_l * 2), 0);
            if (v_role && vu < n_new)
                vblock_load(vpre, stream_rsrc(vs, kv_row), a.v_l, vu * BN, vblk / FG, vblk % FG);
            const int qr_row = (m + 1) * WROWS + ROWS * wave;
            const __amdgpu_buffer_rsrc_t rq = stream_rsrc(qs, qr_row);
            const __amdgpu_buffer_rsrc_t rr = stream_rsrc(rs, qr_row);
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc) {
                const uint32_t col = (32 * kc + 8 * G) * 2;
                qn[kc] = __builtin_bit_cast(bf16x8, bufld16(rq, (uint32_t)(l16 * a.q_l * 2) + col));
                rn[kc] = __builtin_bit_cast(bf16x8, bufld16(rr, (uint32_t)(l16 * a.r_l * 2) + col));
            }
        }
        {
            const int64_t rows = WROWS;
            ks.p += rows * a.k_l * 2;
            ks.rem -= rows * a.k_l * 2;
            vs.p += rows * a.v_l * 2;
            vs.rem -= rows * a.v_l * 2;
            qs.p += rows * a.q_l * 2;
            qs.rem -= rows * a.q_l * 2;
            rs.p += rows * a.r_l * 2;
            rs.rem -= rows * a.r_l * 2;
        }

        // This wavefront's rows: the diagonal stage first, then older window
        // stages, then the sink stage when it lies before the window.
        const int i0w = m * WROWS + ROWS * wave;
        const int row = i0w + l16;
        if (i0w < L) {
            const int lo_w = i0w - window + 1 > 0 ? (i0w - window + 1) / BN : 0;
            const int hi_w = min(i0w + ROWS - 1, L - 1) / BN;
            const int n_win = hi_w - lo_w + 1;
            const int n_st = n_win + (n_sink > 0 && lo_w > 0 ? 1 : 0);
            cx.m_ref = kNegInf;
            cx.msub = 0.f;
            cx.xlane = kNegInf;
            // The common case takes the straight-line pass; the general stage
            // loop below covers the other tiles and the recomputation.
            int pass0 = 0;
            const int nw = !PRECISE && window == 128 && n_sink > 0 && n_sink <= 16 ? 5 : 0;
            if (nw > 0 && n_win == nw && lo_w > 0 && i0w + ROWS <= L) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    cx.accA[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                    cx.accC[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                }
                cx.accL = (f32x4){0.f, 0.f, 0.f, 0.f};
                cx.accS = (f32x4){0.f, 0.f, 0.f, 0.f};
                // Key offsets 16 kt + e visible to this lane's row: at most
                // t_diag in the diagonal stage, at least t_edge in the oldest
                // window stage, at most t_sink among the sinks.
                const int t_diag = row - hi_w * BN - 4 * G;
                const int t_edge = row - (hi_w - nw + 1) * BN - 4 * G - window + 1;
                const int t_sink = n_sink - 1 - 4 * G;
                if constexpr (!PRECISE) {
                    window_pass<D, 5, true>(cx, vf, pw, ring, sinkbuf, hi_w, fa, t_diag, t_edge,
                                            t_sink, c);
                }
                const float xmax = row_max4(cx.xlane);
                if (__builtin_amdgcn_ballot_w64(xmax * c > cx.m_ref + kTauHi) == 0) {
                    pass0 = 2;
                } else {
                    cx.m_ref = xmax * c;
                    cx.msub = cx.m_ref == kNegInf ? 0.f : cx.m_ref;
                    pass0 = 1;
                }
            }
            for (int pass = pass0; pass < 2; ++pass) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    cx.accA[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                    cx.accC[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                }
                cx.accL = (f32x4){0.f, 0.f, 0.f, 0.f};
                cx.accS = (f32x4){0.f, 0.f, 0.f, 0.f};
                // Stage u of the list: window stage hi_w - u, or the sinks.
                auto stage_buf = [&](int u) -> StageBuf<D> & {
                    return u < n_win ? ring[(hi_w - u) % WRING] : sinkbuf;
                };
                // Window stages every row of the wavefront sees in full need
                // no mask: keys [j_full_lo, j_full_hi] are visible to all 16.
                const int j_full_lo = i0w + ROWS - window;
                const int j_full_hi = min(i0w, L - 1);
                // Software pipeline over the stages: step u reads stage u's
                // V^T fragments, issues stage u+1's score MFMAs (their K
                // fragments were read two steps earlier), reads stage u+3's
                // K fragments into the buffer those MFMAs free, and meanwhile
                // forms stage u's weights on the VALU, then issues its value
                // MFMAs.  The matrix core and the VALU of one wavefront then
                // overlap instead of waiting on each other.
                auto step = [&](int u, Scores &cur, KFrags<D> &knext, Scores &nxt)
                    __attribute__((always_inline)) {
                    const int st = u < n_win ? hi_w - u : 0;
                    read_vfrags<D>(vf, stage_buf(u).v, fa);
                    if (u + 1 < n_st)
                        score_mfmas<D>(cx, knext, nxt);
                    if (u + 3 < n_st)
                        read_kfrags<D>(knext, stage_buf(u + 3).k, fa);
                    const int j0 = st * BN;
                    const bool full = u < n_win && j0 >= j_full_lo && j0 + BN - 1 <= j_full_hi;
                    // Lane offsets of its keys from the row: key j0 + 4G + o
                    // is at o - (row - j0 - 4G) from it.
                    const int rel = row - j0 - 4 * G;
                    if (u >= n_win)
                        mask_range(cur, INT32_MIN / 2, n_sink - 1 - 4 * G);  // sinks: j < n_sink
                    else if (j0 < n_sink)
                        mask_scores(cur, j0, row, G, L, window, n_sink);  // sinks inside the span
                    else if (!full)
                        mask_range(cur, rel - window + 1, rel);  // window and causal bounds
                    if (pass == 0 && u == 0)
                        init_offsets<D>(cx, cur, c);
                    weights<D, PRECISE>(cx, cur, pw, c);
                    value_mfmas<D, PRECISE>(cx, vf, pw);
                };
                KFrags<D> kf0, kf1;
                Scores sc0, sc1;
                read_kfrags<D>(kf0, stage_buf(0).k, fa);
                if (n_st > 1)
                    read_kfrags<D>(kf1, stage_buf(1).k, fa);
                score_mfmas<D>(cx, kf0, sc0);
                if (n_st > 2)
                    read_kfrags<D>(kf0, stage_buf(2).k, fa);
                for (int u = 0; u < n_st; u += 2) {
                    step(u, sc0, kf1, sc1);
                    if (u + 1 < n_st)
                        step(u + 1, sc1, kf0, sc0);
                }
                const float xmax = row_max4(cx.xlane);
                if (pass == 1 || __builtin_amdgcn_ballot_w64(xmax * c > cx.m_ref + kTauHi) == 0)
                    break;
                // Exact offsets for the recomputation: each row's true max.
                cx.m_ref = xmax * c;
                cx.msub = cx.m_ref == kNegInf ? 0.f : cx.m_ref;
            }
        }

        if (more) {
            // The new stages' slots held stages the previous tile used last;
            // the current tile does not read them.
#pragma unroll
            for (int u = 0; u < WNEW; ++u)
                if (u < n_new) {
                    StageBuf<D> &buf = ring[(new_lo + u) % WRING];
#pragma unroll
                    for (int ch = 0; ch < KCH; ++ch)
                        *reinterpret_cast<u32x4 *>(&buf.k[(tid + WTHREADS * ch) * 8]) = kpre[u][ch];
                }
            if (v_role && vu < n_new)
                vblock_store(ring[(new_lo + vu) % WRING].v, vpre, vblk / FG, vblk % FG);
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc) {
                cx.qf[kc] = qn[kc];
                cx.rf[kc] = rn[kc];
            }
        }
        // This tile's output goes out only now, after the wait for the
        // prefetched loads above: vmcnt counts stores as well, so stores
        // issued before that wait would hold every wavefront at the tile's
        // end until they are acknowledged.  Issued here, they drain while the
        // next tile is computed.
        __builtin_amdgcn_sched_barrier(0);
        if (i0w < L && row < L) {
            const float ell_t = cx.accL[0];
            const float s_t = cx.accS[0];
            const float inv = 1.f / ell_t;
            const float keep = 1.f - s_t * inv;
            float *ob = a.o + (int64_t)b * a.o_b + (int64_t)h * a.o_h + (int64_t)row * a.o_l;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = (cx.accA[dt][e] * keep + cx.accC[dt][e]) * inv;
                *reinterpret_cast<f32x4 *>(ob + 16 * dt + 4 * G) = out;
            }
            if (G == 0)
                a.lse[(int64_t)bh * L + row] = (cx.m_ref + log2f(ell_t)) * kLn2;
            if constexpr (STATS) {
                float *pb = a.pv + ((int64_t)bh * L + row) * D;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        out[e] = cx.accA[dt][e] * inv;
                    *reinterpret_cast<f32x4 *>(pb + 16 * dt + 4 * G) = out;
                }
                if (G == 0)
                    a.sbar[(int64_t)bh * L + row] = s_t * inv;
            }
        }
        __syncthreads();
    }
}

// Bytes from the first element of a [L, d] slice with row stride ld
// (2-byte elements) through its last element.
int64_t slice_bytes(int64_t L, int64_t ld, int d) { return (L - 1) * ld * 2 + (int64_t)d * 2; }

template <int D>
hipError_t launch_fwd_window(const FwdArgs &a, bool precise, hipStream_t stream) {
    FwdArgs args = a;
    void *params[] = {&args};
    // One round of workgroups: runs of consecutive tiles sized so that the
    // chip's workgroup slots (two per CU at d = 64, one at d = 128, set by
    // LDS) each take about one run.
    const int64_t tiles = ((int64_t)a.L + WROWS - 1) / WROWS;
    const int64_t slots = (int64_t)kWinCUs * (D == 64 ? 2 : 1);
    const int64_t total = (int64_t)a.B * a.H * tiles;
    const int64_t tpw = std::max<int64_t>(1, (total + slots - 1) / slots);
    args.w_tiles = (int)tiles;
    args.w_tpw = (int)std::min<int64_t>(tpw, tiles);
    args.w_runs = (int)((tiles + args.w_tpw - 1) / args.w_tpw);
    args.w_blocks = a.B * a.H * args.w_runs;
    args.w_per_xcd = (args.w_blocks + 7) / 8;
    const void *fn;
    if (a.pv)
        fn = reinterpret_cast<const void *>(&parallax_fwd_window_kernel<D, true, false>);
    else if (precise)
        fn = reinterpret_cast<const void *>(&parallax_fwd_window_kernel<D, false, true>);
    else
        fn = reinterpret_cast<const void *>(&parallax_fwd_window_kernel<D, false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)(8 * args.w_per_xcd)), dim3(WTHREADS), params, 0,
                           stream);
}

template <int D>
hipError_t launch_fwd_t(const FwdArgs &a, bool precise, hipStream_t stream) {
    if (a.window > 0 && a.window <= kFwdWinMax && a.n_sink <= kFwdWinSinkMax &&
        a.q_l <= kFwdWinMaxRowStride && a.k_l <= kFwdWinMaxRowStride &&
        a.v_l <= kFwdWinMaxRowStride && a.r_l <= kFwdWinMaxRowStride)
        return launch_fwd_window<D>(a, precise, stream);
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
        fn = whole ? reinterpret_cast<const void *>(&parallax_fwd_kernel<D, true, true, false>)
                   : reinterpret_cast<const void *>(&parallax_fwd_kernel<D, false, true, false>);
    else if (precise)
        fn = whole ? reinterpret_cast<const void *>(&parallax_fwd_kernel<D, true, false, true>)
                   : reinterpret_cast<const void *>(&parallax_fwd_kernel<D, false, false, true>);
    else
        fn = whole ? reinterpret_cast<const void *>(&parallax_fwd_kernel<D, true, false, false>)
                   : reinterpret_cast<const void *>(&parallax_fwd_kernel<D, false, false, false>);
    return hipLaunchKernel(fn, grid, block, params, 0, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int d, bool precise, hipStream_t stream) {
    return d == 64 ? launch_fwd_t<64>(a, precise, stream) : launch_fwd_t<128>(a, precise, stream);
}

}  // namespace plx
