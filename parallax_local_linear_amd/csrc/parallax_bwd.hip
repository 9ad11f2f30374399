// Causal Parallax prefill backward for gfx950 (MI355X).
//
// Gradients of a loss through o (the log-sum-exp output carries none) with
// respect to q, k, v and the probe rho.  Method: Parallax keeps the softmax
// weights p_ij and multiplies each by 1 + rho_i.(k_j - kbar_i) (review page
// "Parallax: Parameterized Local Linear Attention for Language Modeling",
// sec. 1 and sec. 3).  With s_ij = rho_i.k_j and sbar_i = sum_j p_ij s_ij the
// output is o_i = sum_j p_ij t_ij v_j, t_ij = 1 + s_ij - sbar_i.  The chain
// rule gives, with g_ij = dO_i.v_j, G_i = sum_j p_ij g_ij = dO_i.pv_i
// (pv_i = sum_j p_ij v_j), Y_i = dO_i.o_i and e_ij = g_ij - G_i:
//
//     dv_j   = sum_i p_ij t_ij dO_i
//     dS_ij  = p_ij e_ij                          (gradient of s_ij)
//     dZ_ij  = p_ij (e_ij t_ij + G_i - Y_i)       (gradient of scale q_i.k_j)
//     dq_i   = scale sum_j dZ_ij k_j,    drho_i = sum_j dS_ij k_j
//     dk_j   = scale sum_i dZ_ij q_i  +  sum_i dS_ij rho_i
//
// Four kernels run in order:
//   * stats: per row lse*log2(e), 1 - sbar, G and G - Y (sbar and pv are
//     saved by the forward);
//   * records: q, rho, dO, k and v rearranged per 32-row stage into
//     row-major matrix-core operand blocks (below), so that every stage is
//     copied into LDS as contiguous 1 KiB blocks;
//   * key kernel: a workgroup owns 128 keys (16 per wavefront), streams the
//     query rows that see them and accumulates dv and dk;
//   * query kernel: a workgroup owns 128 query rows (16 per wavefront),
//     streams the keys they see and accumulates dq and drho.
// Eight wavefronts per workgroup, two per SIMD: LDS reads of 16 bytes per
// lane reach about twice the bandwidth with two wavefronts per SIMD as
// with one, and the two overlap each other's exponentials with their
// matrix-core work.
// Both recompute the scores (q.k, rho.k and dO.v) of every visible pair
// with v_mfma_f32_16x16x32_bf16; the weights p t, dS and scale dZ go to
// bfloat16 operands of the accumulating products.
//
// Operand layouts (16x16x32 MFMA: lane l reads row l % 16 and reduction
// positions 8 (l / 16) .. +7 of A; column l % 16 and the same positions of
// B; holds rows 4 (l / 16) .. +3 of column l % 16 of C):
//   * The key kernel computes C = Q K^T per 16 x 16 tile: a lane holds one
//     of the wavefront's 16 keys and four consecutive query rows.  Two
//     query tiles give a lane the
//     rows {4g .. 4g+3, 16+4g .. 16+4g+3} (g = l / 16) of a 32-row stage,
//     which it uses directly as the B operand of dv^T += dO^T (p t) over the
//     stage's 32 rows, provided the A operand lists the rows in the same
//     order.  The key kernel reads that A operand straight out of the
//     row-major q, rho and dO blocks with two ds_read_b64_tr_b16 per
//     fragment (LDS transpose reads), so the stage it copies holds each
//     tensor once.
//   * The query kernel computes C = K Q^T (a lane holds one query row and
//     four consecutive keys), and reads K^T for dq^T += K^T dZ^T out of the
//     row-major k blocks the same way.
//   * Row-major operands (q, rho, dO in the key kernel; k, v in the query
//     kernel) are stored as one 16-byte fragment per lane, so each
//     1 KiB block is read back with one 16-byte read per lane (at a slot
//     permuted so that the transpose reads are free of bank conflicts).  All of a stage's blocks are
//     one contiguous record, copied with one buffer resource and a scalar
//     offset per stage (no per-copy address arithmetic).
//
// Stages of 32 rows stream through three LDS buffers with direct
// global-to-LDS copies, two stages ahead.  Workgroups are issued heaviest
// first; the block index keeps all tiles of one (batch, head) on one XCD
// when B*H is a multiple of 8.  The key kernel walks its query stages from
// the last one down, so the workgroups of one (batch, head) that run at the
// same time read the same stage at about the same time and share it in L2
// (walking up from each block's diagonal would spread them over the
// sequence); the query kernel walks its key stages up from the first one,
// with the same effect.  Sink keys (sliding-window masks, "Sliding-
// window beats linear attention" review, sec. 1) are seen by every later
// row; the key blocks holding them split the rows past the window into
// chunks handled by separate workgroups that add into dk and dv atomically,
// so no workgroup walks the whole sequence.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

constexpr int BS = 32;        // rows per stage
constexpr int NW = 8;         // wavefronts per workgroup (two per SIMD)
constexpr int RT = 1;         // 16-row tiles per wavefront (keys or queries it owns)
constexpr int BT = 16 * RT * NW;  // rows (keys or queries) per workgroup
constexpr int NB = 3;         // LDS stage buffers
constexpr int NTHREADS = 64 * NW;
static_assert(BT == 128, "the host sizes the sink-block split for 128-row workgroups");
constexpr float kPosInf = __builtin_inff();

static_assert(BS == kStageKeys, "stage size shared with the workspace layout");

template <int D>
struct BCfg {
    static constexpr int KC = D / 32;  // reduction chunks of a score product
    static constexpr int DT = D / 16;  // feature tiles of an accumulation
};

// Two floats -> packed bfloat16, round to nearest even.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bool visible(int i, int j, int window, int n_sink) {
    return j <= i && (window <= 0 || i - j < window || j < n_sink);
}

// Barrier without a memory fence (a fence would also wait for the copies
// still in flight); LDS reads issued before it have completed.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void wait_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, (int)off, 0, 0, 0);
}

// Slot of a lane's 16-byte fragment piece within a 1 KiB operand block:
// lanes 16..31 and 48..63 are stored with slot bits 2 and 3 flipped.  The
// transpose reads below address, per 16-lane group, pieces of lanes
// {4G .. 4G+3} and {16+4G .. 16+4G+3}; stored unswizzled those sit 256
// bytes apart, in the same banks (a two-way conflict on every transpose
// read); with the flip they fall on distinct banks for 128-byte and
// 256-byte LDS cycles alike, and each 8 or 16 lanes of a row-major read
// still cover every bank once.
__device__ __forceinline__ int rec_slot(int lane) { return lane ^ (((lane >> 4) & 1) * 12); }

__device__ __forceinline__ bf16x8 lds_frag(const u32x4 *block, int lane) {
    return __builtin_bit_cast(bf16x8, block[rec_slot(lane)]);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Per-row statistics; also clears the rows of dk and dv that atomic chunks
// add into.  16 lanes per row, 16 rows per block.

template <int D>
__global__ __launch_bounds__(256) void parallax_bwd_stats_kernel(BwdArgs a) {
    constexpr int PER = D / 16;  // features per lane
    const int l16 = threadIdx.x & 15;
    const int i = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int L = a.L;
    const int BH = a.B * a.H;
    for (int bh = blockIdx.y; bh < BH; bh += gridDim.y) {
        const int b = bh / a.H;
        const int h = bh - b * a.H;
        float y = 0.f, g = 0.f;
        if (i < L) {
            const uint16_t *dp = a.dout + b * a.do_b + h * a.do_h + (int64_t)i * a.do_l + l16 * PER;
            const int64_t ro = ((int64_t)bh * L + i) * D + l16 * PER;
            uint32_t w[PER / 2];
            if constexpr (PER == 8) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(dp);
                for (int u = 0; u < 4; ++u) w[u] = x[u];
            } else {
                const u32x2 x = *reinterpret_cast<const u32x2 *>(dp);
                for (int u = 0; u < 2; ++u) w[u] = x[u];
            }
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const float d = (u & 1) ? bf16_hi(w[u / 2]) : bf16_lo(w[u / 2]);
                y = fmaf(d, a.o[ro + u], y);
                g = fmaf(d, a.pv[ro + u], g);
            }
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {
            y += __shfl_xor(y, m, 16);
            g += __shfl_xor(g, m, 16);
        }
        if (l16 == 0 && i < a.n_st * BS) {
            float *st = a.stats + ((int64_t)bh * a.n_st + i / BS) * 128 + (i % BS);
            const bool in = i < L;
            st[0] = in ? a.lse[(int64_t)bh * L + i] * kLog2e : kPosInf;
            st[32] = in ? 1.f - a.sbar[(int64_t)bh * L + i] : 0.f;
            st[64] = in ? g : 0.f;
            st[96] = in ? g - y : 0.f;
        }
        if (i < a.zero_rows) {
            const int64_t ro = ((int64_t)bh * L + i) * D + l16 * PER;
#pragma unroll
            for (int u = 0; u < PER; u += 4) {
                *reinterpret_cast<f32x4 *>(a.dk + ro + u) = (f32x4){0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4 *>(a.dv + ro + u) = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Stage records.  A thread copies 16 bytes (8 features) of 8 of a stage's
// rows into their places in the row-major operand blocks.  blockIdx.y picks
// the tensor: 0 q, 1 rho, 2 dO (key-kernel record), 3 k, 4 v (query-kernel
// record).

template <int D>
__global__ __launch_bounds__(256) void parallax_bwd_record_kernel(BwdArgs a) {
    constexpr int KC = D / 32;
    constexpr int FC = D / 8;        // 16-byte feature chunks per row
    constexpr int TPS = 4 * FC;      // threads per stage
    constexpr int SPB = 256 / TPS;   // stages per block
    constexpr int BLK = 64 * 8;      // bf16 elements per operand block
    constexpr int NB = 2 * KC;       // operand blocks per stage (two 16-row halves)
    constexpr int RS = FC + 1;       // LDS row stride in 16-byte pieces (padded)
    static_assert(SPB * NB * 64 == 256 * 8, "each thread stores 8 pieces");
    // The block's stages pass through LDS, so that each store instruction
    // writes one whole 1 KiB operand block (lane i to its slot i) instead of
    // 64 pieces in 64 different lines.
    __shared__ u32x4 rows_lds[SPB * BS * RS];
    const int t = threadIdx.x;
    const int st_in = t / TPS;
    const int s = blockIdx.x * SPB + st_in;
    const int G = (t % TPS) / FC;
    const int fc = t % FC;
    const int which = blockIdx.y;
    const int L = a.L;
    const int BH = a.B * a.H;
    const uint16_t *src = which == 0 ? a.q : which == 1 ? a.r : which == 2 ? a.dout
                        : which == 3 ? a.k : a.v;
    const int64_t sb = which == 0 ? a.q_b : which == 1 ? a.r_b : which == 2 ? a.do_b
                     : which == 3 ? a.k_b : a.v_b;
    const int64_t sh = which == 0 ? a.q_h : which == 1 ? a.r_h : which == 2 ? a.do_h
                     : which == 3 ? a.k_h : a.v_h;
    const int64_t sl = which == 0 ? a.q_l : which == 1 ? a.r_l : which == 2 ? a.do_l
                     : which == 3 ? a.k_l : a.v_l;
    // Record of this tensor, and the position of its blocks in it.
    const bool kv_side = which < 3;
    const int x = kv_side ? which : which - 3;
    const size_t rec_elems = kv_side ? bwd_kv_record_bytes(D) / 2 : bwd_q_record_bytes(D) / 2;
    uint16_t *recs = kv_side ? a.kvrec : a.qrec;
    const int rm_block0 = x * 2 * KC;
    // Stores: wavefront w writes operand blocks 8w .. 8w+7 of the block's
    // stages; lane i holds slot i, the piece of lane rec_slot(i) of the
    // fragment order (rec_slot is its own inverse).
    const int lane = t & 63;
    const int w = t >> 6;
    const int l = rec_slot(lane);
    for (int bh = blockIdx.z; bh < BH; bh += gridDim.z) {
        const int b = bh / a.H;
        const int h = bh - b * a.H;
        if (s < a.n_st) {
            const int i0 = s * BS;
            const uint16_t *base = src + b * sb + h * sh + (int64_t)i0 * sl;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows_bytes(i0, L, sl, D));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 8 * G + e;
                rows_lds[(st_in * BS + row) * RS + fc] =
                    bufld16(rs, (uint32_t)(row * sl * 2 + fc * 16));
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ob = 8 * w + i;
            const int so = ob / NB;           // stage of the block, within this workgroup's
            const int bis = ob - so * NB;     // its block: rows 16 R .., chunks 4 F ..
            const int R = bis / KC, F = bis - R * KC;
            const int s_out = blockIdx.x * SPB + so;
            if (s_out < a.n_st) {
                const u32x4 piece = rows_lds[(so * BS + 16 * R + (l & 15)) * RS + 4 * F + (l >> 4)];
                uint16_t *rec = recs + ((size_t)bh * a.n_st + s_out) * rec_elems;
                *reinterpret_cast<u32x4 *>(rec + (size_t)(rm_block0 + R * KC + F) * BLK +
                                           lane * 8) = piece;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Key kernel: dk and dv.

template <int D>
struct KvStage {
    u32x4 rm[3 * 2 * BCfg<D>::KC][64];  // row-major q, rho, dO: block (x, qt, kc)
    float st[4][BS];
};

// Transposed fragment of a row-major stage tensor from two LDS transpose
// reads (ds_read_b64_tr_b16): the A operand of dv^T += dO^T (p t) and of
// the dk^T products, feature row 16 dt + l16 and the stage rows
// {4G .. 4G+3, 16+4G .. 16+4G+3} (the order of the weights' B operand).
// Within each 16-lane group the read gives lane 4a + b element b of the
// 8-byte pieces addressed by lanes a, a+4, a+8, a+12; lane s of the group
// therefore addresses row 16h + 4G + s/4, features 16 dt + 4 (s % 4) .. +3,
// whose place in the fragment-order row-major blocks is
//   block (h, dt / 2), lane (4G + s/4) + 16 (2 (dt % 2) + (s % 4) / 2),
//   byte 8 ((s % 4) % 2) of its 16 (stored at slot rec_slot(lane)).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
template <int KC>
__device__ __forceinline__ bf16x8 lds_frag_t(const u32x4 (*blocks)[64], int dt, int lane) {
    const int G = lane >> 4, s = lane & 15;
    const int a4 = s & 3;
    const int off =
        rec_slot((4 * G + (s >> 2)) + 16 * (2 * (dt & 1) + (a4 >> 1))) * 16 + 8 * (a4 & 1);
    const char *b0 = reinterpret_cast<const char *>(&blocks[0 * KC + dt / 2][0]) + off;
    const char *b1 = reinterpret_cast<const char *>(&blocks[1 * KC + dt / 2][0]) + off;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(b0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(b1));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

template <int I>
using BufI = std::integral_constant<int, I % NB>;

template <int D>
__global__ __launch_bounds__(NTHREADS) void parallax_bwd_kv_kernel(BwdArgs a) {
    using C = BCfg<D>;
    constexpr int KC = C::KC, DT = C::DT;
    constexpr int NRM = 3 * 2 * KC;      // row-major blocks per stage
    constexpr int NCP = (NRM + NW - 1) / NW;  // block copies per wave per stage
    constexpr int COPIES = NCP + 1;      // + an eighth of the stage's statistics
    __shared__ KvStage<D> sb0, sb1, sb2;
    auto sbuf = [&](auto b) -> KvStage<D> & {
        constexpr int i = decltype(b)::value % NB;
        if constexpr (i == 0)
            return sb0;
        else if constexpr (i == 1)
            return sb1;
        else
            return sb2;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;

    const int BH = a.B * a.H;
    const int L = a.L;
    const int n_st = a.n_st;
    const int window = a.window;
    const int n_sink = a.n_sink;
    const int bh = blockIdx.x % BH;
    const int item = blockIdx.x / BH;
    const int b = bh / a.H;
    const int h = bh - b * a.H;

    // Work item: chunks of sink blocks first, then key blocks.
    const int n_chunk_items = a.n_sb * a.n_chunks;
    int kb, s_begin, s_end;
    bool atomic;
    auto window_end = [&](int kblk) {
        // first stage none of whose rows sees a non-sink key of block kblk
        return window > 0 ? min(n_st, (kblk * BT + BT - 1 + window - 1) / BS + 1) : n_st;
    };
    if (item < n_chunk_items) {
        kb = item / a.n_chunks;
        const int c = item - kb * a.n_chunks;
        s_begin = window_end(kb) + c * kBwdChunk;
        s_end = min(n_st, s_begin + kBwdChunk);
        atomic = true;
    } else {
        kb = item - n_chunk_items;
        s_begin = kb * (BT / BS);
        s_end = window_end(kb);
        atomic = kb < a.n_sb;
    }
    const int n = s_end - s_begin;
    if (n <= 0)
        return;
    const int j0 = kb * BT;
    constexpr int KW = 16 * RT;     // keys per wave
    const int jw = j0 + KW * wave;  // this wave's first key

    // This slice's stage records (one buffer resource for all of them).
    constexpr uint32_t kRec = (uint32_t)bwd_kv_record_bytes(D);
    const __amdgpu_buffer_rsrc_t r_rec =
        make_rsrc(a.kvrec + (size_t)bh * n_st * (kRec / 2), (uint32_t)n_st * kRec);
    const __amdgpu_buffer_rsrc_t r_st =
        make_rsrc(a.stats + (size_t)bh * n_st * 128, (uint32_t)(n_st * 512));

    // This wave's keys as B operands: key jw + 16 kt + l16, features
    // 32 kc + 8 G .. +7 (zeros past the end).
    bf16x8 kf[RT][KC], vf[RT][KC];
    {
        const uint16_t *kbase = a.k + b * a.k_b + h * a.k_h + (int64_t)jw * a.k_l;
        const uint16_t *vbase = a.v + b * a.v_b + h * a.v_h + (int64_t)jw * a.v_l;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, rows_bytes(jw, L, a.k_l, D));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, rows_bytes(jw, L, a.v_l, D));
#pragma unroll
        for (int kt = 0; kt < RT; ++kt)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int row = 16 * kt + l16;
                const int col = 32 * kc + 8 * G;
                kf[kt][kc] = __builtin_bit_cast(bf16x8, bufld16(rk, (uint32_t)((row * a.k_l + col) * 2)));
                vf[kt][kc] = __builtin_bit_cast(bf16x8, bufld16(rv, (uint32_t)((row * a.v_l + col) * 2)));
            }
    }

    f32x4 dv[DT][RT], dk[DT][RT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < RT; ++kt)
            dv[dt][kt] = dk[dt][kt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Copies of this wave's share of stage t (clamped: copies past the last
    // stage reload it into a buffer nobody reads again): record blocks
    // wave, wave + NW, ...; a spare slot repeats a block another wave also
    // copies (the same bytes), so every wave issues the same number of
    // copies.  The record's layout is the LDS stage's layout.
    auto copy = [&](int t, auto buf) __attribute__((always_inline)) {
        const int s = s_end - 1 - min(t, n - 1);
        KvStage<D> &S = sbuf(buf);
#pragma unroll
        for (int c = 0; c < NCP; ++c) {
            int bi = NW * c + wave;
            if (NW * (c + 1) > NRM && bi >= NRM)
                bi -= NRM;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r_rec, (lds_void *)(reinterpret_cast<char *>(&S) + bi * 1024), 16,
                (int)(bi * 1024 + lane * 16), (int)(s * kRec), 0, 0);
        }
        if (lane < 4)
            dma16(r_st, &S.st[0][0] + 16 * wave,
                  (uint32_t)(s * 512 + wave * 64 + lane * 16));
    };

    const float c2 = a.scale * kLog2e;
    const float scale = a.scale;

    auto compute = [&](int t, auto buf) __attribute__((always_inline)) {
        const int i0 = (s_end - 1 - t) * BS;
        // Visibility of this wave's 32 keys from the stage's 32 rows.
        const bool none = jw > i0 + BS - 1 ||
                          (window > 0 && i0 - (jw + KW - 1) >= window && jw >= n_sink);
        if (none)
            return;
        const bool full = jw + KW - 1 <= i0 &&
                          (window <= 0 || (i0 + BS - 1) - jw < window || jw + KW - 1 < n_sink);
        KvStage<D> &S = sbuf(buf);
        f32x4 z[2][RT], sr[2][RT], g[2][RT];  // [qt][kt]
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const bf16x8 aq = lds_frag(S.rm[0 * 2 * KC + qt * KC + kc], lane);
                const bf16x8 ar = lds_frag(S.rm[1 * 2 * KC + qt * KC + kc], lane);
                const bf16x8 ao = lds_frag(S.rm[2 * 2 * KC + qt * KC + kc], lane);
#pragma unroll
                for (int kt = 0; kt < RT; ++kt) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    z[qt][kt] = mfma(aq, kf[kt][kc], kc ? z[qt][kt] : zero);
                    sr[qt][kt] = mfma(ar, kf[kt][kc], kc ? sr[qt][kt] : zero);
                    g[qt][kt] = mfma(ao, vf[kt][kc], kc ? g[qt][kt] : zero);
                }
            }
        // Statistics of rows 16 qt + 4 G + u.
        f32x4 lse2[2], aa[2], gg[2], hh[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            lse2[qt] = *reinterpret_cast<const f32x4 *>(&S.st[0][16 * qt + 4 * G]);
            aa[qt] = *reinterpret_cast<const f32x4 *>(&S.st[1][16 * qt + 4 * G]);
            gg[qt] = *reinterpret_cast<const f32x4 *>(&S.st[2][16 * qt + 4 * G]);
            hh[qt] = *reinterpret_cast<const f32x4 *>(&S.st[3][16 * qt + 4 * G]);
        }
        bf16x8 wb[RT], zb[RT], sb[RT];
#pragma unroll
        for (int kt = 0; kt < RT; ++kt) {
            uint32_t pw[4], pz[4], ps[4];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int u = 0; u < 4; u += 2) {
                    float w2[2], z2[2], s2[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        float x = fmaf(z[qt][kt][u + v], c2, -lse2[qt][u + v]);
                        if (!full) {
                            const int i = i0 + 16 * qt + 4 * G + u + v;
                            const int j = jw + 16 * kt + l16;
                            if (!visible(i, j, window, n_sink))
                                x = -kPosInf;
                        }
                        const float p = exp2_fast(x);
                        const float tt = sr[qt][kt][u + v] + aa[qt][u + v];
                        const float e = g[qt][kt][u + v] - gg[qt][u + v];
                        w2[v] = p * tt;
                        s2[v] = p * e;
                        z2[v] = (p * scale) * fmaf(e, tt, hh[qt][u + v]);
                    }
                    pw[2 * qt + u / 2] = pk_bf16(w2[0], w2[1]);
                    pz[2 * qt + u / 2] = pk_bf16(z2[0], z2[1]);
                    ps[2 * qt + u / 2] = pk_bf16(s2[0], s2[1]);
                }
            wb[kt] = __builtin_bit_cast(bf16x8, (u32x4){pw[0], pw[1], pw[2], pw[3]});
            zb[kt] = __builtin_bit_cast(bf16x8, (u32x4){pz[0], pz[1], pz[2], pz[3]});
            sb[kt] = __builtin_bit_cast(bf16x8, (u32x4){ps[0], ps[1], ps[2], ps[3]});
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 tq = lds_frag_t<KC>(&S.rm[0 * 2 * KC], dt, lane);
            const bf16x8 tr = lds_frag_t<KC>(&S.rm[1 * 2 * KC], dt, lane);
            const bf16x8 to = lds_frag_t<KC>(&S.rm[2 * 2 * KC], dt, lane);
#pragma unroll
            for (int kt = 0; kt < RT; ++kt) {
                dv[dt][kt] = mfma(to, wb[kt], dv[dt][kt]);
                dk[dt][kt] = mfma(tq, zb[kt], dk[dt][kt]);
                dk[dt][kt] = mfma(tr, sb[kt], dk[dt][kt]);
            }
        }
    };

    auto step = [&](int t, auto buf) __attribute__((always_inline)) {
        wait_copies<COPIES>();
        stage_barrier();
        copy(t + 2, BufI<decltype(buf)::value + 2>{});
        compute(t, buf);
    };

    copy(0, BufI<0>{});
    copy(1, BufI<1>{});
    int t = 0;
    for (; t + 2 < n; t += 3) {
        step(t, BufI<0>{});
        step(t + 1, BufI<1>{});
        step(t + 2, BufI<2>{});
    }
    if (t < n) {
        step(t, BufI<0>{});
        if (t + 1 < n)
            step(t + 1, BufI<1>{});
    }
    wait_copies<0>();

    // dk and dv of keys jw + 16 kt + l16, features 16 dt + 4 G .. +3.
#pragma unroll
    for (int kt = 0; kt < RT; ++kt) {
        const int j = jw + 16 * kt + l16;
        if (j >= L)
            continue;
        float *pk = a.dk + ((int64_t)bh * L + j) * D + 4 * G;
        float *pv = a.dv + ((int64_t)bh * L + j) * D + 4 * G;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if (atomic) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    unsafeAtomicAdd(pk + 16 * dt + u, dk[dt][kt][u]);
                    unsafeAtomicAdd(pv + 16 * dt + u, dv[dt][kt][u]);
                }
            } else {
                *reinterpret_cast<f32x4 *>(pk + 16 * dt) = dk[dt][kt];
                *reinterpret_cast<f32x4 *>(pv + 16 * dt) = dv[dt][kt];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Query kernel: dq and drho.

template <int D>
struct QStage {
    u32x4 rm[2 * 2 * BCfg<D>::KC][64];  // row-major k, v: block (x, kt, kc)
};

template <int D>
__global__ __launch_bounds__(NTHREADS) void parallax_bwd_q_kernel(BwdArgs a) {
    using C = BCfg<D>;
    constexpr int KC = C::KC, DT = C::DT;
    constexpr int NRM = 2 * 2 * KC;
    constexpr int NCP = (NRM + NW - 1) / NW;
    __shared__ QStage<D> sb0, sb1, sb2;
    auto sbuf = [&](auto b) -> QStage<D> & {
        constexpr int i = decltype(b)::value % NB;
        if constexpr (i == 0)
            return sb0;
        else if constexpr (i == 1)
            return sb1;
        else
            return sb2;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;

    const int BH = a.B * a.H;
    const int L = a.L;
    const int n_st = a.n_st;
    const int window = a.window;
    const int n_sink = a.n_sink;
    const int n_qb = (L + BT - 1) / BT;
    const int bh = blockIdx.x % BH;
    const int qblk = n_qb - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int i0 = qblk * BT;
    constexpr int QW = 16 * RT;     // rows per wave
    const int iw = i0 + QW * wave;  // this wave's first row

    // Key stages: sink stages below the window, then the window up to the
    // diagonal.
    const int hi = min(n_st - 1, (i0 + BT - 1) / BS);
    const int lo = window > 0 ? max(0, i0 - window + 1) / BS : 0;
    const int ns = (window > 0 && n_sink > 0) ? min((n_sink + BS - 1) / BS, lo) : 0;
    const int n = ns + hi - lo + 1;
    auto stage_of = [&](int t) { return t < ns ? t : lo + (t - ns); };

    constexpr uint32_t kRec = (uint32_t)bwd_q_record_bytes(D);
    const __amdgpu_buffer_rsrc_t r_rec =
        make_rsrc(a.qrec + (size_t)bh * n_st * (kRec / 2), (uint32_t)n_st * kRec);

    // This wave's rows as B operands: row iw + 16 qt + l16, features
    // 32 kc + 8 G .. +7.
    bf16x8 qf[RT][KC], rf[RT][KC], of[RT][KC];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(
            a.q + b * a.q_b + h * a.q_h + (int64_t)iw * a.q_l, rows_bytes(iw, L, a.q_l, D));
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(
            a.r + b * a.r_b + h * a.r_h + (int64_t)iw * a.r_l, rows_bytes(iw, L, a.r_l, D));
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(
            a.dout + b * a.do_b + h * a.do_h + (int64_t)iw * a.do_l, rows_bytes(iw, L, a.do_l, D));
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int row = 16 * qt + l16;
                const int col = 32 * kc + 8 * G;
                qf[qt][kc] = __builtin_bit_cast(bf16x8, bufld16(rq, (uint32_t)((row * a.q_l + col) * 2)));
                rf[qt][kc] = __builtin_bit_cast(bf16x8, bufld16(rr, (uint32_t)((row * a.r_l + col) * 2)));
                of[qt][kc] = __builtin_bit_cast(bf16x8, bufld16(ro, (uint32_t)((row * a.do_l + col) * 2)));
            }
    }
    // Statistics of rows iw + 16 qt + l16 (+inf offset past the end).
    float lse2[RT], aa[RT], gg[RT], hh[RT];
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) {
        const int i = iw + 16 * qt + l16;
        const float *st = a.stats + ((int64_t)bh * n_st + i / BS) * 128 + (i % BS);
        const bool in = i < n_st * BS;
        lse2[qt] = in ? st[0] : kPosInf;
        aa[qt] = in ? st[32] : 0.f;
        gg[qt] = in ? st[64] : 0.f;
        hh[qt] = in ? st[96] : 0.f;
    }

    f32x4 dq[DT][RT], dr[DT][RT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
            dq[dt][qt] = dr[dt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Copies as in the key kernel.
    auto copy = [&](int t, auto buf) __attribute__((always_inline)) {
        const int s = stage_of(min(t, n - 1));
        QStage<D> &S = sbuf(buf);
#pragma unroll
        for (int c = 0; c < NCP; ++c) {
            int bi = NW * c + wave;
            if (NW * (c + 1) > NRM && bi >= NRM)
                bi -= NRM;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r_rec, (lds_void *)(reinterpret_cast<char *>(&S) + bi * 1024), 16,
                (int)(bi * 1024 + lane * 16), (int)(s * kRec), 0, 0);
        }
    };

    const float c2 = a.scale * kLog2e;

    auto compute = [&](int t, auto buf) __attribute__((always_inline)) {
        const int j0 = stage_of(t) * BS;
        const bool none = j0 > iw + QW - 1 ||
                          (window > 0 && iw - (j0 + BS - 1) >= window && j0 >= n_sink);
        if (none)
            return;
        const bool full = j0 + BS - 1 <= iw &&
                          (window <= 0 || (iw + QW - 1) - j0 < window || j0 + BS - 1 < n_sink);
        QStage<D> &S = sbuf(buf);
        f32x4 z[2][RT], sr[2][RT], g[2][RT];  // [kt][qt]
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 ak = lds_frag(S.rm[0 * 2 * KC + kt * KC + kc], lane);
                const bf16x8 av = lds_frag(S.rm[1 * 2 * KC + kt * KC + kc], lane);
#pragma unroll
                for (int qt = 0; qt < RT; ++qt) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    z[kt][qt] = mfma(ak, qf[qt][kc], kc ? z[kt][qt] : zero);
                    sr[kt][qt] = mfma(ak, rf[qt][kc], kc ? sr[kt][qt] : zero);
                    g[kt][qt] = mfma(av, of[qt][kc], kc ? g[kt][qt] : zero);
                }
            }
        bf16x8 zb[RT], sb[RT];
#pragma unroll
        for (int qt = 0; qt < RT; ++qt) {
            uint32_t pz[4], ps[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int u = 0; u < 4; u += 2) {
                    float z2[2], s2[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        float x = fmaf(z[kt][qt][u + v], c2, -lse2[qt]);
                        if (!full) {
                            const int i = iw + 16 * qt + l16;
                            const int j = j0 + 16 * kt + 4 * G + u + v;
                            if (!visible(i, j, window, n_sink))
                                x = -kPosInf;
                        }
                        const float p = exp2_fast(x);
                        const float tt = sr[kt][qt][u + v] + aa[qt];
                        const float e = g[kt][qt][u + v] - gg[qt];
                        s2[v] = p * e;
                        z2[v] = p * fmaf(e, tt, hh[qt]);
                    }
                    pz[2 * kt + u / 2] = pk_bf16(z2[0], z2[1]);
                    ps[2 * kt + u / 2] = pk_bf16(s2[0], s2[1]);
                }
            zb[qt] = __builtin_bit_cast(bf16x8, (u32x4){pz[0], pz[1], pz[2], pz[3]});
            sb[qt] = __builtin_bit_cast(bf16x8, (u32x4){ps[0], ps[1], ps[2], ps[3]});
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 tk = lds_frag_t<KC>(&S.rm[0], dt, lane);
#pragma unroll
            for (int qt = 0; qt < RT; ++qt) {
                dq[dt][qt] = mfma(tk, zb[qt], dq[dt][qt]);
                dr[dt][qt] = mfma(tk, sb[qt], dr[dt][qt]);
            }
        }
    };

    auto step = [&](int t, auto buf) __attribute__((always_inline)) {
        wait_copies<NCP>();
        stage_barrier();
        copy(t + 2, BufI<decltype(buf)::value + 2>{});
        compute(t, buf);
    };

    copy(0, BufI<0>{});
    copy(1, BufI<1>{});
    int t = 0;
    for (; t + 2 < n; t += 3) {
        step(t, BufI<0>{});
        step(t + 1, BufI<1>{});
        step(t + 2, BufI<2>{});
    }
    if (t < n) {
        step(t, BufI<0>{});
        if (t + 1 < n)
            step(t + 1, BufI<1>{});
    }
    wait_copies<0>();

    const float scale = a.scale;
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) {
        const int i = iw + 16 * qt + l16;
        if (i >= L)
            continue;
        float *pq = a.dq + ((int64_t)bh * L + i) * D + 4 * G;
        float *pr = a.dr + ((int64_t)bh * L + i) * D + 4 * G;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 x = dq[dt][qt];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                x[u] *= scale;
            *reinterpret_cast<f32x4 *>(pq + 16 * dt) = x;
            *reinterpret_cast<f32x4 *>(pr + 16 * dt) = dr[dt][qt];
        }
    }
}

template <int D>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
    BwdArgs args = a;
    void *params[] = {&args};
    const int BH = a.B * a.H;
    const unsigned gz = (unsigned)min(BH, 65535);
    hipError_t e;
    {
        const dim3 grid((unsigned)((a.n_st * BS + 15) / 16), gz);
        e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_bwd_stats_kernel<D>), grid,
                            dim3(256), params, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    {
        constexpr int SPB = 256 / (4 * (D / 8));
        const dim3 grid((unsigned)((a.n_st + SPB - 1) / SPB), 5, gz);
        e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_bwd_record_kernel<D>), grid,
                            dim3(256), params, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    const int n_kb = (a.L + BT - 1) / BT;
    {
        const dim3 grid((unsigned)(BH * (n_kb + a.n_sb * a.n_chunks)));
        e = hipLaunchKernel(reinterpret_cast<const void *>(&parallax_bwd_kv_kernel<D>), grid,
                            dim3(NTHREADS), params, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    const dim3 grid((unsigned)(BH * n_kb));
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_bwd_q_kernel<D>), grid,
                           dim3(NTHREADS), params, 0, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int d, hipStream_t stream) {
    return d == 64 ? launch_bwd_t<64>(a, stream) : launch_bwd_t<128>(a, stream);
}

}  // namespace plx
