// Fused input projections for gfx950: [Q | K | V | R] = X W^T in one GEMM.
//
// Parallax computes its probe from the layer input with a learned
// projection, rho_i = x_i W_R, next to the usual query, key and value
// projections (review page "Parallax: Parameterized Local Linear Attention
// for Language Modeling", sec. 1 and sec. 3).  Stacking W_Q, W_K, W_V and
// W_R row-wise makes the four projections one GEMM whose output row i is
// [q_i | k_i | v_i | rho_i] (each H heads of d features); the attention
// kernels read the four parts as strided [B, H, L, d] views of that output
// (row stride 4 H d, head stride d), so nothing is copied.
//
//   X: bf16 [M, K] row-major (M = B L tokens, K = model width)
//   W: bf16 [N, K] row-major (N = 4 H d output features, K contiguous)
//   Y: bf16 [M, N] row-major, fp32 accumulation, rounded to nearest even
//
// Mapping onto CDNA4:
//   * A workgroup computes a 256 x 256 tile of Y with 4 wavefronts (2 x 2),
//     one per SIMD, each a 128 x 128 tile as 8 x 8 blocks of 16 x 16 (256
//     accumulator registers), with v_mfma_f32_16x16x32_bf16 over 32-wide k
//     chunks.  The product is taken transposed (Y^T = W X^T): a lane's
//     accumulator holds four consecutive output features of one token,
//     stored as one 8-byte write.
//   * Each k chunk of both operands is copied into LDS as 1 KiB blocks in
//     fragment order (lane l holds row l % 16, k offsets 8 (l / 16) .. +7),
//     directly from global memory, three chunks ahead of use in four stage
//     buffers; fragment reads are one 16-byte LDS read per lane at l * 16.
//   * The fragments of chunk k + 1 are read into a second register set
//     while the 64 MFMAs of chunk k run, so LDS latency and the per-chunk
//     barrier hide behind the matrix cores.
//   * Blocks past the edges of X or W read zeros (buffer resources that end
//     at the last row); rows and columns past M and N are not stored.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

constexpr int TM = 256;      // tokens per workgroup tile
constexpr int TN = 256;      // output features per workgroup tile
constexpr int TK = 32;       // k per stage
constexpr int PW = 4;        // wavefronts per workgroup
constexpr int WM = 128;      // tokens per wavefront tile
constexpr int WN = 128;      // features per wavefront tile
constexpr int NSTAGE = 4;
constexpr int XBLK = TM / 16;  // X blocks per stage (16 rows x 32 k each)
constexpr int WBLK = TN / 16;  // W blocks per stage
constexpr int CPW = (XBLK + WBLK) / PW;  // copies per wave per stage

static_assert((XBLK + WBLK) % PW == 0 && XBLK % PW == 0, "copy split");
static_assert(TM == 2 * WM && TN == 2 * WN, "2 x 2 wavefronts");

struct ProjStage {
    u32x4 x[XBLK][64];
    u32x4 w[WBLK][64];
};

template <int I>
using SBuf = std::integral_constant<int, I % NSTAGE>;

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

__global__ __launch_bounds__(64 * PW) void parallax_proj_kernel(ProjArgs a) {
    __shared__ ProjStage s0, s1, s2, s3;
    auto sbuf = [&](auto b) -> ProjStage & {
        constexpr int i = decltype(b)::value % NSTAGE;
        if constexpr (i == 0) return s0;
        else if constexpr (i == 1) return s1;
        else if constexpr (i == 2) return s2;
        else return s3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;
    const int wm = wave / 2;  // wavefront row (tokens)
    const int wn = wave % 2;  // wavefront column (features)

    // Tile order.  Workgroups are dealt to the 8 XCDs round-robin
    // (blockIdx % 8), each XCD with its own L2, so the block index is first
    // renumbered to give every XCD one contiguous run of tiles; within the
    // run, tiles walk M fastest inside groups of GROUP M tiles, so that the
    // workgroups running together on one XCD share their X and W tiles in
    // that XCD's L2.
    const int n_tm = (a.M + TM - 1) / TM;
    const int n_tn = (a.N + TN - 1) / TN;
    const int n_tiles = n_tm * n_tn;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    const int per = n_tiles / 8, extra = n_tiles % 8;
    const int bid = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) +
                    slot;
    constexpr int GROUP = 8;
    const int group = bid / (GROUP * n_tn);
    const int first_m = group * GROUP;
    const int gsize = min(n_tm - first_m, GROUP);
    const int tile_m = first_m + (bid % (GROUP * n_tn)) % gsize;
    const int tile_n = (bid % (GROUP * n_tn)) / gsize;
    const int m0 = tile_m * TM;
    const int n0 = tile_n * TN;

    const int K = a.K;
    const int nk = (K + TK - 1) / TK;
    // Buffer resources over this tile's rows (rows past M or N read zeros;
    // columns past K read zeros because K is a multiple of 8 and each
    // 16-byte chunk is either fully inside or fully outside).
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(a.x + (int64_t)m0 * a.ldx, rows_bytes(m0, a.M, a.ldx, K));
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(a.w + (int64_t)n0 * a.ldw, rows_bytes(n0, a.N, a.ldw, K));

    // This lane's byte offsets for its copies (block c: rows 16 blk + l16,
    // k offset 8 G within the chunk); the chunk adds 2 * TK * kk bytes.
    uint32_t xoff[CPW], loff[CPW];
    bool is_x[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int bi = PW * c + wave;
        is_x[c] = bi < XBLK;
        const int blk = is_x[c] ? bi : bi - XBLK;
        const int row = 16 * blk + l16;
        const int64_t ld = is_x[c] ? a.ldx : a.ldw;
        // k positions past K are zero-filled by a second resource check:
        // the chunk lies inside the row whenever 8 G + 32 kk < K.
        xoff[c] = (uint32_t)(row * ld * 2 + 16 * G);
        loff[c] = (uint32_t)(bi * 1024);
    }
    auto copy = [&](int kk, auto buf) __attribute__((always_inline)) {
        const int kc = min(kk, nk - 1);
        char *base = reinterpret_cast<char *>(&sbuf(buf));
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            // Columns k >= K are outside every row's data only at the last
            // chunk; K % 32 == 0 is required by the host, so no chunk
            // crosses the end of a row.
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_x[c] ? rx : rw,
                                                     (lds_void *)(base + loff[c]), 16,
                                                     (int)xoff[c], kc * TK * 2, 0, 0);
        }
    };

    f32x4 acc[WN / 16][WM / 16];  // [feature tile][token tile], Y^T blocks
#pragma unroll
    for (int i = 0; i < WN / 16; ++i)
#pragma unroll
        for (int j = 0; j < WM / 16; ++j)
            acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Fragments of one chunk in registers.
    struct Frags {
        bf16x8 w[WN / 16], x[WM / 16];
    };
    auto read = [&](Frags &f, auto buf) __attribute__((always_inline)) {
        const ProjStage &S = sbuf(buf);
#pragma unroll
        for (int i = 0; i < WN / 16; ++i)
            f.w[i] = __builtin_bit_cast(bf16x8, S.w[wn * (WN / 16) + i][lane]);
#pragma unroll
        for (int j = 0; j < WM / 16; ++j)
            f.x[j] = __builtin_bit_cast(bf16x8, S.x[wm * (WM / 16) + j][lane]);
    };
    auto mfmas = [&](const Frags &f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WN / 16; ++i)
#pragma unroll
            for (int j = 0; j < WM / 16; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[i], f.x[j], acc[i][j], 0,
                                                                    0, 0);
    };
    // Step kk (chunk kk in buffer kk % 4, its fragments already in `cur`):
    // wait for this wave's copies of chunk kk + 1; the barrier then also
    // means every wave is done with the buffer of chunk kk - 1, which the
    // copy of chunk kk + 3 refills; read chunk kk + 1 into `nxt` and run
    // the MFMAs of chunk kk.
    auto step = [&](int kk, Frags &cur, Frags &nxt, auto buf) __attribute__((always_inline)) {
        wait_copies<CPW>();
        stage_barrier();
        copy(kk + 3, SBuf<decltype(buf)::value + 3>{});
        read(nxt, SBuf<decltype(buf)::value + 1>{});
        if (kk < nk)
            mfmas(cur);
    };

    Frags fa, fb;
    copy(0, SBuf<0>{});
    copy(1, SBuf<1>{});
    copy(2, SBuf<2>{});
    wait_copies<2 * CPW>();  // chunk 0
    stage_barrier();
    read(fa, SBuf<0>{});
    // Four steps per iteration keep the buffer numbers compile-time; the
    // fragment sets alternate.  Steps past the last chunk copy and read
    // the last chunk again (in bounds) and skip their MFMAs.
    for (int kk = 0; kk < nk; kk += 4) {
        step(kk, fa, fb, SBuf<0>{});
        step(kk + 1, fb, fa, SBuf<1>{});
        step(kk + 2, fa, fb, SBuf<2>{});
        step(kk + 3, fb, fa, SBuf<3>{});
    }
    wait_copies<0>();

    // Y^T block (i, j): lane holds features 4 G .. 4 G + 3 of token l16.
#pragma unroll
    for (int j = 0; j < WM / 16; ++j) {
        const int m = m0 + wm * WM + 16 * j + l16;
        if (m >= a.M)
            continue;
        uint16_t *yrow = a.y + (int64_t)m * a.ldy;
#pragma unroll
        for (int i = 0; i < WN / 16; ++i) {
            const int n = n0 + wn * WN + 16 * i + 4 * G;
            if (n >= a.N)
                continue;
            const f32x4 c = acc[i][j];
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
            const bf16x4 h = __builtin_convertvector(c, bf16x4);
            *reinterpret_cast<u32x2 *>(yrow + n) = __builtin_bit_cast(u32x2, h);
        }
    }
}

}  // namespace

size_t proj_tiles(int M, int N) {
    return (size_t)((M + TM - 1) / TM) * (size_t)((N + TN - 1) / TN);
}

hipError_t launch_proj(const ProjArgs &a, hipStream_t stream) {
    ProjArgs args = a;
    void *params[] = {&args};
    const dim3 grid((unsigned)proj_tiles(a.M, a.N));
    return hipLaunchKernel(reinterpret_cast<const void *>(&parallax_proj_kernel), grid,
                           dim3(64 * PW), params, 0, stream);
}

}  // namespace plx
