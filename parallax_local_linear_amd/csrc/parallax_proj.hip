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
//   * A workgroup computes a 256 x 256 tile of Y with 8 wavefronts (2 x 4),
//     two per SIMD, each a 128 x 64 tile as 4 x 8 blocks of 16 x 16 (128
//     accumulator registers), with v_mfma_f32_16x16x32_bf16 over 32-wide k
//     chunks.  Two wavefronts per SIMD read LDS at about 1.4 times the rate
//     of one, and each covers the other's waits.  The product is taken transposed (Y^T = W X^T): a lane's
//     accumulator holds four consecutive output features of one token,
//     stored as one 8-byte write.
//   * Operands reach LDS in stages 64 k wide, copied directly from global
//     memory into two stage buffers, a stage's copy issued while the stage
//     before it runs.  Each copy moves
//     8 rows x 128 bytes, whole 128-byte lines: copies of 16 rows x 64 bytes
//     (a 32-k chunk) move about a quarter as many bytes per clock from L2.
//     A row's eight 16-byte pieces land in LDS XOR-swizzled by the row
//     (piece c of row r at slot c ^ (r % 8) ^ ((r / 8) % 2)), so the
//     fragment reads (16 rows x 16 bytes per 16 lanes) hit distinct banks.
//   * The fragments of the next 32-k half are read into a second register
//     set while the MFMAs of the current half run, so LDS latency and the
//     per-stage barrier hide behind the matrix cores.  A half runs in four
//     fenced chunks, each a few fragment reads (and, in a second half, two
//     copies) followed by 8 MFMAs, so reads and copies leave spread over
//     the half instead of in one burst.
//   * Persistent: one workgroup per compute unit walks its tiles with one
//     stream of stages across them, so the next tile's first stages are
//     copied while the current tile's last ones run and its outputs are
//     stored while the next tile's first MFMAs run.
//   * Blocks past the edges of X or W read zeros (buffer resources that end
//     at the last row); rows and columns past M and N are not stored.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

constexpr int TM = 256;      // tokens per workgroup tile
constexpr int TN = 256;      // output features per workgroup tile
constexpr int TK = 64;       // k per stage (two 32-k halves)
constexpr int PW = 8;        // wavefronts per workgroup (2 x 4, two per SIMD)
constexpr int WM = 128;      // tokens per wavefront tile
constexpr int WN = 64;       // features per wavefront tile
constexpr int XGRP = TM / 8;  // 8-row copy groups of X per stage
constexpr int WGRP = TN / 8;  // of W
constexpr int CPW = (XGRP + WGRP) / PW;  // copies per wave per stage

static_assert((XGRP + WGRP) % PW == 0 && XGRP % PW == 0, "copy split");
static_assert(TM == 2 * WM && TN == 4 * WN, "2 x 4 wavefronts");

// One stage: rows of 128 bytes (64 k), pieces swizzled as described above.
struct ProjStage {
    u32x4 x[TM][8];
    u32x4 w[TN][8];
};

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

// LDS slot of 16-byte piece c of row r within its stage operand.
__device__ __forceinline__ int piece_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef __attribute__((address_space(3))) void lds_void;

struct Tile {
    int m0, n0;
};

// Tile of virtual block v.  Workgroups are dealt to the 8 XCDs round-robin
// (v % 8, with a grid that is a multiple of 8), each XCD with its own L2, so
// v is first renumbered to give every XCD one contiguous run of tiles;
// within the run, tiles walk M fastest inside groups of GROUP M tiles, so
// that the workgroups running together on one XCD share their X and W tiles
// in that XCD's L2.
__device__ __forceinline__ Tile tile_of(int v, int n_tm, int n_tn) {
    const int n_tiles = n_tm * n_tn;
    const int xcd = v % 8;
    const int slot = v / 8;
    const int per = n_tiles / 8, extra = n_tiles % 8;
    const int bid = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) +
                    slot;
    constexpr int GROUP = 8;
    const int group = bid / (GROUP * n_tn);
    const int first_m = group * GROUP;
    const int gsize = min(n_tm - first_m, GROUP);
    const int tile_m = first_m + (bid % (GROUP * n_tn)) % gsize;
    const int tile_n = (bid % (GROUP * n_tn)) / gsize;
    return {tile_m * TM, tile_n * TN};
}

// ODD: K % 64 == 32 (each tile's last stage has one live half).
template <bool ODD>
__global__ __launch_bounds__(64 * PW) void parallax_proj_kernel(ProjArgs a) {
    __shared__ ProjStage stg[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int G = lane >> 4;
    const int wm = wave / 4;  // wavefront row (tokens)
    const int wn = wave % 4;  // wavefront column (features)

    const int n_tm = (a.M + TM - 1) / TM;
    const int n_tn = (a.N + TN - 1) / TN;
    const int n_tiles = n_tm * n_tn;
    const int grid = (int)gridDim.x;
    // This workgroup's tiles: virtual blocks blockIdx.x + t * grid.
    const int ntl = (n_tiles - (int)blockIdx.x + grid - 1) / grid;

    const int K = a.K;
    const int nh = K / 32;           // 32-k halves (the host requires K % 32 == 0)
    const int ns = (nh + 1) / 2;     // stages per tile
    // Buffer resources over a tile's rows: rows past M or N read zeros.
    // With K % 64 == 32 the last stage's second half reads the 64 bytes past
    // K of each row (the next row's start, row padding, or zeros past the
    // resource); its MFMAs are skipped.
    auto rsrc_x = [&](int m0) {
        return make_rsrc(a.x + (int64_t)m0 * a.ldx, rows_bytes(m0, a.M, a.ldx, K));
    };
    auto rsrc_w = [&](int n0) {
        return make_rsrc(a.w + (int64_t)n0 * a.ldw, rows_bytes(n0, a.N, a.ldw, K));
    };

    // This lane's copies: copy c of wave w moves 8-row group g = PW c + w
    // (of X for g < XGRP, then of W), row 8 g' + l / 8 of the operand, the
    // 16-byte piece whose swizzled slot is l % 8, into 1 KiB of LDS per
    // group, lane-linear.  The swizzle of row 8 g' + l / 8 is
    // (l / 8) ^ (g' % 2) = (l / 8) ^ (w % 2) (PW is even), the same for
    // every copy of the wave, so copies differ by the uniform 8 PW rows per
    // copy: one per-lane offset per operand and scalar offsets.
    static_assert(PW % 2 == 0, "swizzle of a copy group");
    const int crow = 8 * wave + (lane >> 3);
    const int cpiece = (lane & 7) ^ piece_swizzle(crow);
    const uint32_t gx = (uint32_t)(crow * a.ldx * 2 + 16 * cpiece);
    const uint32_t gw = (uint32_t)(crow * a.ldw * 2 + 16 * cpiece);
    const uint32_t sx = (uint32_t)(8 * PW * a.ldx * 2);  // per copy
    const uint32_t sw_ = (uint32_t)(8 * PW * a.ldw * 2);
    // Copy stream: stage c_st of this workgroup's c_tile-th tile; past the
    // last stage it copies the last stage again (in bounds, never used).
    int c_tile = 0, c_st = 0;
    Tile ct = tile_of((int)blockIdx.x, n_tm, n_tn);
    __amdgpu_buffer_rsrc_t crx = rsrc_x(ct.m0), crw = rsrc_w(ct.n0);
    auto copy_one = [&](int buf, int c) __attribute__((always_inline)) {
        char *base = reinterpret_cast<char *>(&stg[buf]);
        const int gi = PW * c + wave;
        if (PW * c < XGRP)  // the same for every wave
            __builtin_amdgcn_raw_ptr_buffer_load_lds(crx, (lds_void *)(base + gi * 1024), 16,
                                                     (int)gx, (int)(c * sx) + c_st * TK * 2, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                crw, (lds_void *)(base + (int)sizeof(ProjStage::x) + (gi - XGRP) * 1024), 16,
                (int)gw, (int)((c - XGRP / PW) * sw_) + c_st * TK * 2, 0, 0);
    };
    auto copy_advance = [&]() __attribute__((always_inline)) {
        if (c_st + 1 < ns) {
            ++c_st;
        } else if (c_tile + 1 < ntl) {
            c_st = 0;
            ++c_tile;
            ct = tile_of((int)blockIdx.x + c_tile * grid, n_tm, n_tn);
            crx = rsrc_x(ct.m0);
            crw = rsrc_w(ct.n0);
        }
    };
    auto copy_next = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
            copy_one(buf, c);
        copy_advance();
    };

    f32x4 acc[WN / 16][WM / 16];  // [feature tile][token tile], Y^T blocks

    // Fragment reads: lane l holds row l16 of a 16-row block, k offsets
    // 8 G .. 8 G + 7 of a 32-k half h, i.e. piece 4 h + G of the row.  Rows
    // of a block are 16-aligned, so the swizzle depends on l16 only.
    const int sw = piece_swizzle(l16);
    const int roff0 = l16 * 8 + ((0 + G) ^ sw);
    const int roff1 = l16 * 8 + ((4 + G) ^ sw);
    struct Frags {
        bf16x8 w[WN / 16], x[WM / 16];
    };
    auto read = [&](Frags &f, int buf, int ro) __attribute__((always_inline)) {
        const u32x4 *S = &stg[buf].x[0][0];
        const u32x4 *Wp = &stg[buf].w[0][0];
#pragma unroll
        for (int i = 0; i < WN / 16; ++i)
            f.w[i] = __builtin_bit_cast(bf16x8, Wp[(wn * WN + 16 * i) * 8 + ro]);
#pragma unroll
        for (int j = 0; j < WM / 16; ++j)
            f.x[j] = __builtin_bit_cast(bf16x8, S[(wm * WM + 16 * j) * 8 + ro]);
    };
    // A half in WN / 16 chunks: chunk i runs the MFMAs of feature block i
    // with the reads of one W and two X fragments of the other register set
    // (and, in a second half, two of the copies of the stage after next)
    // placed before them, each chunk fenced, so reads and copies spread over
    // the half instead of leaving in one burst.
    static_assert(WM / 16 == 2 * (WN / 16) && CPW == 2 * (WN / 16), "chunk split");
    auto chunk_reads = [&](Frags &f, int b, int ro, int i) __attribute__((always_inline)) {
        const u32x4 *S = &stg[b].x[0][0];
        const u32x4 *Wp = &stg[b].w[0][0];
        f.w[i] = __builtin_bit_cast(bf16x8, Wp[(wn * WN + 16 * i) * 8 + ro]);
        f.x[2 * i] = __builtin_bit_cast(bf16x8, S[(wm * WM + 32 * i) * 8 + ro]);
        f.x[2 * i + 1] = __builtin_bit_cast(bf16x8, S[(wm * WM + 32 * i + 16) * 8 + ro]);
    };
    auto chunk_mfmas = [&](const Frags &f, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < WM / 16; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[i], f.x[j], acc[i][j], 0, 0, 0);
    };
    Frags fa, fb;
    int buf = 0;  // buffer of the current stage
    auto first_half = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WN / 16; ++i) {
            chunk_reads(fb, buf, roff1, i);
            chunk_mfmas(fa, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_copies<0>();
        stage_barrier();
    };
    auto second_half = [&]() __attribute__((always_inline)) {
        const int old = buf;
        buf ^= 1;
#pragma unroll
        for (int i = 0; i < WN / 16; ++i) {
            copy_one(old, 2 * i);
            copy_one(old, 2 * i + 1);
            chunk_reads(fa, buf, roff0, i);
            chunk_mfmas(fb, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        copy_advance();
    };

    copy_next(0);
    copy_next(1);
    wait_copies<CPW>();  // stage 0
    stage_barrier();
    read(fa, 0, roff0);
    for (int t = 0; t < ntl; ++t) {
#pragma unroll
        for (int i = 0; i < WN / 16; ++i)
#pragma unroll
            for (int j = 0; j < WM / 16; ++j)
                acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        // Second half: read the next stage's first half into `fa` (the next
        // tile's, after a tile's last stage) and run.  With K % 64 == 32 the
        // last stage's second half lies past K: its fragments (whatever the
        // bytes past K hold) are replaced by zeros, so it adds nothing.
        for (int st = 0; st < ns; ++st) {
            first_half();
            if constexpr (ODD) {
                const bool past_k = st == ns - 1;
#pragma unroll
                for (int i = 0; i < WN / 16; ++i)
                    fb.w[i] = past_k ? bf16x8{} : fb.w[i];
#pragma unroll
                for (int j = 0; j < WM / 16; ++j)
                    fb.x[j] = past_k ? bf16x8{} : fb.x[j];
            }
            second_half();
        }
        // Y^T block (i, j): lane holds features 4 G .. 4 G + 3 of token l16.
        const Tile tt = tile_of((int)blockIdx.x + t * grid, n_tm, n_tn);
#pragma unroll
        for (int j = 0; j < WM / 16; ++j) {
            const int m = tt.m0 + wm * WM + 16 * j + l16;
            if (m >= a.M)
                continue;
            uint16_t *yrow = a.y + (int64_t)m * a.ldy;
#pragma unroll
            for (int i = 0; i < WN / 16; ++i) {
                const int n = tt.n0 + wn * WN + 16 * i + 4 * G;
                if (n >= a.N)
                    continue;
                const f32x4 c = acc[i][j];
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                const bf16x4 h = __builtin_convertvector(c, bf16x4);
                *reinterpret_cast<u32x2 *>(yrow + n) = __builtin_bit_cast(u32x2, h);
            }
        }
    }
    wait_copies<0>();
}

}  // namespace

size_t proj_tiles(int M, int N) {
    return (size_t)((M + TM - 1) / TM) * (size_t)((N + TN - 1) / TN);
}

hipError_t launch_proj(const ProjArgs &a, hipStream_t stream) {
    ProjArgs args = a;
    void *params[] = {&args};
    // One workgroup per compute unit (the kernel's LDS allows one), a
    // multiple of 8 so that every workgroup stays on one XCD's tiles.
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const size_t tiles = proj_tiles(a.M, a.N);
    size_t g = tiles < (size_t)cus ? tiles : (size_t)cus;
    if (g >= 8)
        g -= g % 8;
    const dim3 grid((unsigned)(g > 0 ? g : 1));
    const void *fn = (a.K % 64) ? reinterpret_cast<const void *>(&parallax_proj_kernel<true>)
                                : reinterpret_cast<const void *>(&parallax_proj_kernel<false>);
    return hipLaunchKernel(fn, grid,
                           dim3(64 * PW), params, 0, stream);
}

}  // namespace plx
