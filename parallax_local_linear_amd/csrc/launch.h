// Internal launch interface between the C-ABI layer and the gfx950 kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace plx {

struct FwdArgs {
    const uint16_t *q, *k, *v, *r;  // bf16 bits, [B,H,L,d] with the strides below
    float *o;                       // [B,H,L,d] with o strides
    float *lse;                     // [B,H,L] contiguous
    float *sbar;                    // optional [B,H,L] contiguous: sum_j p_ij rho_i.k_j
    float *pv;                      // optional [B,H,L,d] contiguous: sum_j p_ij v_j
    uint16_t *vt;                   // workspace: f16 bits, [B*H][n_st][d][32] (see below)
    unsigned *counters;             // workspace after the image: [0] = query tiles recomputed
    int64_t q_b, q_h, q_l;
    int64_t k_b, k_h, k_l;
    int64_t v_b, v_h, v_l;
    int64_t r_b, r_h, r_l;
    int64_t o_b, o_h, o_l;
    int B, H, L;
    int n_qtiles;      // ceil(L / BM)
    int n_st;          // ceil(L / 32): 32-key stages per (batch, head)
    float scale_log2;  // softmax_scale * log2(e), > 0
    int window;        // 0 = none
    int n_sink;
    // Windowed kernel only (set by its launcher): 64-row tiles per (batch,
    // head), tiles per workgroup run, runs per (batch, head), workgroups
    // with work, and workgroups per XCD.
    int w_tiles, w_tpw, w_runs, w_blocks, w_per_xcd;
};

// Workspace layout: for each (batch, head) and each 32-key stage s, the
// values of keys 32s .. 32s+31 as float16, transposed to [d features][32
// positions] with the keys permuted as the prefill's value MFMA reads them
// (zeros for keys >= L).
// After the image, a block of counters: [0] counts the 128-row query tiles
// of the general kernel that took the exact second pass.
constexpr int kStageKeys = 32;
constexpr size_t kFwdCounterBytes = 256;
inline size_t fwd_image_bytes(int64_t B, int64_t H, int64_t L, int d) {
    return (size_t)(B * H * ((L + kStageKeys - 1) / kStageKeys) * kStageKeys * d * 2);
}
inline size_t fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d) {
    const size_t image = fwd_image_bytes(B, H, L, d);
    return image ? image + kFwdCounterBytes : 0;
}

// The prefill's windowed kernel takes windows of at most this many keys with
// at most kFwdWinSinkMax sinks; other masks use the general kernel.
constexpr int kFwdWinMax = 128;
constexpr int kFwdWinSinkMax = 32;
constexpr int64_t kFwdWinMaxRowStride = int64_t(1) << 20;

// Device memory the library owns for the prefill's workspace when the caller
// cannot allocate (parallax_attn_fwd_noalloc): one array of this many bytes
// per GPU, for the life of the process.
constexpr size_t kFwdScratchBytes = (size_t(64) << 20) + kFwdCounterBytes;
// Device address of the current GPU's array (looked up once per device).
hipError_t fwd_scratch(void **ptr);

struct DecodeArgs {
    const uint16_t *q, *r;          // bf16 [B,H,d] contiguous
    const uint16_t *k, *v;          // bf16 [B,H,Lmax,d] with strides
    const int32_t *seqlens;         // device [B] or nullptr
    float *o;                       // [B,H,d]
    float *lse;                     // [B,H]
    int64_t k_b, k_h, k_l;
    int64_t v_b, v_h, v_l;
    int B, H, Lmax;
    float scale_log2;
};

struct ProjArgs {
    const uint16_t *x;   // bf16 [M, K] with row stride ldx
    const uint16_t *w;   // bf16 [N, K] with row stride ldw
    uint16_t *y;         // bf16 [M, N] with row stride ldy
    int64_t ldx, ldw, ldy;
    int M, N, K;
};

struct HadArgs {
    const float *o;                 // fp32 [B, H, L, d], element strides below, d contiguous
    int64_t o_b, o_h, o_l;
    const float *alpha, *beta;      // fp32 [n] or nullptr (ones / zeros)
    uint16_t *y;                    // bf16 [B * L, n], row stride ldy; rows ordered (b, l)
    int64_t ldy;
    int M;                          // B * L (< 2^31)
    int L;
    int log2d;                      // feature index i reads head i >> log2d, feature i & (d - 1)
};

// Based linear attention (second-order Taylor kernel, 16 query/key
// features): prefill in 512-token segments, decode on a fixed-size state.
constexpr int kBasedSegment = 512;
constexpr int kBasedQueryTile = 256;  // queries per output workgroup
struct BasedArgs {
    const uint16_t *q, *k, *v;      // bf16 [B,H,L,16], [B,H,L,16], [B,H,L,dv]; strides below
    float *o;                       // fp32 [B,H,L,dv]
    int64_t q_b, q_h, q_l;
    int64_t k_b, k_h, k_l;
    int64_t v_b, v_h, v_l;
    int64_t o_b, o_h, o_l;
    int B, H, L;
    int n_seg;                      // ceil(L / kBasedSegment)
    int n_qt;                       // ceil(L / kBasedQueryTile): output workgroups per (batch, head)
    float scale;                    // x = scale * q.k
    float *dstate;                  // workspace: fp32 [B*H][n_seg][160][16 (dv/16 + 1)]
    uint16_t *sfrag;                // workspace: bf16 prefix-state fragments per segment
    float *state;                   // optional: fp32 [B*H][160][16 (dv/16 + 1)] final state
};

struct PagedDecodeArgs {
    const uint16_t *q, *r;          // bf16 [B,Hq,d] contiguous
    const uint16_t *k, *v;          // bf16 cache: element strides along page, kv head, row
    const int32_t *block_table;     // device [B][max_pages] page indices, or nullptr
    const int32_t *seqlens;         // device [B] or nullptr
    float *o;                       // [B,Hq,d]
    float *lse;                     // [B,Hq]
    int64_t k_p, k_h, k_l;
    int64_t v_p, v_h, v_l;
    int B, Hq, Hkv;
    int page_shift;                 // log2(page size) when paged
    int max_pages;                  // block-table row length when paged
    int num_pages;                  // pages in the pool (page indices are clamped into it)
    int max_len;                    // longest sequence the cache holds
    float scale_log2;
    int window, n_sink;
    // Grouped-head kernel only: the visible keys of each (sequence, kv head)
    // are split over `ksplit` workgroups (1: no split), whose partial states
    // go to `part` ([B*Hq][ksplit][2d+3] floats) for a merge launch.
    int ksplit;
    float *part;
};

// Most key splits of the grouped-head decode, and the workspace its partial
// states need: [B*Hq][splits][m, ell, S, A[d], C[d]] floats.
constexpr int kDecodeMaxKeySplits = 8;
inline size_t decode_paged_workspace_bytes(int64_t B, int64_t Hq, int d) {
    return (size_t)(B * Hq * kDecodeMaxKeySplits * (2 * d + 3)) * sizeof(float);
}

struct BwdArgs {
    const uint16_t *q, *k, *v, *r, *dout;  // bf16 bits, [B,H,L,d] with the strides below
    const float *o, *lse, *sbar, *pv;      // from the forward, contiguous
    float *dq, *dk, *dv, *dr;              // [B,H,L,d] contiguous
    float *stats;                          // workspace, see below
    uint16_t *kvrec;                       // workspace: key-kernel stage records
    uint16_t *qrec;                        // workspace: query-kernel stage records
    int64_t q_b, q_h, q_l;
    int64_t k_b, k_h, k_l;
    int64_t v_b, v_h, v_l;
    int64_t r_b, r_h, r_l;
    int64_t do_b, do_h, do_l;
    int B, H, L;
    int n_st;          // ceil(L / 32): 32-row stages per (batch, head)
    float scale;       // softmax scale
    int window;        // 0 = none
    int n_sink;
    // Key-block work split (see the backward kernels): key blocks below
    // n_sb hold sink keys; their rows past the window are cut into chunks
    // of kBwdChunk stages and added into dk and dv atomically.
    int n_sb;
    int n_chunks;
    int zero_rows;     // rows of dk and dv that the first kernel clears
};

// Backward workspace.  Per (batch, head) and 32-row stage s:
//   stats: float [4][32] -- lse*log2(e) (+inf for rows >= L), 1 - sbar,
//          G = dout.pv, G - dout.o
//   key-kernel record (the query side of the stage, as the key kernel's LDS
//          stage holds it): 1 KiB operand blocks, each block 64 lanes x 16
//          bytes in lane order --
//            row-major q, rho, dout: block (t, c) for rows 16t + (l % 16),
//              features 32c + 8 (l / 16) .. +7          (2 * d/32 blocks each)
//   query-kernel record (the key side of the stage): row-major k and v in
//          the same block format.
//   The kernels read the transposed operands they need out of these
//   blocks with LDS transpose reads.
// Rows >= L are zeros.
constexpr int kBwdChunk = 16;
__host__ __device__ inline size_t bwd_stats_bytes(int64_t BH, int64_t n_st) {
    return (size_t)(BH * n_st * 128 * 4);
}
__host__ __device__ constexpr size_t bwd_kv_record_bytes(int d) { return (size_t)3 * kStageKeys * d * 2; }
__host__ __device__ constexpr size_t bwd_q_record_bytes(int d) { return (size_t)2 * kStageKeys * d * 2; }
inline size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d) {
    const int64_t n_st = (L + kStageKeys - 1) / kStageKeys;
    return bwd_stats_bytes(B * H, n_st) +
           (size_t)(B * H * n_st) * (bwd_kv_record_bytes(d) + bwd_q_record_bytes(d));
}

// Prefill workgroup shape: 8 wavefronts of 16 query rows for either feature
// dimension.
constexpr int fwd_waves(int) { return 8; }
constexpr int fwd_block_rows(int d) { return 16 * fwd_waves(d); }

hipError_t launch_fwd(const FwdArgs &a, int d, bool precise, hipStream_t stream);

// fp32 prefill (parallax_attn_fwd_f32): fp32 tensors, element strides.
struct F32Args {
    const float *q, *k, *v, *r;
    float *o, *lse;
    int64_t q_b, q_h, q_l, k_b, k_h, k_l, v_b, v_h, v_l, r_b, r_h, r_l, o_b, o_h, o_l;
    int B, H, L;
    float scale;
    int window, n_sink;
};
hipError_t launch_fwd_f32(const F32Args &a, int d, hipStream_t stream);
int64_t fwd_f32_blocks(int B, int H, int L);
hipError_t launch_bwd(const BwdArgs &a, int d, hipStream_t stream);
hipError_t launch_proj(const ProjArgs &a, hipStream_t stream);
hipError_t launch_hadamard(const HadArgs &a, int log2n, hipStream_t stream);
hipError_t launch_based_fwd(const BasedArgs &a, int dv, hipStream_t stream);
hipError_t launch_based_decode(const BasedArgs &a, int dv, hipStream_t stream);
size_t based_workspace_bytes(int64_t B, int64_t H, int64_t L, int dv);
size_t based_state_floats(int dv);
int64_t hadamard_blocks(int64_t M, int log2n);
size_t proj_tiles(int M, int N);
hipError_t launch_decode(const DecodeArgs &a, int d, int num_splits, hipStream_t stream);
hipError_t launch_decode_paged(const PagedDecodeArgs &a, int d, int num_splits, hipStream_t stream);

}  // namespace plx
