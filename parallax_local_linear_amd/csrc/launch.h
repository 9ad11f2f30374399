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
    uint16_t *vt;                   // workspace: f16 bits, [B*H][n_st][d][32] (see below)
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
};

// Workspace layout: for each (batch, head) and each 32-key stage s, the
// values of keys 32s .. 32s+31 as float16, transposed to [d features][32
// positions] with the keys permuted as the prefill's value MFMA reads them
// (zeros for keys >= L).
constexpr int kStageKeys = 32;
inline size_t fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d) {
    return (size_t)(B * H * ((L + kStageKeys - 1) / kStageKeys) * kStageKeys * d * 2);
}

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

// Prefill workgroup shape: 8 wavefronts of 16 query rows for either feature
// dimension.
constexpr int fwd_waves(int) { return 8; }
constexpr int fwd_block_rows(int d) { return 16 * fwd_waves(d); }

hipError_t launch_fwd(const FwdArgs &a, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int d, int num_splits, hipStream_t stream);

}  // namespace plx
