// Internal launch interface between the C-ABI layer and the gfx950 kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

struct FwdArgs {
    const uint16_t *q, *k, *v, *r;  // bf16 bits, [B,H,L,d] with the strides below
    float *o;                       // [B,H,L,d] with o strides
    float *lse;                     // [B,H,L] contiguous
    int64_t q_b, q_h, q_l;
    int64_t k_b, k_h, k_l;
    int64_t v_b, v_h, v_l;
    int64_t r_b, r_h, r_l;
    int64_t o_b, o_h, o_l;
    int B, H, L;
    int n_qtiles;      // ceil(L / BM)
    float scale_log2;  // softmax_scale * log2(e), > 0
    int window;        // 0 = none
    int n_sink;
};

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

// Query rows per prefill workgroup.
constexpr int kFwdBlockM = 64;

hipError_t launch_fwd(const FwdArgs &a, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int d, int num_splits, hipStream_t stream);

}  // namespace plx
