// Parallax prefill forward in fp32 throughout, for fp32 inputs.
//
// The same operation as the matrix-core prefill (review page "Parallax:
// Parameterized Local Linear Attention for Language Modeling", sec. 1 and
// sec. 3): for query i and its visible keys j (causal, optional window and
// sinks, "Sliding-window beats linear attention" review, sec. 1)
//
//     p_ij = softmax_j(scale q_i.k_j),  s_ij = rho_i.k_j,
//     o_i  = sum_j p_ij (1 + s_ij - sbar_i) v_j,   sbar_i = sum_j p_ij s_ij,
//     lse_i = log sum_j exp(scale q_i.k_j),
//
// but with every product, exponential and sum in fp32 (expf, logf), so
// that fp32 inputs are not rounded to bfloat16 first.  It is untiled, with
// O(L^2 d) work per head: meant for small problems (the tiny reference
// workload), where the bf16 path's input rounding is the larger error.
//
// One wavefront per query row:
//   1. lanes take the visible keys 64 at a time, one key per lane, and form
//      its score q.k in fp32; the row max m comes from a wavefront max;
//   2. over the same chunks each lane forms p = exp(scale q.k - m) and
//      w = p rho.k for its key; the lanes then walk the chunk's keys with
//      the key's p and w broadcast, each lane accumulating A = sum p v and
//      C = sum w v for its features (feature f = lane + 64 t), while
//      l = sum p and S = sum w are summed per lane and reduced at the end;
//   3. o = (A (1 - S / l) + C) / l, lse = m + log l.
#include "device_common.h"
#include "launch.h"

namespace plx {
namespace {

constexpr int F32_WAVES = 4;  // query rows per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(64 * F32_WAVES) void parallax_fwd_f32_kernel(F32Args a) {
    constexpr int FT = D / 64;  // features per lane
    __shared__ float qs[F32_WAVES][D], rs[F32_WAVES][D];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rows_per_bh = (a.L + F32_WAVES - 1) / F32_WAVES;
    const int bh = blockIdx.x / rows_per_bh;
    const int i = (blockIdx.x - bh * rows_per_bh) * F32_WAVES + wave;
    const int b = bh / a.H, h = bh - b * a.H;
    const float *qb = a.q + b * a.q_b + h * a.q_h;
    const float *kb = a.k + b * a.k_b + h * a.k_h;
    const float *vb = a.v + b * a.v_b + h * a.v_h;
    const float *rb = a.r + b * a.r_b + h * a.r_h;
    const bool live = i < a.L;
    if (live) {
#pragma unroll
        for (int t = 0; t < FT; ++t) {
            qs[wave][lane + 64 * t] = qb[(int64_t)i * a.q_l + lane + 64 * t];
            rs[wave][lane + 64 * t] = rb[(int64_t)i * a.r_l + lane + 64 * t];
        }
    }
    __syncthreads();
    if (!live)
        return;

    // Visible keys: the sinks below the window, then [lo, i].
    int lo = 0, ns = 0;
    if (a.window > 0) {
        lo = i - a.window + 1 > 0 ? i - a.window + 1 : 0;
        ns = a.n_sink < lo ? a.n_sink : lo;
    }
    const int nvis = ns + (i - lo + 1);
    auto key = [&](int u) { return u < ns ? u : lo + (u - ns); };

    // Scores of key j with q and rho.
    auto dots = [&](int j, float &sq, float &sr) {
        const float *kr = kb + (int64_t)j * a.k_l;
        float x = 0.f, y = 0.f;
#pragma unroll 8
        for (int f = 0; f < D; ++f) {
            const float kv = kr[f];
            x = fmaf(qs[wave][f], kv, x);
            y = fmaf(rs[wave][f], kv, y);
        }
        sq = x * a.scale;
        sr = y;
    };

    float m = -__builtin_inff();
    for (int u0 = 0; u0 < nvis; u0 += 64) {
        const int u = u0 + lane;
        if (u < nvis) {
            float sq, sr;
            dots(key(u), sq, sr);
            m = fmaxf(m, sq);
        }
    }
    m = wave_max(m);

    float ell = 0.f, ssum = 0.f;
    float acc_a[FT], acc_c[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t)
        acc_a[t] = acc_c[t] = 0.f;
    for (int u0 = 0; u0 < nvis; u0 += 64) {
        const int u = u0 + lane;
        float p = 0.f, w = 0.f;
        if (u < nvis) {
            float sq, sr;
            dots(key(u), sq, sr);
            p = expf(sq - m);
            w = p * sr;
        }
        ell += p;
        ssum += w;
        const int cnt = nvis - u0 < 64 ? nvis - u0 : 64;
        for (int kk = 0; kk < cnt; ++kk) {
            const float pk = __shfl(p, kk, 64);
            const float wk = __shfl(w, kk, 64);
            const float *vr = vb + (int64_t)key(u0 + kk) * a.v_l;
#pragma unroll
            for (int t = 0; t < FT; ++t) {
                const float vv = vr[lane + 64 * t];
                acc_a[t] = fmaf(pk, vv, acc_a[t]);
                acc_c[t] = fmaf(wk, vv, acc_c[t]);
            }
        }
    }
    ell = wave_sum(ell);
    ssum = wave_sum(ssum);
    const float inv = 1.f / ell;
    const float keep = 1.f - ssum * inv;
    float *orow = a.o + b * a.o_b + h * a.o_h + (int64_t)i * a.o_l;
#pragma unroll
    for (int t = 0; t < FT; ++t)
        orow[lane + 64 * t] = (acc_a[t] * keep + acc_c[t]) * inv;
    if (lane == 0)
        a.lse[(int64_t)bh * a.L + i] = m + logf(ell);
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args &a, int d, hipStream_t stream) {
    F32Args args = a;
    void *params[] = {&args};
    const int64_t blocks = (int64_t)a.B * a.H * ((a.L + F32_WAVES - 1) / F32_WAVES);
    const void *fn = d == 64 ? reinterpret_cast<const void *>(&parallax_fwd_f32_kernel<64>)
                             : reinterpret_cast<const void *>(&parallax_fwd_f32_kernel<128>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * F32_WAVES), params, 0, stream);
}

int64_t fwd_f32_blocks(int B, int H, int L) {
    return (int64_t)B * H * ((L + F32_WAVES - 1) / F32_WAVES);
}

}  // namespace plx
