// Walsh-Hadamard output projection for gfx950:
//     y = alpha (.) (O H_n / sqrt(n)) + beta
// with O the attention output of one token, its H heads of d features
// concatenated (n = H d, a power of two), H_n the Sylvester-ordered Hadamard
// matrix and alpha, beta per-feature vectors (review page "Rethinking
// Attention Output Projection: Structured Hadamard Transforms for Efficient
// Transformers", sec. 2 "Methodology": a fixed, parameter-free transform and
// a learned affine rescaling in place of the dense output projection).
//
// H_n is the n-fold Kronecker product of [[1, 1], [1, -1]], so the transform
// is a butterfly (a + b, a - b) along each of the log2(n) bits of the
// feature index, in any order: n log2(n) additions, no multiplications.
//
// Mapping onto CDNA4 (the kernel is bound by HBM: 4 bytes read and 2 bytes
// written per feature):
//   * Each lane holds 64 features of one token; a token spans P = n / 64
//     lanes and a wavefront holds 64 / P tokens.  Lane p of a token loads
//     16-byte chunks c = 0..15 at features 4 P c + 4 p .. +3, straight from
//     the [B, H, L, d] attention output (no concatenation pass), so the 6
//     feature bits {0, 1} and the top 4 are in registers: 6 butterfly
//     stages run in registers.
//   * The other log2(n) - 6 bits (2 .. log2(P) + 1) are brought into
//     registers by one transpose through LDS, their butterflies run in
//     registers, and the values go back through LDS to the load layout,
//     from which each lane stores 4 bf16 (8 bytes) per chunk, contiguous
//     across the lanes of a token.
//   * LDS rows are padded by 4 floats after every chunk and by P floats per
//     token, which makes the transposed reads free of bank conflicts.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace plx {
namespace {

constexpr int HW = 1;  // wavefronts per workgroup (one: the most workgroups in flight per CU)

template <int LOGN>
struct HadShape {
    static constexpr int N = 1 << LOGN;
    static constexpr int LOGP = LOGN - 6;
    static constexpr int P = 1 << LOGP;         // lanes per token
    static constexpr int RW = 64 / P;           // tokens per wavefront
    static constexpr int CH = 4 * P;            // features per chunk
    static constexpr int RS = N + 64 + P;       // LDS floats per token
    static_assert(LOGN >= 8 && LOGN <= 12, "n in [256, 4096]");
};

// Position of feature i of a token in its padded LDS row.
template <int LOGN>
__device__ __forceinline__ int had_pos(int i) {
    return i + 4 * (i >> (HadShape<LOGN>::LOGP + 2));
}

template <int LOGN, int LOG2D>
__global__ __launch_bounds__(64 * HW) void parallax_hadamard_kernel(HadArgs a) {
    using S = HadShape<LOGN>;
    constexpr int D = 1 << LOG2D;
    __shared__ float lds[HW][S::RW * S::RS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rr = lane >> S::LOGP;         // token within the wavefront
    const int p = lane & (S::P - 1);        // lane within the token
    const int m = (blockIdx.x * HW + wave) * S::RW + rr;  // B * L < 2^31 (host check)
    const bool live = m < a.M;
    float *row = &lds[wave][rr * S::RS];

    // Load: chunk c holds features 4 P c + 4 p + j, j = 0..3.  Tokens past
    // the end read the last token (in bounds) and store nothing.  The lane's
    // part of the address is formed once; each chunk adds a uniform offset.
    float x[64];
    {
        const int ml = live ? m : a.M - 1;
        const int b = ml / a.L, l = ml - b * a.L;
        const int i0 = 4 * p;
        const float *src = a.o + (int64_t)b * a.o_b + (int64_t)l * a.o_l;
        src += S::CH >= D ? (int64_t)(i0 >> LOG2D) * a.o_h + (i0 & (D - 1)) : i0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int64_t off = S::CH >= D
                                    ? (int64_t)(c * (S::CH / D)) * a.o_h
                                    : (int64_t)((S::CH * c) >> LOG2D) * a.o_h +
                                          ((S::CH * c) & (D - 1));
            const f32x4 v =
                __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + off));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[4 * c + j] = v[j];
        }
    }

    // Butterflies over the register bits (feature bits 0, 1 and the top 4).
#pragma unroll
    for (int s = 0; s < 6; ++s)
#pragma unroll
        for (int r = 0; r < 64; ++r)
            if (!(r & (1 << s))) {
                const float u = x[r], w = x[r | (1 << s)];
                x[r] = u + w;
                x[r | (1 << s)] = u - w;
            }

    // Transpose through LDS: register g * P + u holds feature
    // j + 4 u + CH c with (j, c) taken from wbits = p + P g.
#pragma unroll
    for (int c = 0; c < 16; ++c)
        *reinterpret_cast<f32x4 *>(row + had_pos<LOGN>(S::CH * c + 4 * p)) =
            (f32x4){x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
    __syncthreads();
#pragma unroll
    for (int g = 0; g < S::RW; ++g) {
        const int wbits = p + S::P * g;
        const int base = (wbits & 3) + S::CH * (wbits >> 2);
#pragma unroll
        for (int u = 0; u < S::P; ++u)
            x[g * S::P + u] = row[had_pos<LOGN>(base + 4 * u)];
    }

    // Butterflies over the remaining bits (feature bits 2 .. LOGP + 1).
#pragma unroll
    for (int s = 0; s < S::LOGP; ++s)
#pragma unroll
        for (int r = 0; r < 64; ++r)
            if (!(r & (1 << s))) {
                const float u = x[r], w = x[r | (1 << s)];
                x[r] = u + w;
                x[r | (1 << s)] = u - w;
            }

    // Back to the load layout.  Each lane rewrites exactly the positions it
    // read, so only the reads of the next step need the barrier.
#pragma unroll
    for (int g = 0; g < S::RW; ++g) {
        const int wbits = p + S::P * g;
        const int base = (wbits & 3) + S::CH * (wbits >> 2);
#pragma unroll
        for (int u = 0; u < S::P; ++u)
            row[had_pos<LOGN>(base + 4 * u)] = x[g * S::P + u];
    }
    __syncthreads();
    if (!live)
        return;

    // Normalise, rescale, round to bf16 and store 8 bytes per chunk (one
    // copy of the loop per presence of alpha and beta, chosen uniformly).
    const float norm = __builtin_sqrtf(1.0f / (float)S::N);
    uint16_t *dst = a.y + (int64_t)m * a.ldy;
    auto epilogue = [&](auto has_alpha, auto has_beta) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int i = S::CH * c + 4 * p;
            f32x4 t = *reinterpret_cast<const f32x4 *>(row + had_pos<LOGN>(i));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                t[j] *= norm;
            if constexpr (decltype(has_alpha)::value) {
                const f32x4 al = *reinterpret_cast<const f32x4 *>(a.alpha + i);
                if constexpr (decltype(has_beta)::value) {
                    const f32x4 be = *reinterpret_cast<const f32x4 *>(a.beta + i);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        t[j] = __builtin_fmaf(t[j], al[j], be[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        t[j] *= al[j];
                }
            } else if constexpr (decltype(has_beta)::value) {
                const f32x4 be = *reinterpret_cast<const f32x4 *>(a.beta + i);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    t[j] += be[j];
            }
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
            const bf16x4 h = __builtin_convertvector(t, bf16x4);
            __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h),
                                        reinterpret_cast<u32x2 *>(dst + i));
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    if (a.alpha) {
        if (a.beta)
            epilogue(T{}, T{});
        else
            epilogue(T{}, F{});
    } else {
        if (a.beta)
            epilogue(F{}, T{});
        else
            epilogue(F{}, F{});
    }
}

template <int LOGN>
hipError_t launch_hadamard_t(const HadArgs &a, hipStream_t stream) {
    using S = HadShape<LOGN>;
    HadArgs args = a;
    void *params[] = {&args};
    const int64_t rows_per_block = (int64_t)HW * S::RW;
    const dim3 grid((unsigned)((a.M + rows_per_block - 1) / rows_per_block));
    const void *k = a.log2d == 6
                        ? reinterpret_cast<const void *>(&parallax_hadamard_kernel<LOGN, 6>)
                        : reinterpret_cast<const void *>(&parallax_hadamard_kernel<LOGN, 7>);
    return hipLaunchKernel(k, grid, dim3(64 * HW), params, 0, stream);
}

}  // namespace

int64_t hadamard_blocks(int64_t M, int log2n) {
    const int64_t rows_per_block = (int64_t)HW * (64 >> (log2n - 6));
    return (M + rows_per_block - 1) / rows_per_block;
}

hipError_t launch_hadamard(const HadArgs &a, int log2n, hipStream_t stream) {
    switch (log2n) {
    case 8: return launch_hadamard_t<8>(a, stream);
    case 9: return launch_hadamard_t<9>(a, stream);
    case 10: return launch_hadamard_t<10>(a, stream);
    case 11: return launch_hadamard_t<11>(a, stream);
    case 12: return launch_hadamard_t<12>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace plx
