// Device-side types and helpers shared by the gfx950 Parallax kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 16-byte global load of 8 bf16 values (raw bits).
__device__ __forceinline__ u32x4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Buffer resource over [base, base + nbytes): loads at or past nbytes return
// zeros, so no lane ever reads outside that range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                             0x00020000);
}

// 16-byte buffer load at a per-lane byte offset.
__device__ __forceinline__ u32x4 bufld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// Bytes from the start of row j0 through the last element of row L-1 of a
// [rows, d] slice with row stride `ld` elements (2-byte elements), clamped
// to the 32-bit range of a buffer resource (0 when j0 is past the end).
__device__ __forceinline__ uint32_t rows_bytes(int j0, int L, int64_t ld, int d) {
    const int64_t rows = (int64_t)L - 1 - j0;
    const uint64_t n = (uint64_t)(rows < 0 ? 0 : rows) * (uint64_t)ld * 2u + (uint64_t)d * 2u;
    const uint64_t clamped = n < 0xffffffffull ? n : 0xffffffffull;
    return rows < 0 ? 0u : (uint32_t)clamped;
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed f16x2, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x2 cvt_f16x2(float a, float b) {
    return __builtin_convertvector((f32x2){a, b}, f16x2);
}

// 2^x on the hardware exp unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ 32): the other half-wave.
__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

}  // namespace plx
