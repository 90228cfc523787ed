// common.h -- device helpers shared by the BinaryAttention HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace binattn {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Workgroups are handed to the eight XCDs round-robin (block b runs on XCD b % 8).
// Give XCD x one contiguous range of logical block ids instead, so that blocks that
// share inputs (same head, or same bias slice) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nblk) {
    const int xcd = b & 7, slot = b >> 3;
    const int full = nblk >> 3, rem = nblk & 7;
    return xcd < rem ? xcd * (full + 1) + slot : rem * (full + 1) + (xcd - rem) * full + slot;
}

// Four bits (bit k = channel k) -> four bytes 0/1 (byte k = bit k).  The multiply by
// 0x204081 = 1 + 2^7 + 2^14 + 2^21 moves bit k to bit 8k without carries.
__device__ __forceinline__ uint32_t spread4(uint32_t nib) { return (nib * 0x00204081u) & 0x01010101u; }

// 16 sign bits -> 16 int8 values {0, 1} in four dwords (byte k = bit k).
__device__ __forceinline__ void unpack_bits16(uint32_t bits16, uint32_t out[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = spread4((bits16 >> (4 * q)) & 0xFu);
}

// 16 sign bits -> 16 int8 values {+2, -2} in four dwords (0x02 where the bit is set, 0xFE where clear).
__device__ __forceinline__ void unpack_signs16_x2(uint32_t bits16, uint32_t out[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = spread4((~bits16 >> (4 * q)) & 0xFu) * 0xFCu + 0x02020202u;
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16x128 MFMA on fp8 (E4M3) operands, fp32 accumulate, no block scaling.
__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// fp8 E4M3 encodings used as exact small integers: 1.0, 2.0 and -2.0.
constexpr uint32_t kF8One = 0x38u, kF8Two = 0x40u, kF8MinusTwo = 0xC0u;

// 32 sign bits -> 32 fp8 values {0, 1.0} (byte k = bit k ? 1.0 : 0), eight dwords.
__device__ __forceinline__ void unpack_bits32_f8(uint32_t w, uint32_t out[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = __builtin_amdgcn_perm(0u, kF8One << 8, spread4((w >> (4 * q)) & 0xFu));
}

// 32 sign bits -> 32 fp8 values {+2.0, -2.0} (byte k = bit k ? 2.0 : -2.0), eight dwords.
__device__ __forceinline__ void unpack_signs32_f8x2(uint32_t w, uint32_t out[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
        out[q] = __builtin_amdgcn_perm(0u, (kF8MinusTwo << 8) | kF8Two, spread4((~w >> (4 * q)) & 0xFu));
}

// Raw buffer resource over [base, base + bytes): loads past the end read as zero.
// bytes is a per-head or per-wave extent, always far below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}

// A wave-uniform zero the compiler cannot see through (an s_mov in inline asm), for offsets
// that must keep a load inside its loop.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), with the
// gfx950 row-swap permutes: after the 32-swap each lane sees rows {r, r^2}, after the
// 16-swap all four.
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace binattn
