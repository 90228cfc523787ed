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

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16x128 MFMA on fp4 (E2M1) operands, fp32 accumulate, no block scaling.  Lane (row r,
// group g) holds k = 32g .. 32g+31 of its row as four dwords of eight 4-bit codes: dword i,
// nibble j is k = 32g + 8i + j (the upper half of the 8-dword operand is unused for fp4).
__device__ __forceinline__ v4f mfma_f4(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0},
                                                           v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0}, c, 4, 4, 0,
                                                           0, 0, 0);
}

// E2M1 codes used as exact small integers: 1.0 = 0x2, 2.0 = 0x4, -2.0 = 0xC.
// A lane's 32 channels are laid out with channel 4j + i of its 32-bit sign word in dword i,
// nibble j.  The order inside the operand is immaterial to the dot product as long as both MFMA
// operands use the same one, and this one moves every bit with one shift and one mask: bit
// 4j + i sits at bit i of nibble j already.
// 32 sign bits -> 32 fp4 values {0, 1.0} (bit set: 1.0): code bit 1 of each nibble.
__device__ __forceinline__ void unpack_bits32_f4(uint32_t w, uint32_t out[4]) {
    out[0] = (w << 1) & 0x22222222u;
    out[1] = w & 0x22222222u;
    out[2] = (w >> 1) & 0x22222222u;
    out[3] = (w >> 2) & 0x22222222u;
}

// 32 sign bits -> 32 fp4 values {+2.0, -2.0} (bit set: +2.0; 0xC ^ 0x8 = 0x4), same order.
__device__ __forceinline__ void unpack_signs32_f4x2(uint32_t w, uint32_t out[4]) {
    out[0] = 0xCCCCCCCCu ^ ((w << 3) & 0x88888888u);
    out[1] = 0xCCCCCCCCu ^ ((w << 2) & 0x88888888u);
    out[2] = 0xCCCCCCCCu ^ ((w << 1) & 0x88888888u);
    out[3] = 0xCCCCCCCCu ^ (w & 0x88888888u);
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
