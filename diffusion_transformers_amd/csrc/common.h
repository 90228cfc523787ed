// common.h -- device helpers shared by the BinaryAttention HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace binattn {

typedef int v4i __attribute__((ext_vector_type(4)));
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

// 16 sign bits (bit k = channel k, 1 = non-negative) -> 16 int8 values in four dwords,
// byte k = +1 (0x01) or -1 (0xFF).  The nibble multiply spreads bit k to bit 8k.
__device__ __forceinline__ void unpack_signs16(uint32_t bits16, uint32_t out[4]) {
    const uint32_t nb = ~bits16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t nib = (nb >> (4 * q)) & 0xFu;
        const uint32_t neg = (nib * 0x00204081u) & 0x01010101u;  // byte k = 1 where channel is negative
        out[q] = neg * 0xFEu + 0x01010101u;                      // 0x01 -> +1, 0xFF -> -1
    }
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace binattn
