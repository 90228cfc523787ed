// pack.hip -- sign bits and per-token scale of Q or K.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 1 (Scaled Binary
// Representations): each channel keeps only its sign, and a per-token scale mu
// keeps the magnitude.  mu is taken as mean |x| over the d channels.
//
// HBM-bound: a token is read once (2d or 4d bytes) and 4*ceil(d/32) + 4 bytes are
// written.  One thread per token: its 16-byte chunks are loaded together (the 64 lanes of a
// wave cover 64 consecutive tokens, so the loads of one wave cover one contiguous span), the
// sign words and mu are formed in registers and stored directly -- no LDS, no barrier.
#include "common.h"
#include "internal.h"
#include "prep.h"

namespace binattn {

template <typename T>
__global__ __launch_bounds__(256) void pack_qk_kernel(const T* __restrict__ x, int64_t ntok, int d, int W,
                                                      uint32_t* __restrict__ bits, float* __restrict__ mu) {
    pack_wave<T>(x, ntok, d, W, bits, mu, (int64_t)blockIdx.x);
}

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s) {
    const int W = (d + 31) / 32;
    const dim3 block(256), grid((unsigned)pack_blocks(ntok));
    if (f32)
        hipLaunchKernelGGL(pack_qk_kernel<float>, grid, block, 0, s, (const float*)x, ntok, d, W, bits, mu);
    else
        hipLaunchKernelGGL(pack_qk_kernel<_Float16>, grid, block, 0, s, (const _Float16*)x, ntok, d, W, bits, mu);
    return hipGetLastError();
}

}  // namespace binattn
