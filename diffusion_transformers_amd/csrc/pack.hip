// pack.hip -- sign bits and per-token scale of Q or K.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 1 (Scaled Binary
// Representations): each channel keeps only its sign, and a per-token scale mu
// keeps the magnitude.  mu is taken as mean |x| over the d channels.
//
// HBM-bound: a token is read once (2d or 4d bytes) and 4*ceil(d/32) + 4 bytes are
// written.  A workgroup owns T = floor(256 / (d/8)) consecutive tokens -- a
// contiguous span of memory -- and each thread loads one 8-channel chunk of it, so
// every load instruction is contiguous and the launch has enough waves to hide
// memory latency.  Per chunk a thread forms one byte of sign bits and a partial
// |x| sum; the bytes and partial sums meet in LDS, where thread t assembles token
// t's words and mu in channel order.
#include "common.h"
#include "internal.h"
#include "prep.h"

namespace binattn {

template <typename T>
__global__ __launch_bounds__(256) void pack_qk_kernel(const T* __restrict__ x, int64_t ntok, int d, int W,
                                                      uint32_t* __restrict__ bits, float* __restrict__ mu) {
    __shared__ __attribute__((aligned(16))) uint8_t sBits[256 * 16];  // 16 sign bytes per token
    __shared__ float sSum[256];                                        // partial |x| sum per chunk
    pack_block<T>(x, ntok, d, W, bits, mu, blockIdx.x, sBits, sSum);
}

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s) {
    const int W = (d + 31) / 32;
    const dim3 block(256), grid((unsigned)pack_blocks<float>(ntok, d));
    if (f32)
        hipLaunchKernelGGL(pack_qk_kernel<float>, grid, block, 0, s, (const float*)x, ntok, d, W, bits, mu);
    else
        hipLaunchKernelGGL(pack_qk_kernel<_Float16>, grid, block, 0, s, (const _Float16*)x, ntok, d, W, bits, mu);
    return hipGetLastError();
}

}  // namespace binattn
