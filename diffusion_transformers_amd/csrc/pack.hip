// pack.hip -- sign bits and per-token scale of Q or K.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 1 (Scaled Binary
// Representations): each channel keeps only its sign, and a per-token scale mu
// keeps the magnitude.  mu is taken as mean |x| over the d channels.
//
// HBM-bound: a token is read once (2d or 4d bytes) and 4*ceil(d/32) + 4 bytes are
// written.  One thread per token, 16-byte vector loads; within one load
// instruction the lanes stride by one token row, and the row's remaining bytes
// are consumed by the following loads while the line is still in cache.
#include "common.h"
#include "internal.h"

namespace binattn {

template <typename T>
__global__ __launch_bounds__(256) void pack_qk_kernel(const T* __restrict__ x, int64_t ntok, int d, int W,
                                                      uint32_t* __restrict__ bits, float* __restrict__ mu) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ntok) return;
    constexpr int VE = 16 / sizeof(T);  // elements per 16-byte load (8 halves or 4 floats)
    typedef T vecT __attribute__((ext_vector_type(VE)));
    const T* row = x + t * d;
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    float sum = 0.0f;
    for (int c0 = 0; c0 < d; c0 += VE) {
        const vecT v = *reinterpret_cast<const vecT*>(row + c0);
        uint32_t part = 0;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float f = (float)v[e];
            part |= (f >= 0.0f ? 1u : 0u) << e;  // -0.0 >= 0 holds: zero counts as +1
            sum += fabsf(f);
        }
        const uint32_t sh = part << (c0 & 31);
        const int wi = c0 >> 5;
        w0 |= wi == 0 ? sh : 0u;
        w1 |= wi == 1 ? sh : 0u;
        w2 |= wi == 2 ? sh : 0u;
        w3 |= wi == 3 ? sh : 0u;
    }
    uint32_t* out = bits + t * W;
    out[0] = w0;
    if (W > 1) out[1] = w1;
    if (W > 2) out[2] = w2;
    if (W > 3) out[3] = w3;
    mu[t] = sum / (float)d;
}

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s) {
    const int W = (d + 31) / 32;
    const dim3 block(256), grid((unsigned)((ntok + 255) / 256));
    if (f32)
        hipLaunchKernelGGL(pack_qk_kernel<float>, grid, block, 0, s, (const float*)x, ntok, d, W, bits, mu);
    else
        hipLaunchKernelGGL(pack_qk_kernel<_Float16>, grid, block, 0, s, (const _Float16*)x, ntok, d, W, bits, mu);
    return hipGetLastError();
}

}  // namespace binattn
