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

namespace binattn {

template <typename T>
__global__ __launch_bounds__(256) void pack_qk_kernel(const T* __restrict__ x, int64_t ntok, int d, int W,
                                                      uint32_t* __restrict__ bits, float* __restrict__ mu) {
    typedef T vec8 __attribute__((ext_vector_type(8)));  // one chunk: 8 channels
    __shared__ __attribute__((aligned(16))) uint8_t sBits[256 * 16];  // 16 sign bytes per token
    __shared__ float sSum[256];                                        // partial |x| sum per chunk
    const int tid = threadIdx.x;
    const int cpt = d >> 3;                               // chunks per token
    const int ntw = 256 / cpt;                            // tokens per workgroup
    const int64_t t0 = (int64_t)blockIdx.x * ntw;
    const int t = tid / cpt, part = tid - t * cpt;
    const int64_t tok = t0 + t;
    uint32_t byte = 0;
    float sum = 0.0f;
    if (t < ntw && tok < ntok) {
        const vec8 v = *reinterpret_cast<const vec8*>(x + tok * d + 8 * part);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = (float)v[e];
            byte |= (f >= 0.0f ? 1u : 0u) << e;  // -0.0 >= 0 holds: zero counts as +1
            sum += fabsf(f);
        }
    }
    // bytes past the token's d channels read as zero
    reinterpret_cast<uint4*>(sBits)[tid] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    if (t < ntw) {
        sBits[t * 16 + part] = (uint8_t)byte;
        sSum[tid] = sum;  // tid == t * cpt + part
    }
    __syncthreads();
    if (tid < ntw && t0 + tid < ntok) {
        const int64_t o = t0 + tid;
        const uint4 w = reinterpret_cast<const uint4*>(sBits)[tid];
        uint32_t* out = bits + o * W;
        out[0] = w.x;
        if (W > 1) out[1] = w.y;
        if (W > 2) out[2] = w.z;
        if (W > 3) out[3] = w.w;
        float acc = 0.0f;
        for (int p = 0; p < cpt; ++p) acc += sSum[tid * cpt + p];
        mu[o] = acc / (float)d;
    }
}

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s) {
    const int W = (d + 31) / 32;
    const int T = 256 / (d / 8);
    const dim3 block(256), grid((unsigned)((ntok + T - 1) / T));
    if (f32)
        hipLaunchKernelGGL(pack_qk_kernel<float>, grid, block, 0, s, (const float*)x, ntok, d, W, bits, mu);
    else
        hipLaunchKernelGGL(pack_qk_kernel<_Float16>, grid, block, 0, s, (const _Float16*)x, ntok, d, W, bits, mu);
    return hipGetLastError();
}

}  // namespace binattn
