// pack.hip -- sign bits and per-token scale of Q or K.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 1 (Scaled Binary
// Representations): each channel keeps only its sign, and a per-token scale mu
// keeps the magnitude.  mu is taken as mean |x| over the d channels.
//
// HBM-bound: a token is read once (2d or 4d bytes) and 4*ceil(d/32) + 4 bytes are
// written.  A wave owns 64 consecutive tokens, a contiguous span of memory, and
// reads it in 8-channel chunks with lane i taking chunk i (+64, +128, ...), so each
// load instruction covers one contiguous kilobyte (fp16).  Per chunk a lane forms
// one byte of sign bits and a partial |x| sum; the bytes and partial sums meet in
// LDS, where lane t assembles token t's words and mu in channel order.
#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kPackTok = 64;  // tokens per wave

template <typename T>
__global__ __launch_bounds__(256) void pack_qk_kernel(const T* __restrict__ x, int64_t ntok, int d, int W,
                                                      uint32_t* __restrict__ bits, float* __restrict__ mu) {
    typedef T vec8 __attribute__((ext_vector_type(8)));  // one chunk: 8 channels
    constexpr int MAXC = 16;                              // chunks of the largest token (d = 128)
    __shared__ __attribute__((aligned(16))) uint8_t sBits[4][kPackTok * 16];
    __shared__ float sSum[4][kPackTok * MAXC];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t0 = ((int64_t)blockIdx.x * 4 + wave) * kPackTok;  // first token of this wave
    const int cpt = d >> 3;                                           // chunks per token
    const uint32_t magic = ((1u << 20) + cpt - 1) / cpt;              // ceil(2^20 / cpt)
    const int64_t nchunk_total = ntok * cpt;
    const int64_t c0 = t0 * cpt;
    const T* base = x + t0 * d;
    // all loads first, so they are in flight together
    vec8 v[MAXC];
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        if (k < cpt && c0 + lane + 64 * k < nchunk_total)
            v[k] = *reinterpret_cast<const vec8*>(base + 8 * (lane + 64 * k));
    }
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        if (k < cpt) {
            const int c = lane + 64 * k;  // chunk within the wave's span
            uint32_t byte = 0;
            float sum = 0.0f;
            if (c0 + c < nchunk_total) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = (float)v[k][e];
                    byte |= (f >= 0.0f ? 1u : 0u) << e;  // -0.0 >= 0 holds: zero counts as +1
                    sum += fabsf(f);
                }
            }
            const int t = (int)(((uint32_t)c * magic) >> 20), part = c - t * cpt;  // c / cpt for c < 1024
            sBits[wave][t * 16 + part] = (uint8_t)byte;
            sSum[wave][t * MAXC + part] = sum;
        }
    }
    if (cpt < 16) {  // bytes past the token's d channels read as zero
        for (int i = cpt; i < 16; ++i) sBits[wave][lane * 16 + i] = 0;
    }
    __syncthreads();
    const int64_t t = t0 + lane;
    if (t < ntok) {
        const uint4 w = *reinterpret_cast<const uint4*>(&sBits[wave][lane * 16]);
        uint32_t* out = bits + t * W;
        out[0] = w.x;
        if (W > 1) out[1] = w.y;
        if (W > 2) out[2] = w.z;
        if (W > 3) out[3] = w.w;
        float sum = 0.0f;
        for (int part = 0; part < cpt; ++part) sum += sSum[wave][lane * MAXC + part];
        mu[t] = sum / (float)d;
    }
}

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s) {
    const int W = (d + 31) / 32;
    const dim3 block(256), grid((unsigned)((ntok + 4 * kPackTok - 1) / (4 * kPackTok)));
    if (f32)
        hipLaunchKernelGGL(pack_qk_kernel<float>, grid, block, 0, s, (const float*)x, ntok, d, W, bits, mu);
    else
        hipLaunchKernelGGL(pack_qk_kernel<_Float16>, grid, block, 0, s, (const _Float16*)x, ntok, d, W, bits, mu);
    return hipGetLastError();
}

}  // namespace binattn
