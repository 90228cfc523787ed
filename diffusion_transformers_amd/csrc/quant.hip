// quant.hip -- channel-wise symmetric int8 quantisation of V.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 3 (Hybrid
// Quantization): V is quantised channel-wise to 8 bits.  Per (batch, head,
// channel c), in fp32 with IEEE division and round-half-even:
//   a = max_n |v[n,c]|, inv = 127/a, vq = clamp(rint(v*inv), -127, 127),
// and the dequantisation scale is a/127 (computed by the consumer from a).
//
// Output layout is channel-major, vq[bh][c][n] with key stride ldv (N rounded up
// to 64, tail zero-filled): the integer PV product contracts over keys, and an
// MFMA operand wants each lane's 16 key values contiguous.  The transpose is done
// here, through LDS, once per call.
//
// Two kernels: the channel absmax (one workgroup per head, or per 1024-token
// chunk of a long head with atomicMax on the fp32 bit pattern, valid since
// |v| >= 0, into a zeroed output), then the quantise/transpose kernel over
// (head, 64-token block) workgroups, which reads the finished absmax.  Each
// thread issues its loads together, so both kernels hide memory latency across
// many workgroups.
#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kChunk = 1024;  // tokens per absmax workgroup
constexpr int kBatch = 8;     // tokens per thread whose loads are in flight together
constexpr int kTPad = 16;     // LDS row padding (bytes) of the transpose tile

template <typename T>
struct VecOf {
    static constexpr int VE = 16 / sizeof(T);
    typedef T type __attribute__((ext_vector_type(VE)));
};

// Channel absmax over tokens [n0, n1) of one head: thread (part, grp) covers channels
// part*VE .. +VE of tokens grp, grp+G, ...; reduced through LDS.  ATOMIC: fold into a
// zeroed amax with atomicMax (several chunks per head), else store.
template <typename T, bool ATOMIC>
__global__ __launch_bounds__(256) void absmax_kernel(const T* __restrict__ v, int N, int d, int nchunk,
                                                     float* __restrict__ amax) {
    constexpr int VE = VecOf<T>::VE;
    typedef typename VecOf<T>::type vecT;
    __shared__ float sRed[2048];
    const int64_t bh = blockIdx.x / nchunk;
    const int n0 = (blockIdx.x % nchunk) * kChunk, n1 = min(N, n0 + kChunk);
    const T* vh = v + bh * (int64_t)N * d;
    const int P = d / VE, G = 256 / P, tid = threadIdx.x;
    const int part = tid % P, grp = tid / P;
    float m[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) m[e] = 0.0f;
    if (grp < G) {
        for (int nb = n0 + grp; nb < n1; nb += G * kBatch) {
            vecT x[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int n = nb + G * k;
                if (n < n1) {
                    x[k] = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) x[k][e] = (T)0;
                }
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
#pragma unroll
                for (int e = 0; e < VE; ++e) m[e] = fmaxf(m[e], fabsf((float)x[k][e]));
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) sRed[grp * d + part * VE + e] = m[e];
    }
    __syncthreads();
    if (tid < d) {
        float a = 0.0f;
        for (int g = 0; g < G; ++g) a = fmaxf(a, sRed[g * d + tid]);
        if (ATOMIC)
            atomicMax(reinterpret_cast<unsigned int*>(amax + bh * d + tid), __float_as_uint(a));
        else
            amax[bh * d + tid] = a;
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Quantise tokens [j0, j0+64) of one head (tokens >= N become 0) and store them
// channel-major: vq[c*ldv + j0 .. +64).
template <typename T>
__global__ __launch_bounds__(256) void quant_kernel(const T* __restrict__ v, int N, int d, int64_t ldv,
                                                    const float* __restrict__ amax, int8_t* __restrict__ vq) {
    constexpr int VE = VecOf<T>::VE;
    typedef typename VecOf<T>::type vecT;
    constexpr int TS = 64 + kTPad;
    __shared__ __attribute__((aligned(16))) uint8_t sT[128 * TS];
    const int nblk = (int)(ldv / 64);
    const int64_t bh = blockIdx.x / nblk;
    const int j0 = (blockIdx.x % nblk) * 64;
    const T* vh = v + bh * (int64_t)N * d;
    const int P = d / VE, G = 256 / P, tid = threadIdx.x;
    const int part = tid % P, grp = tid / P;
    constexpr int MAXK = 32 / VE;  // G = 256 / (d / VE) >= 256 VE / 128, so MAXK * G >= 64 for every d <= 128
    vecT x[MAXK];
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
        const int nl = grp + G * k, n = j0 + nl;
        if (grp < G && nl < 64 && n < N) {
            x[k] = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) x[k][e] = (T)0;
        }
    }
    if (grp < G) {
        float inv[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float a = amax[bh * d + part * VE + e];
            inv[e] = a > 0.0f ? 127.0f / a : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < MAXK; ++k) {
            const int nl = grp + G * k;
            if (nl < 64) {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    float r = __builtin_rintf((float)x[k][e] * inv[e]);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    sT[(part * VE + e) * TS + nl] = (uint8_t)(int8_t)(int)r;
                }
            }
        }
    }
    __syncthreads();
    int8_t* vqh = vq + bh * d * ldv;
    for (int id = tid; id < d * 4; id += 256) {
        const int c = id >> 2, q = id & 3;
        *reinterpret_cast<uint4*>(vqh + (int64_t)c * ldv + j0 + 16 * q) =
            *reinterpret_cast<const uint4*>(sT + c * TS + 16 * q);
    }
}

template <typename T>
static hipError_t launch_quant_t(const T* v, int BH, int N, int d, int64_t ldv, int8_t* vq, float* vamax,
                                 hipStream_t s) {
    // one-dimensional grids, head-major: (head, chunk) and (head, 64-token block)
    const int nchunk = (N + kChunk - 1) / kChunk;
    const int64_t nblk = ldv / 64;
    if ((int64_t)BH * nblk > 0x7fffffff) return hipErrorInvalidValue;
    if (nchunk == 1) {
        hipLaunchKernelGGL((absmax_kernel<T, false>), dim3((unsigned)BH), dim3(256), 0, s, v, N, d, 1, vamax);
    } else {
        const int64_t n = (int64_t)BH * d;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, vamax, n);
        hipLaunchKernelGGL((absmax_kernel<T, true>), dim3((unsigned)((int64_t)BH * nchunk)), dim3(256), 0, s, v,
                           N, d, nchunk, vamax);
    }
    hipLaunchKernelGGL(quant_kernel<T>, dim3((unsigned)(BH * nblk)), dim3(256), 0, s, v, N, d, ldv,
                       (const float*)vamax, vq);
    return hipGetLastError();
}

hipError_t launch_quant_v(const void* v, int f32, int BH, int N, int d, int64_t ldv, int8_t* vq, float* vamax,
                          hipStream_t s) {
    if (f32) return launch_quant_t<float>((const float*)v, BH, N, d, ldv, vq, vamax, s);
    return launch_quant_t<_Float16>((const _Float16*)v, BH, N, d, ldv, vq, vamax, s);
}

// The canonical token-major copy of a channel-major V^ ([B,H,d,ldv] -> [B,H,N,d]; bytes only).
// A workgroup takes one 64-token block of a head at a time (heads strided by gridDim.y): the d
// channel rows of the block (64 bytes each, 16-byte loads; ldv is a multiple of 64) go to an LDS
// tile [channel][token], then each thread assembles 8 channels of a token and stores them as one
// 8-byte word (d is a multiple of 8).
__global__ __launch_bounds__(256) void vq_canonical_kernel(const int8_t* __restrict__ vq, int64_t BH, int N, int d,
                                                           int64_t ldv, int8_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t sT[128][80];  // rows of 64 tokens, 16-byte aligned
    const int n0 = blockIdx.x * 64, tid = threadIdx.x, ng = d / 8;
    for (int64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
        const int8_t* src = vq + bh * d * ldv + n0;
        for (int i = tid; i < 4 * d; i += 256) {
            const int c = i >> 2, q = i & 3;
            *reinterpret_cast<uint4*>(&sT[c][16 * q]) = *reinterpret_cast<const uint4*>(src + (int64_t)c * ldv + 16 * q);
        }
        __syncthreads();
        for (int i = tid; i < 64 * ng; i += 256) {
            const int t = i / ng, cg = i - t * ng;
            if (n0 + t < N) {
                uint32_t lo = 0u, hi = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo |= (uint32_t)sT[8 * cg + e][t] << (8 * e);
                    hi |= (uint32_t)sT[8 * cg + 4 + e][t] << (8 * e);
                }
                *reinterpret_cast<uint2*>(out + (bh * N + n0 + t) * d + 8 * cg) = make_uint2(lo, hi);
            }
        }
        __syncthreads();  // the tile is read before the next head's block overwrites it
    }
}

hipError_t launch_vq_canonical(const int8_t* vq, int64_t BH, int N, int d, int64_t ldv, int8_t* out, hipStream_t s) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)(BH < 65535 ? BH : 65535));
    hipLaunchKernelGGL(vq_canonical_kernel, grid, dim3(256), 0, s, vq, BH, N, d, ldv, out);
    return hipGetLastError();
}

}  // namespace binattn
