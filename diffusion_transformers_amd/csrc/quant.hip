// quant.hip -- channel-wise symmetric int8 quantisation of V.
//
// "BinaryAttention" paper notes (CVPR 2026), key design 3 (Hybrid
// Quantization): V is quantised channel-wise to 8 bits.  Per (batch, head,
// channel c), in fp32 with IEEE division and round-half-even:
//   a = max_n |v[n,c]|, scale = a/127, inv = 127/a, vq = clamp(rint(v*inv), -127, 127).
//
// Output layout is channel-major, vq[bh][c][n] with key stride ldv (N rounded up
// to 64, tail zero-filled): the integer PV product contracts over keys, and an
// MFMA operand wants each lane's 16 key values contiguous.  The transpose is done
// here, through LDS, once per call.
//
// Two schedules (the same arithmetic):
//   fused  (a head fits): one workgroup per head; the head is read from HBM once
//          into registers, reduced, quantised and transposed on chip.
//   split  (long N): zero-fill, absmax over (head, chunk) with atomicMax on the
//          fp32 bit pattern (valid since |v| >= 0), quantise over (head, 64-key
//          block), then scale = a/127 in place.
#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kFusedMaxTok = 24;       // tokens per thread held in registers by the fused schedule
constexpr int kFusedMaxImg = 48 * 1024; // bytes of the channel-major LDS image of one head
constexpr int kChunk = 1024;  // tokens per absmax workgroup in the split schedule
constexpr int kTPad = 16;     // LDS row padding (bytes) of the transpose tile

template <typename T>
struct VecOf {
    static constexpr int VE = 16 / sizeof(T);
    typedef T type __attribute__((ext_vector_type(VE)));
};

// Per-thread partial absmax over tokens [n0, n1) for channels [part*VE, part*VE+VE),
// reduced over the workgroup into amax[0..d).  All 256 threads must call it.
template <typename T>
__device__ void head_absmax(const T* __restrict__ vh, int n0, int n1, int d, float* sRed, float* amax) {
    constexpr int VE = VecOf<T>::VE;
    typedef typename VecOf<T>::type vecT;
    const int P = d / VE, G = 256 / P, tid = threadIdx.x;
    const int part = tid % P, grp = tid / P;
    float m[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) m[e] = 0.0f;
    if (grp < G) {
        for (int n = n0 + grp; n < n1; n += G) {
            const vecT v = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
#pragma unroll
            for (int e = 0; e < VE; ++e) m[e] = fmaxf(m[e], fabsf((float)v[e]));
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) sRed[grp * d + part * VE + e] = m[e];
    }
    __syncthreads();
    if (tid < d) {
        float a = 0.0f;
        for (int g = 0; g < G; ++g) a = fmaxf(a, sRed[g * d + tid]);
        amax[tid] = a;
    }
    __syncthreads();
}

// Quantise tokens [j0, j0+64) of one head (tokens >= N become 0) and store them
// channel-major: vq[c*ldv + j0 .. +64).  inv[c] = 127/a_c (0 when a_c == 0).
template <typename T>
__device__ void quant_block(const T* __restrict__ vh, int N, int d, int64_t ldv, int j0, const float* inv,
                            uint8_t* sT, int8_t* __restrict__ vqh) {
    constexpr int VE = VecOf<T>::VE;
    typedef typename VecOf<T>::type vecT;
    const int P = d / VE, G = 256 / P, tid = threadIdx.x;
    const int part = tid % P, grp = tid / P;
    constexpr int TS = 64 + kTPad;
    if (grp < G) {
        for (int nl = grp; nl < 64; nl += G) {
            const int n = j0 + nl;
            vecT v;
            if (n < N) {
                v = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) v[e] = (T)0;
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const int c = part * VE + e;
                float r = __builtin_rintf((float)v[e] * inv[c]);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                sT[c * TS + nl] = (uint8_t)(int8_t)(int)r;
            }
        }
    }
    __syncthreads();
    for (int id = tid; id < d * 4; id += 256) {
        const int c = id >> 2, q = id & 3;
        const uint4 val = *reinterpret_cast<const uint4*>(sT + c * TS + 16 * q);
        *reinterpret_cast<uint4*>(vqh + (int64_t)c * ldv + j0 + 16 * q) = val;
    }
    __syncthreads();
}

// Fused schedule: every token of the head is loaded once into registers (thread
// (part, grp) holds tokens grp, grp+G, ...; consecutive lanes read consecutive 16-byte
// chunks), the channel absmax is reduced through LDS, the register copies are
// quantised into a zeroed channel-major LDS image of the head, and the image is stored
// with contiguous 16-byte writes.
template <typename T, int MAXT>
__global__ __launch_bounds__(256) void quant_v_fused_kernel(const T* __restrict__ v, int N, int d, int64_t ldv,
                                                            int8_t* __restrict__ vq, float* __restrict__ vscale) {
    constexpr int VE = VecOf<T>::VE;
    typedef typename VecOf<T>::type vecT;
    extern __shared__ __attribute__((aligned(16))) uint8_t sImg[];  // [d][ldv] int8
    __shared__ float sRed[2048];
    __shared__ float sInv[128];
    const int64_t bh = blockIdx.x;
    const T* vh = v + bh * (int64_t)N * d;
    const int P = d / VE, G = 256 / P, tid = threadIdx.x;
    const int part = tid % P, grp = tid / P;
    const bool active = grp < G;
    vecT x[MAXT];
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
        const int n = grp + G * k;
        if (active && n < N) {
            x[k] = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) x[k][e] = (T)0;
        }
    }
    // zero the image (tokens N .. ldv-1 stay zero) while the loads are in flight
    const int nvec = (int)(d * ldv / 16);
    for (int id = tid; id < nvec; id += 256) reinterpret_cast<uint4*>(sImg)[id] = make_uint4(0, 0, 0, 0);
    float m[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) m[e] = 0.0f;
#pragma unroll
    for (int k = 0; k < MAXT; ++k)
#pragma unroll
        for (int e = 0; e < VE; ++e) m[e] = fmaxf(m[e], fabsf((float)x[k][e]));
    if (active) {
#pragma unroll
        for (int e = 0; e < VE; ++e) sRed[grp * d + part * VE + e] = m[e];
    }
    __syncthreads();
    if (tid < d) {
        float a = 0.0f;
        for (int g = 0; g < G; ++g) a = fmaxf(a, sRed[g * d + tid]);
        vscale[bh * d + tid] = a / 127.0f;
        sInv[tid] = a > 0.0f ? 127.0f / a : 0.0f;
    }
    __syncthreads();
    if (active) {
        float inv[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) inv[e] = sInv[part * VE + e];
#pragma unroll
        for (int k = 0; k < MAXT; ++k) {
            const int n = grp + G * k;
            if (n < N) {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    float r = __builtin_rintf((float)x[k][e] * inv[e]);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    sImg[(int64_t)(part * VE + e) * ldv + n] = (uint8_t)(int8_t)(int)r;
                }
            }
        }
    }
    __syncthreads();
    int8_t* vqh = vq + bh * d * ldv;
    for (int id = tid; id < nvec; id += 256)
        reinterpret_cast<uint4*>(vqh)[id] = reinterpret_cast<const uint4*>(sImg)[id];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <typename T>
__global__ __launch_bounds__(256) void absmax_split_kernel(const T* __restrict__ v, int N, int d,
                                                           float* __restrict__ amax_out) {
    __shared__ float sRed[2048];
    __shared__ float sAmax[128];
    const int64_t bh = blockIdx.y;
    const int n0 = blockIdx.x * kChunk, n1 = min(N, n0 + kChunk);
    head_absmax<T>(v + bh * (int64_t)N * d, n0, n1, d, sRed, sAmax);
    if ((int)threadIdx.x < d)
        atomicMax(reinterpret_cast<unsigned int*>(amax_out + bh * d + threadIdx.x), __float_as_uint(sAmax[threadIdx.x]));
}

template <typename T>
__global__ __launch_bounds__(256) void quant_split_kernel(const T* __restrict__ v, int N, int d, int64_t ldv,
                                                          const float* __restrict__ amax, int8_t* __restrict__ vq) {
    __shared__ float sInv[128];
    __shared__ __attribute__((aligned(16))) uint8_t sT[128 * (64 + kTPad)];
    const int64_t bh = blockIdx.y;
    if ((int)threadIdx.x < d) {
        const float a = amax[bh * d + threadIdx.x];
        sInv[threadIdx.x] = a > 0.0f ? 127.0f / a : 0.0f;
    }
    __syncthreads();
    quant_block<T>(v + bh * (int64_t)N * d, N, d, ldv, blockIdx.x * 64, sInv, sT, vq + bh * d * ldv);
}

__global__ __launch_bounds__(256) void finalize_scale_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = p[i] / 127.0f;
}

template <typename T>
static hipError_t launch_quant_t(const T* v, int BH, int N, int d, int64_t ldv, int8_t* vq, float* vscale,
                                 hipStream_t s) {
    constexpr int VE = VecOf<T>::VE;
    const int G = 256 / (d / VE);
    const int64_t img = (int64_t)d * ldv;
    const int tpt = (N + G - 1) / G;  // tokens per thread
    if (tpt <= kFusedMaxTok && img <= kFusedMaxImg) {
        if (tpt <= 8)
            hipLaunchKernelGGL((quant_v_fused_kernel<T, 8>), dim3(BH), dim3(256), (size_t)img, s, v, N, d, ldv, vq, vscale);
        else if (tpt <= 16)
            hipLaunchKernelGGL((quant_v_fused_kernel<T, 16>), dim3(BH), dim3(256), (size_t)img, s, v, N, d, ldv, vq, vscale);
        else
            hipLaunchKernelGGL((quant_v_fused_kernel<T, 24>), dim3(BH), dim3(256), (size_t)img, s, v, N, d, ldv, vq, vscale);
        return hipGetLastError();
    }
    const int64_t n = (int64_t)BH * d;
    const dim3 lin((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(fill_zero_kernel, lin, dim3(256), 0, s, vscale, n);
    hipLaunchKernelGGL(absmax_split_kernel<T>, dim3((N + kChunk - 1) / kChunk, BH), dim3(256), 0, s, v, N, d,
                       vscale);
    hipLaunchKernelGGL(quant_split_kernel<T>, dim3((unsigned)(ldv / 64), BH), dim3(256), 0, s, v, N, d, ldv,
                       (const float*)vscale, vq);
    hipLaunchKernelGGL(finalize_scale_kernel, lin, dim3(256), 0, s, vscale, n);
    return hipGetLastError();
}

hipError_t launch_quant_v(const void* v, int f32, int BH, int N, int d, int64_t ldv, int8_t* vq, float* vscale,
                          hipStream_t s) {
    if (f32) return launch_quant_t<float>((const float*)v, BH, N, d, ldv, vq, vscale, s);
    return launch_quant_t<_Float16>((const _Float16*)v, BH, N, d, ldv, vq, vscale, s);
}

}  // namespace binattn
