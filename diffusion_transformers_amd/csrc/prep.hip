// prep.hip -- the input side of the forward in one launch: sign words and mu of Q and of K
// ([notes] key design 1) and the channel-wise int8 V ([notes] key design 3), where
// [notes] is the "BinaryAttention" paper notes page (CVPR 2026), Method details.
//
// One grid, two kinds of workgroup: the first B*H quantise one head each with its V held in
// registers (the long ones, dispatched first so that none starts late), the rest pack spans of
// 256 Q tokens and then of K tokens (K only when the forward packs Q itself).  Heads whose V does not fit the register budget take the
// general path: the pack kernel, then the absmax and quantise kernels.
#include "common.h"
#include "internal.h"
#include "prep.h"

namespace binattn {

template <typename T, int MAXC>
__global__ __launch_bounds__(256) void prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, int BH, int N, int d, int W,
                                                   int64_t ldv, int64_t npack, uint32_t* __restrict__ qbits,
                                                   float* __restrict__ qmu, uint32_t* __restrict__ kbits,
                                                   float* __restrict__ kmu, int8_t* __restrict__ vq,
                                                   float* __restrict__ vamax) {
    // LDS of the quantise role: sRed (8 KB) + sAmax + the transpose tile (packing uses none).
    __shared__ __attribute__((aligned(16))) uint8_t smem[2048 * 4 + 128 * 4 + 128 * kQuantTS];
    const int64_t b = blockIdx.x;
    if (b < BH) {
        quant_head_regs<T, MAXC>(v, N, d, ldv, b, vq, vamax, reinterpret_cast<float*>(smem),
                                 reinterpret_cast<float*>(smem + 2048 * 4), smem + 2048 * 4 + 128 * 4);
        return;
    }
    const int64_t ntok = (int64_t)BH * N;
    const int64_t pb = b - BH;
    if (q && pb < npack)
        pack_wave<T>(q, ntok, d, W, qbits, qmu, pb);
    else
        pack_wave<T>(k, ntok, d, W, kbits, kmu, q ? pb - npack : pb);
}

template <typename T>
static hipError_t launch_prepare_t(const T* q, const T* k, const T* v, int BH, int N, int d, int64_t ldv,
                                   uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq,
                                   float* vamax, hipStream_t s) {
    const int W = (d + 31) / 32;
    const int64_t ntok = (int64_t)BH * N;
    const int64_t npack = pack_blocks(ntok);
    const int nc = quant_chunks_per_thread<T>(N, d);
    const int64_t nblocks = BH + (q ? 2 : 1) * npack;  // (no Q: K and V only)
    if (nblocks <= 0x7fffffff && nc <= 20) {
        const dim3 grid((unsigned)nblocks), block(256);
        if (nc <= 8)
            hipLaunchKernelGGL((prep_kernel<T, 8>), grid, block, 0, s, q, k, v, BH, N, d, W, ldv, npack, qbits, qmu,
                               kbits, kmu, vq, vamax);
        else
            hipLaunchKernelGGL((prep_kernel<T, 20>), grid, block, 0, s, q, k, v, BH, N, d, W, ldv, npack, qbits,
                               qmu, kbits, kmu, vq, vamax);
        return hipGetLastError();
    }
    const int f32 = sizeof(T) == 4;
    hipError_t e = q ? launch_pack_qk(q, f32, ntok, d, qbits, qmu, s) : hipSuccess;
    if (e == hipSuccess) e = launch_pack_qk(k, f32, ntok, d, kbits, kmu, s);
    if (e == hipSuccess) e = launch_quant_v(v, f32, BH, N, d, ldv, vq, vamax, s);
    return e;
}

hipError_t launch_prepare(const void* q, const void* k, const void* v, int f32, int BH, int N, int d, int64_t ldv,
                          uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq, float* vamax,
                          hipStream_t s) {
    if (f32)
        return launch_prepare_t<float>((const float*)q, (const float*)k, (const float*)v, BH, N, d, ldv, qbits, qmu,
                                       kbits, kmu, vq, vamax, s);
    return launch_prepare_t<_Float16>((const _Float16*)q, (const _Float16*)k, (const _Float16*)v, BH, N, d, ldv,
                                      qbits, qmu, kbits, kmu, vq, vamax, s);
}

}  // namespace binattn
