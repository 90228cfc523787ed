// prep.h -- device bodies of the input-side steps, shared by the single-purpose kernels and
// the one-launch preparation kernel.
//
// "BinaryAttention" paper notes (CVPR 2026), Method details:
//   key design 1: each channel of Q and K keeps only its sign; a per-token scale mu
//                 (mean |x| over the d channels) keeps the magnitude;
//   key design 3: V is quantised channel-wise to int8 with scale a_c / 127, a_c the
//                 channel's absmax over the tokens of one (batch, head).
#pragma once

#include <algorithm>

#include "common.h"

namespace binattn {

// One 8-channel fp16 chunk: the sign byte (bit e = x_e >= 0, so -0.0 counts as +1) and the
// fp32 sum of |x_e| (a fixed chain of v_dot2_f32_f16 against 1.0, so every caller gets the same
// rounding).  The sign test reads the bit patterns of a channel pair: a half is negative when
// its sign bit is set and its magnitude is not 0, and magnitude + 0x7FFF carries into the sign
// position exactly when the magnitude is not 0 (no carry crosses into the other half).
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void chunk_sign_abs(const h8& x, uint32_t& byte, float& sum) {
    const h2 one = h2{(_Float16)1, (_Float16)1};
    uint32_t y = 0;  // channel 2i >= 0 at bit 2i, channel 2i+1 >= 0 at bit 16 + 2i
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = __builtin_bit_cast(uint32_t, h2{x[2 * i], x[2 * i + 1]});
        const uint32_t mag = w & 0x7FFF7FFFu;
        const uint32_t nonneg = ~(w & (mag + 0x7FFF7FFFu)) & 0x80008000u;
        y |= nonneg >> (15 - 2 * i);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, mag), one, acc, false);
    }
    byte = (y & 0x55u) | ((y >> 15) & 0xAAu);
    sum = acc;
}

// Sign words and mu of one token per thread: token 256 blk + 64 wave + lane (tokens >= ntok read
// as zero and are not written).  All of the token's 16-byte chunks are
// loaded first; each 8-channel chunk then gives one sign byte and a partial |x| sum
// (chunk_sign_abs for fp16; channel order for fp32), and the partial sums add up in channel
// order.  No LDS and no barrier: a workgroup is four independent waves.
template <typename T>
__device__ __forceinline__ void pack_wave(const T* __restrict__ x, int64_t ntok, int d, int W,
                                          uint32_t* __restrict__ bits, float* __restrict__ mu, int64_t blk) {
    constexpr int ES = sizeof(T);
    constexpr int LPC = 8 * ES / 16;  // 16-byte loads per 8-channel chunk
    constexpr int MAXC = 16;          // chunks of d <= 128
    const int lane = threadIdx.x & 63;
    const int64_t tok0 = blk * 256 + 64 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int cpt = d >> 3;
    const int64_t left = ntok - tok0;
    const int ntw = left < 64 ? (int)left : 64;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x + tok0 * d, ntw * d * ES);
    const int off = lane * d * ES;
    uint4 v[MAXC * LPC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
        if (c < cpt) {
#pragma unroll
            for (int l = 0; l < LPC; ++l)
                v[c * LPC + l] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16 * (c * LPC + l), 0, 0));
        }
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (c < cpt) {
            uint32_t byte = 0;
            float sum = 0.0f;
            if constexpr (ES == 2) {
                chunk_sign_abs(__builtin_bit_cast(h8, v[c]), byte, sum);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint4 q = v[c * LPC + e / 4];
                    const float f = __uint_as_float(e % 4 == 0 ? q.x : e % 4 == 1 ? q.y : e % 4 == 2 ? q.z : q.w);
                    byte |= (f >= 0.0f ? 1u : 0u) << e;  // -0.0 >= 0 holds: zero counts as +1
                    sum += fabsf(f);
                }
            }
            words[c >> 2] |= byte << (8 * (c & 3));
            acc += sum;
        }
    }
    if (lane < ntw) {
        const int64_t tok = tok0 + lane;
        uint32_t* out = bits + tok * W;
        switch (W) {
            case 1: out[0] = words[0]; break;
            case 2: *reinterpret_cast<uint2*>(out) = make_uint2(words[0], words[1]); break;
            case 3: out[0] = words[0]; out[1] = words[1]; out[2] = words[2]; break;
            default: *reinterpret_cast<uint4*>(out) = make_uint4(words[0], words[1], words[2], words[3]); break;
        }
        mu[tok] = acc / (float)d;
    }
}

// Workgroups of 256 tokens (four waves of 64) over ntok tokens.
__host__ __device__ inline int64_t pack_blocks(int64_t ntok) { return (ntok + 255) / 256; }

constexpr int kQuantTB = 128;     // tokens per block of the transpose tile
constexpr int kQuantTS = 128 + 4;  // LDS row stride (bytes) of that tile: 33 dwords, so rows of
                                   // consecutive channels fall in different banks

template <typename T>
struct QuantVec {
    static constexpr int VE = 16 / sizeof(T);  // elements per 16-byte chunk
    typedef T type __attribute__((ext_vector_type(VE)));
};

// Chunks (one token x VE channels) per thread when thread (part, grp) of one head holds the
// 4-token groups grp, grp + G, ... (G = 256 / (d / VE)) of its channel part.
template <typename T>
__host__ __device__ inline int quant_chunks_per_thread(int N, int d) {
    const int G = 256 / (d / QuantVec<T>::VE);
    return 4 * (((N + 3) / 4 + G - 1) / G);
}

// 4 tokens x 4 channels of int8 (dword t = token t, byte c = channel c) -> dword c = channel c,
// byte t = token t.
__device__ __forceinline__ void transpose4x4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // a0 b0 a1 b1
    const uint32_t ab_hi = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // a2 b2 a3 b3
    const uint32_t cd_lo = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t cd_hi = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);  // a0 b0 c0 d0
    out[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);  // a1 b1 c1 d1
    out[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

// Channel-wise int8 quantisation of one head with its V held in registers (MAXC chunks per
// thread, in groups of 4 consecutive tokens): absmax per channel (registers; then the 256
// threads reduce the per-thread maxima, 256/d threads per channel, meeting in an LDS max),
// IEEE 127 / a, rint -- every chunk quantised in registers -- then per 128-token block each
// 4-token group is transposed in registers (v_perm) into one dword per channel, written to an
// LDS tile of channel rows, and stored as rows of ldv keys (16-byte stores); tokens >= N are
// written as 0.
// sRed: 256*VE floats, sAmax: 128 words, sT: 128 * kQuantTS bytes (16-byte aligned).
template <typename T, int MAXC>
__device__ __forceinline__ void quant_head_regs(const T* __restrict__ v, int N, int d, int64_t ldv, int64_t bh,
                                                int8_t* __restrict__ vq, float* __restrict__ vamax, float* sRed,
                                                float* sAmax, uint8_t* sT) {
    constexpr int VE = QuantVec<T>::VE;
    constexpr int VW = VE / 4;  // dwords of quantised bytes per chunk
    constexpr int MAXU = MAXC / 4;
    typedef typename QuantVec<T>::type vecT;
    const int tid = threadIdx.x;
    const int P = d / VE, G = 256 / P;
    const int part = tid % P, grp = tid / P;
    const T* vh = v + bh * (int64_t)N * d;
    uint32_t* sAmaxU = reinterpret_cast<uint32_t*>(sAmax);
    if (tid < 128) sAmaxU[tid] = 0u;  // the max of non-negative floats, compared as their bit patterns
    vecT x[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int n = 4 * (grp + G * (i >> 2)) + (i & 3);
        if (grp < G && n < N) {
            x[i] = *reinterpret_cast<const vecT*>(vh + (int64_t)n * d + part * VE);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) x[i][e] = (T)0;
        }
    }
    // absmax in the input precision (exact: max and |.| do not round)
    vecT mv;
#pragma unroll
    for (int e = 0; e < VE; ++e) mv[e] = (T)0;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) mv = __builtin_elementwise_max(mv, __builtin_elementwise_abs(x[i]));
    if (grp < G) {
#pragma unroll
        for (int e = 0; e < VE; ++e) sRed[grp * d + part * VE + e] = (float)mv[e];
    }
    __syncthreads();
    {
        const int K = 256 / d;  // threads per channel
        if (tid < K * d) {
            const int c = tid % d, s0 = tid / d;
            float a = 0.0f;
            for (int g = s0; g < G; g += K) a = fmaxf(a, sRed[g * d + c]);
            atomicMax(&sAmaxU[c], __float_as_uint(a));
        }
    }
    __syncthreads();
    if (tid < d) vamax[bh * d + tid] = __uint_as_float(sAmaxU[tid]);
    float inv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const float a = grp < G ? __uint_as_float(sAmaxU[part * VE + e]) : 0.0f;
        inv[e] = a > 0.0f ? 127.0f / a : 0.0f;
    }
    // quantise every chunk and transpose each 4-token group: qt[u][e] = channel part*VE+e,
    // bytes = tokens 4*(grp+G*u) .. +3
    uint32_t qt[MAXU][VE];
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        uint32_t qb[4][VW];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int w = 0; w < VW; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    // |x| <= a gives |x * fl32(127/a)| < 127.0001, so rint is already within +-127
                    const float q = __builtin_rintf((float)x[4 * u + r][4 * w + b] * inv[4 * w + b]);
                    word = __builtin_amdgcn_cvt_pk_u8_f32(q + 128.0f, b, word);  // exact: q is an integer
                }
                qb[r][w] = word ^ 0x80808080u;  // back to two's-complement int8
            }
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            const uint32_t in[4] = {qb[0][w], qb[1][w], qb[2][w], qb[3][w]};
            uint32_t out[4];
            transpose4x4(in, out);
#pragma unroll
            for (int c = 0; c < 4; ++c) qt[u][4 * w + c] = out[c];
        }
    }
    int8_t* vqh = vq + bh * d * ldv;
    for (int j0 = 0; j0 < ldv; j0 += kQuantTB) {
        const int nb = (int)std::min<int64_t>(kQuantTB, ldv - j0);  // 64 or 128 keys
        if (j0 > 0) __syncthreads();  // the previous block's tile has been stored
        if (j0 + nb > N) {  // ragged last block: positions past N stay 0
            for (int id = tid; id < 128 * kQuantTS / 16; id += 256) reinterpret_cast<uint4*>(sT)[id] = make_uint4(0, 0, 0, 0);
            __syncthreads();
        }
        if (grp < G) {
#pragma unroll
            for (int u = 0; u < MAXU; ++u) {
                const int n0 = 4 * (grp + G * u);  // first token of the group (tokens past N hold 0)
                if (n0 >= j0 && n0 < j0 + nb && n0 < N) {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        *reinterpret_cast<uint32_t*>(sT + (part * VE + e) * kQuantTS + (n0 - j0)) = qt[u][e];
                }
            }
        }
        __syncthreads();
        const int qw = nb / 16;  // 16-byte pieces per row: one global store each
        for (int id = tid; id < d * qw; id += 256) {
            const int c = id / qw, q = id - c * qw;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(sT + c * kQuantTS + 16 * q);
            *reinterpret_cast<uint4*>(vqh + (int64_t)c * ldv + j0 + 16 * q) = make_uint4(src[0], src[1], src[2], src[3]);
        }
    }
}

}  // namespace binattn
