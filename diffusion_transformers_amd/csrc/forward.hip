// forward.hip -- fused BinaryAttention forward (and the integer-score export).
//
// "BinaryAttention" paper notes (CVPR 2026), Method details:
//   key design 1: D_ij = s_i.t_j from the sign bits, scaled by mu_q mu_k;
//   key design 2: S_ij = mu_q mu_k D_ij / sqrt(d) + b_ij (dense or relative-position b);
//   key design 3: softmax output quantised to u8 with scale 1/255, V int8 per channel,
//                 integer PV product, float dequantisation;
//   hardware implementation bullet: one FlashAttention2-style tiled kernel.
//
// gfx950 design (one workgroup = 4 waves = 128 queries of one (b,h); key tiles of 64):
//  * QK^T on the int8 MFMA (v_mfma_i32_16x16x64_i8) with sign bits unpacked to
//    +-1 bytes: exact integer D.  The tile is computed transposed (keys are MFMA
//    rows, queries columns) and the key rows are permuted so that lane (query n,
//    group g) ends up holding the 16 consecutive keys 16g..16g+15 of the tile for
//    query n -- exactly the A-operand layout of the PV MFMA, so P never leaves
//    registers, and the per-lane bias run is contiguous in memory.
//  * K bits are unpacked once per workgroup per tile into LDS in MFMA-operand
//    order (each lane reads 16 consecutive bytes); V^ (channel-major in HBM) is
//    staged the same way.
//  * Online softmax in fp32 with the running max reduced over the 4 lanes that
//    share a query.  p = 255 * exp(S - m) = exp2(S*log2e - m*log2e + log2 255),
//    P^ = rint(p) via v_cvt_pk_u8_f32.
//  * PV with signed int8 MFMA: sum (P^-128) V^ + 128 sum V^, the column sum coming
//    from one extra MFMA against a ones operand.  The int32 accumulators run on
//    across tiles while no row max in the wave changes; when one does, the wave
//    folds them into fp32 accumulators rescaled by exp(m_old - m_new).
//  * Epilogue: O = acc * vscale_c / sum(p).
#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kWaves = 4;
constexpr int kCB = 2;                      // 16-query column blocks per wave
constexpr int kBR = kWaves * kCB * 16;      // queries per workgroup
constexpr int kBC = 64;                     // keys per tile
constexpr int kRelposWin = 3072;            // fp32 entries of the staged relative-position window
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.99435343685886f;

enum { BK_NONE = 0, BK_DENSE_F16 = 1, BK_DENSE_F32 = 2, BK_RELPOS = 3 };

// Keys of one 64-key tile as A-operand rows: MFMA tile t, row m <-> key 16*(m/4) + 4t + (m%4).
// After the MFMA, lane (n, g) register r of tile t holds key 16g + 4t + r.
__device__ __forceinline__ int key_slot(int j, int& t) {
    t = (j & 15) >> 2;
    return 4 * (j >> 4) + (j & 3);
}

template <int KC>
struct KTile {
    // [kc][t][lane] x 16 bytes: the A operand of QK MFMA (kc, t) for each lane.
    uint32_t w[KC * 4 * kWave * 4];
};

// Unpack the K sign bits of keys [j0, j0+64) into LDS operand order (+-1 int8, zero for
// channels >= d and keys >= N).
template <int KC>
__device__ __forceinline__ void stage_k(const uint32_t* __restrict__ kb, int N, int d, int W, int j0,
                                        KTile<KC>& sK) {
    for (int id = threadIdx.x; id < kBC * 4 * KC; id += 256) {
        const int j = id / (4 * KC), grp = id % (4 * KC);
        const int kc = grp >> 2, g = grp & 3;
        const int ch0 = 64 * kc + 16 * g;
        uint32_t word = 0;
        if (j0 + j < N && ch0 < d) word = kb[(int64_t)(j0 + j) * W + (ch0 >> 5)];
        uint32_t o[4];
        unpack_signs16((word >> (ch0 & 16)) & 0xFFFFu, o);
        const bool live = j0 + j < N;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = (live && ch0 + 4 * q < d) ? o[q] : 0u;
        int t;
        const int m = key_slot(j, t);
        const int lane = m + 16 * g;
        uint4* dst = reinterpret_cast<uint4*>(&sK.w[((kc * 4 + t) * kWave + lane) * 4]);
        *dst = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Q operand (B of the QK MFMA) for one lane: query row, channels 64kc + 16g .. +15.
template <int KC>
__device__ __forceinline__ void load_q(const uint32_t* __restrict__ qrow, bool live, int d, int g, v4i q[KC]) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int ch0 = 64 * kc + 16 * g;
        uint32_t word = (live && ch0 < d) ? qrow[ch0 >> 5] : 0u;
        uint32_t o[4];
        unpack_signs16((word >> (ch0 & 16)) & 0xFFFFu, o);
#pragma unroll
        for (int c = 0; c < 4; ++c) q[kc][c] = (live && ch0 + 4 * c < d) ? (int)o[c] : 0;
    }
}

template <int KC>
__device__ __forceinline__ void qk_tile(const KTile<KC>& sK, const v4i q[KC], int lane, v4i D[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        D[t] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const v4i a = *reinterpret_cast<const v4i*>(&sK.w[((kc * 4 + t) * kWave + lane) * 4]);
            D[t] = mfma_i8(a, q[kc], D[t]);
        }
    }
}

__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float quad_sum(float v) {
    v += __shfl_xor(v, 16);
    return v + __shfl_xor(v, 32);
}

template <int NT, int BIAS>
__global__ __launch_bounds__(256, 2) void binattn_fwd_kernel(FwdArgs a) {
    constexpr int KC = (NT + 3) / 4;
    __shared__ __attribute__((aligned(16))) KTile<KC> sK;
    __shared__ __attribute__((aligned(16))) uint32_t sV[NT * kWave * 4];
    __shared__ __attribute__((aligned(16))) float sMu[kBC];
    __shared__ float sT[BIAS == BK_RELPOS ? kRelposWin : 1];

    const int N = a.N, d = a.d, W = a.W;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    int bh, qb;
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
        // dense bias is shared over the batch: keep the batch items of one (h, query block) together
        const int b = lb % a.B, hq = lb / a.B;
        qb = hq % nqb;
        bh = b * a.H + hq / nqb;
    } else {
        bh = lb / nqb;
        qb = lb % nqb;
    }
    const int h = bh % a.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int q0 = qb * kBR;

    const uint32_t* kbh = a.kbits + (int64_t)bh * N * W;
    const float* kmuh = a.kmu + (int64_t)bh * N;
    const int8_t* vqh = a.vq + (int64_t)bh * d * a.ldv;

    // per column block: Q operand, row scale, running max, partial row sum
    v4i qop[kCB][KC];
    float cq[kCB], mrun[kCB], lpart[kCB];
    int qi[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
        const int i = q0 + (wave * kCB + cb) * 16 + n16;
        const bool live = i < N;
        qi[cb] = live ? i : N - 1;
        load_q<KC>(a.qbits + ((int64_t)bh * N + qi[cb]) * W, live, d, g, qop[cb]);
        cq[cb] = live ? a.qmu[(int64_t)bh * N + i] * a.qk_scale : 0.0f;
        mrun[cb] = -INFINITY;
        lpart[cb] = 0.0f;
    }
    v4i acci[kCB][NT], cs[NT];
    v4f accf[kCB][NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        cs[ct] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            acci[cb][ct] = v4i{0, 0, 0, 0};
            accf[cb][ct] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};

    const int ntiles = (N + kBC - 1) / kBC;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int j0 = tile * kBC;
        // ---- stage K operand, V^ operand, mu_k (and the relative-position window)
        stage_k<KC>(kbh, N, d, W, j0, sK);
        for (int id = tid; id < NT * 16 * 4; id += 256) {
            const int c = id >> 2, gg = id & 3;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (c < d) val = *reinterpret_cast<const uint4*>(vqh + (int64_t)c * a.ldv + j0 + 16 * gg);
            const int ln = (c & 15) + 16 * gg;
            *reinterpret_cast<uint4*>(&sV[((c >> 4) * kWave + ln) * 4]) = val;
        }
        if (tid < kBC) sMu[tid] = (j0 + tid < N) ? kmuh[j0 + tid] : 0.0f;
        int dr_lo = 0, row_len = 0;
        if (BIAS == BK_RELPOS) {
            const int gw = a.gw;
            const int ri_min = q0 / gw, ri_max = (min(q0 + kBR, N) - 1) / gw;
            const int rj_min = j0 / gw, rj_max = (min(j0 + kBC, N) - 1) / gw;
            dr_lo = ri_min - rj_max + a.gh - 1;
            const int rows = (ri_max - ri_min) + (rj_max - rj_min) + 1;
            row_len = 2 * gw - 1;
            const int64_t tsz = (int64_t)(2 * a.gh - 1) * row_len;
            const int64_t base = (int64_t)h * tsz + (int64_t)dr_lo * row_len;
            for (int id = tid; id < rows * row_len; id += 256)
                sT[id] = a.bias_f32 ? ((const float*)a.bias)[base + id] : (float)((const _Float16*)a.bias)[base + id];
        }
        __syncthreads();

        // ---- QK^T (exact integers), scale + bias, running max
        v4i kop[KC][4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                kop[kc][t] = *reinterpret_cast<const v4i*>(&sK.w[((kc * 4 + t) * kWave + lane) * 4]);
        float muk[16];
#pragma unroll
        for (int k = 0; k < 16; k += 4) {
            const float4 m4 = *reinterpret_cast<const float4*>(&sMu[16 * g + k]);
            muk[k] = m4.x; muk[k + 1] = m4.y; muk[k + 2] = m4.z; muk[k + 3] = m4.w;
        }
        const int jg = j0 + 16 * g;  // first key of this lane's run
        const bool last = (tile == ntiles - 1);
        float s[kCB][16];
        float mnew[kCB];
        bool any_up = false;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            v4i D[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                D[t] = v4i{0, 0, 0, 0};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) D[t] = mfma_i8(kop[kc][t], qop[cb][kc], D[t]);
            }
            float bia[16];
            if (BIAS == BK_DENSE_F16) {
                const _Float16* br = (const _Float16*)a.bias + ((int64_t)h * N + qi[cb]) * a.bias_ld + jg;
                const h8 zero8 = h8{0, 0, 0, 0, 0, 0, 0, 0};
                const h8 lo = (jg < N) ? *reinterpret_cast<const h8*>(br) : zero8;
                const h8 hi = (jg + 8 < N) ? *reinterpret_cast<const h8*>(br + 8) : zero8;
#pragma unroll
                for (int k = 0; k < 8; ++k) { bia[k] = (float)lo[k]; bia[k + 8] = (float)hi[k]; }
            } else if (BIAS == BK_DENSE_F32) {
                const float* br = (const float*)a.bias + ((int64_t)h * N + qi[cb]) * a.bias_ld + jg;
#pragma unroll
                for (int k = 0; k < 16; k += 4) {
                    const float4 f4 = (jg + k < N) ? *reinterpret_cast<const float4*>(br + k) : make_float4(0, 0, 0, 0);
                    bia[k] = f4.x; bia[k + 1] = f4.y; bia[k + 2] = f4.z; bia[k + 3] = f4.w;
                }
            } else if (BIAS == BK_RELPOS) {
                const int gw = a.gw;
                const int ri = qi[cb] / gw, ci = qi[cb] % gw;
                const int rj = jg / gw, cj = jg % gw;
                const int idx0 = (ri - rj + a.gh - 1 - dr_lo) * row_len + (ci - cj + gw - 1);
                if (jg < N) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) bia[k] = sT[idx0 - k];
                } else {
#pragma unroll
                    for (int k = 0; k < 16; ++k) bia[k] = 0.0f;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) bia[k] = 0.0f;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float x = (float)D[k >> 2][k & 3] * muk[k];
                float sv = __builtin_fmaf(x, cq[cb], bia[k]);
                if (last && jg + k >= N) sv = -INFINITY;
                s[cb][k] = sv;
                mloc = fmaxf(mloc, sv);
            }
            mloc = quad_max(mloc);
            mnew[cb] = fmaxf(mrun[cb], mloc);
            any_up |= mnew[cb] > mrun[cb];
        }

        // ---- the row max moved somewhere in the wave: fold int32 partials into fp32, rescaled
        if (__any(any_up)) {
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
                const float alpha = fast_exp2((mrun[cb] - mnew[cb]) * kLog2e);  // 0 on the first tile
                lpart[cb] *= alpha;
                float ar[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tot = acci[cb][ct][r] + 128 * cs[ct][r];
                        accf[cb][ct][r] = (accf[cb][ct][r] + (float)tot) * ar[r];
                    }
                    acci[cb][ct] = v4i{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) cs[ct] = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) mrun[cb] = mnew[cb];

        // ---- P^ = rint(255 exp(S - m)) - 128 as int8, row sums, integer PV
        v4i vop[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            vop[ct] = *reinterpret_cast<const v4i*>(&sV[(ct * kWave + lane) * 4]);
            cs[ct] = mfma_i8(ones, vop[ct], cs[ct]);
        }
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            const float negm = kLog2_255 - mrun[cb] * kLog2e;
            v4i pw;
            float lsum = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t word = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(s[cb][4 * t + r], kLog2e, negm));
                    lsum += p;
                    word = __builtin_amdgcn_cvt_pk_u8_f32(p, r, word);
                }
                pw[t] = (int)(word ^ 0x80808080u);
            }
            lpart[cb] += lsum;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acci[cb][ct] = mfma_i8(pw, vop[ct], acci[cb][ct]);
        }
        __syncthreads();
    }

    // ---- epilogue: O = acc * vscale / sum(p)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
        const float L = quad_sum(lpart[cb]);
        float inv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) inv[r] = 1.0f / __shfl(L, 4 * g + r);
        const int ibase = q0 + (wave * kCB + cb) * 16 + 4 * g;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int c = ct * 16 + n16;
            if (c >= d) continue;
            const float sv = a.vscale[(int64_t)bh * d + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ibase + r;
                if (i >= N) continue;
                const int tot = acci[cb][ct][r] + 128 * cs[ct][r];
                const float o = (accf[cb][ct][r] + (float)tot) * sv * inv[r];
                const int64_t off = ((int64_t)bh * N + i) * d + c;
                if (a.out_f32)
                    ((float*)a.out)[off] = o;
                else
                    ((_Float16*)a.out)[off] = (_Float16)o;
            }
        }
    }
}

// Integer score export through the same K staging and QK tile as the forward kernel.
template <int KC>
__global__ __launch_bounds__(256, 2) void binattn_scores_kernel(FwdArgs a) {
    __shared__ __attribute__((aligned(16))) KTile<KC> sK;
    const int N = a.N, d = a.d, W = a.W;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    const int bh = lb / nqb, qb = lb % nqb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int q0 = qb * kBR;
    v4i qop[kCB][KC];
    int qi[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
        const int i = q0 + (wave * kCB + cb) * 16 + n16;
        qi[cb] = i;
        load_q<KC>(a.qbits + ((int64_t)bh * N + (i < N ? i : N - 1)) * W, i < N, d, g, qop[cb]);
    }
    const uint32_t* kbh = a.kbits + (int64_t)bh * N * W;
    const int ntiles = (N + kBC - 1) / kBC;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int j0 = tile * kBC;
        stage_k<KC>(kbh, N, d, W, j0, sK);
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            v4i D[4];
            qk_tile<KC>(sK, qop[cb], lane, D);
            if (qi[cb] < N) {
                int32_t* row = a.scores + ((int64_t)bh * N + qi[cb]) * N;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = j0 + 16 * g + 4 * t + r;
                        if (j < N) row[j] = D[t][r];
                    }
            }
        }
        __syncthreads();
    }
}

template <int NT>
static hipError_t launch_fwd_nt(const FwdArgs& a, int bk, hipStream_t s) {
    const int nqb = (a.N + kBR - 1) / kBR;
    const dim3 grid((unsigned)(a.B * a.H * nqb)), block(256);
    switch (bk) {
        case BK_NONE: hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK_NONE>), grid, block, 0, s, a); break;
        case BK_DENSE_F16: hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK_DENSE_F16>), grid, block, 0, s, a); break;
        case BK_DENSE_F32: hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK_DENSE_F32>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK_RELPOS>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int bias_kind, hipStream_t s) {
    int bk = BK_NONE;
    if (bias_kind == 1) bk = a.bias_f32 ? BK_DENSE_F32 : BK_DENSE_F16;
    if (bias_kind == 2) bk = BK_RELPOS;
    switch ((a.d + 15) / 16) {
        case 1: return launch_fwd_nt<1>(a, bk, s);
        case 2: return launch_fwd_nt<2>(a, bk, s);
        case 3: return launch_fwd_nt<3>(a, bk, s);
        case 4: return launch_fwd_nt<4>(a, bk, s);
        case 5: return launch_fwd_nt<5>(a, bk, s);
        case 6: return launch_fwd_nt<6>(a, bk, s);
        case 7: return launch_fwd_nt<7>(a, bk, s);
        default: return launch_fwd_nt<8>(a, bk, s);
    }
}

hipError_t launch_scores(const FwdArgs& a, hipStream_t s) {
    const int nqb = (a.N + kBR - 1) / kBR;
    const dim3 grid((unsigned)(a.B * a.H * nqb)), block(256);
    if (a.d <= 64)
        hipLaunchKernelGGL(binattn_scores_kernel<1>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(binattn_scores_kernel<2>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace binattn
