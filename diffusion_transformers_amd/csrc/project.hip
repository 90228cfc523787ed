// project.hip -- the QKV projection with the binarisation of Q and K in its epilogue.
//
// "BinaryAttention" paper notes (CVPR 2026), "Method details", key design 1 (Scaled Binary
// Representations): the attention uses Q and K only through each channel's sign and each
// token's mean |x|.  So the linear projection that produces them hands over just those: the
// epilogue of every output tile packs the tile's Q and K heads (the arithmetic of
// binattn_pack_qk) and never writes them in fp16 unless asked.  V is stored in fp16: key design
// 3 quantises it per channel over all N tokens of a head, which no projection tile sees whole.
//
// y = x w^T (+ bias): x [M, C] token-major fp16 (C = H d), w [3C, C] fp16, fp32 accumulation on
// v_mfma_f32_16x16x32_f16, rounded to fp16 (round-to-nearest-even) as a projection stores it.
// Output feature o = p C + h d + c is channel c of head h of part p (Q, K, V).
//
// Tiling: a workgroup (four waves) owns 256 tokens x one run of HPT consecutive head sections
// (16 NB features, whole heads, so a token's head is complete inside the tile); a wave owns 64
// tokens x all of the tile's features: 4 x NB accumulator tiles.  The x operand is private to a
// wave, so it goes from global memory straight into MFMA operand registers, one k-step ahead;
// the w operand is shared by the four waves and staged through LDS, double-buffered, one barrier
// per 32-wide k-step.  Tiles are numbered so that an XCD runs consecutive ones, in bands of a few
// token blocks whose x rows stay in that XCD's L2 while the feature runs go by, each w slab
// serving the band's token blocks together.
// Epilogue: the fp32 tile plus bias, rounded to fp16, goes to LDS as [token][feature]; then
// each lane owns one token and, per head section, stores its d values (V, and Q or K when
// asked) or packs them into sign words and mu (Q, K).
#include "common.h"
#include "internal.h"
#include "prep.h"

namespace binattn {

namespace {

constexpr int kPM = 256;      // tokens per workgroup (64 per wave)
constexpr int kPK = 32;       // k per step (one MFMA depth)
constexpr int kPBP = kPK + 8;  // halfs per staged w row: 80-byte pitch
constexpr int kBand = 8;      // token blocks per band of the tile order

__device__ __forceinline__ v4f mfma_h(h8 a, h8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int NB>
struct alignas(16) ProjLds {
    static constexpr int BN = 16 * NB, EP = BN + 8;  // tile features; epilogue row pitch (halfs)
    union {
        _Float16 b[2][(BN + 63) / 64 * 64 * kPBP];  // staged w rows [feature][k] (every thread's chunks)
        _Float16 e[kPM * EP];      // epilogue tile [token][feature]
    };
};

template <int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_pack_kernel(ProjArgs a) {
    typedef ProjLds<NB> Lt;
    constexpr int BN = Lt::BN, EP = Lt::EP;
    constexpr int NBL = (BN * 4 + 255) / 256;  // 16-byte w chunks per thread and k-step
    __shared__ Lt L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    // tile order: bands of kBand token blocks; inside a band the token block runs fastest, so
    // the workgroups that run together on one XCD share their w slabs as well as their x rows
    const int tau = xcd_logical_block(blockIdx.x, a.nmt * a.nnt);
    const int band = tau / (kBand * a.nnt), in_band = tau - band * kBand * a.nnt;
    const int gm = min(kBand, a.nmt - band * kBand);
    const int nt = in_band / gm, mt = band * kBand + (in_band - nt * gm);
    const int64_t m0 = (int64_t)mt * kPM;
    const int s0 = nt * a.hpt, nsec = min(a.hpt, a.nsec - s0), ncol = nsec * a.d;
    const int C = a.C, nk = (C + kPK - 1) / kPK;
    const _Float16* __restrict__ wt = a.w + (int64_t)s0 * a.d * C;  // the tile's first w row

    // Ranged buffer loads: x rows past M and w rows past the tile's features read as zero.  A
    // k chunk past C (C % 32 != 0) is zeroed on the w side only: its x chunk is finite data of
    // the next row or zero, and meets a zero weight.
    const __amdgpu_buffer_rsrc_t xr =
        buffer_rsrc(a.x + m0 * C, (int)(min((int64_t)kPM, a.M - m0) * C * 2));
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wt, ncol * C * 2);
    int aoff[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) aoff[rb] = ((64 * wave + 16 * rb + l16) * C + 8 * g) * 2;
    int boff[NBL];
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        const int id = tid + 256 * i;
        boff[i] = id < BN * 4 ? ((id >> 2) * C + 8 * (id & 3)) * 2 : -1;
    }
    auto load_a = [&](int ks, h8* dst) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            dst[rb] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(xr, aoff[rb] + ks * (2 * kPK), 0, 0));
    };
    auto load_b = [&](int ks, uint4* dst) {
        const int k0 = ks * kPK;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const int id = tid + 256 * i;
            const int off = (boff[i] >= 0 && k0 + 8 * (id & 3) < C) ? boff[i] + 2 * k0 : -16;  // -16: past any range
            dst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
        }
    };
    auto store_b = [&](int buf, const uint4* src) {
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const int id = tid + 256 * i;
            *reinterpret_cast<uint4*>(&L.b[buf][(id >> 2) * kPBP + 8 * (id & 3)]) = src[i];
        }
    };

    v4f acc[4][NB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Two register sets per operand (steps of even and odd parity): step ks stores the w chunks
    // of step ks + 1 (loaded a step earlier) into LDS, loads those of step ks + 2 into the set it
    // just freed, computes with its x set and then loads step ks + 2's x into it, so every load
    // has a whole step to land.  The steady state has no branches: loads for steps past the end
    // read zeros or unused rows (ranged buffer loads) and the last store fills a buffer nobody
    // reads.
    h8 a0[4], a1[4];
    uint4 b0[NBL], b1[NBL];
    load_b(0, b0);
    load_a(0, a0);
    store_b(0, b0);
    load_b(1, b1);
    load_a(1, a1);
    auto step = [&](int ks, h8* av, uint4* bnext, uint4* bfree) {
        __syncthreads();  // w step ks is in LDS; every wave is done with step ks - 1's buffer
        store_b((ks + 1) & 1, bnext);
        load_b(ks + 2, bfree);
        __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the step's MFMAs
        const _Float16* lb = L.b[ks & 1];
        h8 bf[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) bf[cb] = *reinterpret_cast<const h8*>(&lb[(16 * cb + l16) * kPBP + 8 * g]);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) acc[rb][cb] = mfma_h(av[rb], bf[cb], acc[rb][cb]);
        load_a(ks + 2, av);
    };
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
        step(ks, a0, b1, b0);
        step(ks + 1, a1, b0, b1);
    }
    if (ks < nk) step(ks, a0, b1, b0);

    // ---- epilogue: + bias, fp16, [token][feature] in LDS
    __syncthreads();  // every wave is done with the w buffers (the epilogue tile overlays them)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int col = 16 * cb + l16;
        const float bv = (a.bias && col < ncol) ? (float)a.bias[(int64_t)s0 * a.d + col] : 0.0f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) L.e[(64 * wave + 16 * rb + 4 * g + r) * EP + col] = (_Float16)(acc[rb][cb][r] + bv);
    }
    __syncthreads();
    const int64_t m = m0 + 64 * wave + lane;
    if (m >= a.M) return;
    const int d = a.d, H = a.H, N = a.N, W = a.W, cpt = d >> 3;
    const int64_t bb = m / N, n = m - bb * N;
    const _Float16* row = &L.e[(64 * wave + lane) * EP];
    for (int s = 0; s < nsec; ++s) {
        const int gs = s0 + s, part = gs / H, h = gs - part * H;
        const int64_t th = (bb * H + h) * N + n;  // token index in [B, H, N]
        const _Float16* src = row + s * d;
        _Float16* dst = part == 2 ? a.v : (part == 0 ? a.q : a.k);
        if (dst) {
            _Float16* o = dst + th * d;
            for (int c = 0; c < cpt; ++c)
                *reinterpret_cast<uint4*>(o + 8 * c) = *reinterpret_cast<const uint4*>(src + 8 * c);
        }
        if (part < 2) {  // sign words and mu: binattn_pack_qk's arithmetic on the fp16 values
            uint32_t words[4] = {0u, 0u, 0u, 0u};
            float sum = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c < cpt) {
                    uint32_t byte;
                    float part_sum;
                    chunk_sign_abs(*reinterpret_cast<const h8*>(src + 8 * c), byte, part_sum);
                    words[c >> 2] |= byte << (8 * (c & 3));
                    sum += part_sum;
                }
            uint32_t* ob = (part == 0 ? a.qbits : a.kbits) + th * W;
            switch (W) {
                case 1: ob[0] = words[0]; break;
                case 2: *reinterpret_cast<uint2*>(ob) = make_uint2(words[0], words[1]); break;
                case 3: ob[0] = words[0]; ob[1] = words[1]; ob[2] = words[2]; break;
                default: *reinterpret_cast<uint4*>(ob) = make_uint4(words[0], words[1], words[2], words[3]); break;
            }
            (part == 0 ? a.qmu : a.kmu)[th] = sum / (float)d;
        }
    }
}

}  // namespace

// Head sections per tile: as many whole heads as fit in 144 features (at least one); the tile
// width rounds up to the MFMA's 16 and to at least 80 features (one instantiation per 5..9).
void qkv_pack_plan(int H, int d, int64_t M, int* hpt, int* nb, int* nmt, int* nnt) {
    const int nsec = 3 * H;
    int s = 144 / d;
    if (s < 1) s = 1;
    if (s > nsec) s = nsec;
    int b = (s * d + 15) / 16;
    if (b < 5) b = 5;
    *hpt = s;
    *nb = b;
    *nmt = (int)((M + kPM - 1) / kPM);
    *nnt = (nsec + s - 1) / s;
}

hipError_t launch_qkv_pack(const ProjArgs& args, hipStream_t s) {
    ProjArgs a = args;
    int nb = 0;
    qkv_pack_plan(a.H, a.d, a.M, &a.hpt, &nb, &a.nmt, &a.nnt);
    a.nsec = 3 * a.H;
    a.C = a.H * a.d;
    a.W = (a.d + 31) / 32;
    const dim3 grid((unsigned)((int64_t)a.nmt * a.nnt)), block(256);
    switch (nb) {
        case 5: hipLaunchKernelGGL(qkv_pack_kernel<5>, grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL(qkv_pack_kernel<6>, grid, block, 0, s, a); break;
        case 7: hipLaunchKernelGGL(qkv_pack_kernel<7>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(qkv_pack_kernel<8>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(qkv_pack_kernel<9>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace binattn
