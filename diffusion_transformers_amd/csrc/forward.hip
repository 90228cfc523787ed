// forward.hip -- fused BinaryAttention forward (and the integer-score export).
//
// "BinaryAttention" paper notes (CVPR 2026), Method details:
//   key design 1: D_ij = s_i.t_j from the sign bits, scaled by mu_q mu_k;
//   key design 2: S_ij = mu_q mu_k D_ij / sqrt(d) + b_ij (dense or relative-position b);
//   key design 3: softmax output quantised to u8 with scale 1/255, V int8 per channel,
//                 integer PV product, float dequantisation;
//   hardware implementation bullet: one FlashAttention2-style tiled kernel.
//
// gfx950 design (one workgroup = 4 waves x 16 queries of one (b,h); key tiles of 64):
//  * QK^T on the block-scaled MFMA with fp4 (E2M1) operands (v_mfma_f32_16x16x128_f8f6f4,
//    cbsz = blgp = 4; one instruction covers d <= 128, 16 bytes of operand per lane).
//    With s = +-1 query signs and b = 0/1 key bits, s.t = sum s (2b - 1) = 2 s.b - sum(s):
//    the K operand is the bits as fp4 {0, 1}, the Q operand is fp4 {+-2}, and the
//    accumulator is seeded with -sum(s) of the lane's query.  Every product and partial
//    sum is a small integer, so the fp32 result is D exactly, already in float.
//  * The score tile is computed transposed (keys are MFMA rows, queries columns) with the
//    key rows permuted so that lane (query n, group g) holds the 16 consecutive keys
//    16g..16g+15 of the tile for its query n.  That register set is exactly the B operand
//    of the int8 PV MFMA computed as O^T = V^T P^T, so P never leaves registers, the bias
//    run of a lane is contiguous, and every lane owns one query: the softmax statistics
//    need no shuffles.  V^ channels are permuted on staging so that a lane's output
//    registers are 4*ceil(d/16) consecutive channels of its query (vector stores).
//  * K bits are unpacked once per workgroup per tile into LDS in MFMA-operand order;
//    V^ (channel-major in HBM) is staged the same way.  All global reads go through
//    buffer resources rebased per tile on the scalar unit, so addresses cost no vector
//    ALU and reads past a head's end return zero.
//  * Rows that a workgroup can hold (at most four tiles, N <= 256; or at most ten tiles at
//    d <= 64 without the relative-position bias) take the exact row max in the head-resident
//    kernel of tile.h: every tile is staged in LDS at once, pass 1 computes the scores into
//    registers and the max, pass 2 quantises exp(S - max) and accumulates P^ V^ in int32 with
//    no rescaling.  Longer rows stream the tiles through a two-stage LDS ring with the
//    FlashAttention-2 running max (this file).
//  * p = 255 exp(S - m) = exp2(S log2e - m log2e + log2 255), P^ = rint(p) via
//    v_cvt_pk_u8_f32; the row sum is taken over the unquantised p.
//  * PV with signed int8 MFMA: sum P^ V^ = sum (P^-128) V^ + 128 sum V^.  Short rows take
//    the column sums once per head while staging and start the accumulator there; streamed
//    rows use the bytes 127 - P^ (also int8 for every P^) and accumulate the negated sum,
//    sum (127 - P^) V^ - 127 sum V^, with one constant MFMA (B = -127) per channel tile.
//  * Epilogue: O = acc * s_c / sum(p), s_c = a_c / 127 from the channel absmax a_c.
#include "stream.h"

namespace binattn {

// Integer score export through the same K staging, Q operand and QK tile as the forward kernels.
template <int NT>
__global__ __launch_bounds__(256) void binattn_scores_kernel(FwdArgs a) {
    constexpr int W = (NT + 1) / 2;
    typedef TileRegs<NT, 4> Regs;
    typedef TileLds<NT, 4> Lds;
    __shared__ Lds lds;
    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    const int bh = lb / nqb, qb = lb % nqb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int q0 = qb * kBR;
    v4i qop;
    const int i = q0 + wave * 16 + n16;
    const float seed = load_q<W>(a.qbits + ((int64_t)bh * N + (i < N ? i : N - 1)) * W, i < N, d, g, qop);
    const v4f dseed = v4f{seed, seed, seed, seed};
    const uint32_t* kbh = a.kbits + (int64_t)bh * N * W;
    const int ntiles = (N + kBC - 1) / kBC;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int j0 = tile * kBC;
        Regs r;
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbh + j0 * W, (N - j0) * W * 4);
#pragma unroll
        for (int u = 0; u < Regs::KT; ++u) r.kw[u] = __builtin_amdgcn_raw_buffer_load_b32(kr, (tid + 256 * u) * 4, 0, 0);
#pragma unroll
        for (int u = 0; u < Regs::VCH; ++u) r.v[u] = make_uint4(0, 0, 0, 0);
        r.mu = 0.0f;
        store_tile<NT, 4>(r, lds, d);
        __syncthreads();
        v4f D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // lanes with g >= W read group 0: their Q operand is zero
            const uint32_t* src = &lds.k[((t * W + (g < W ? g : 0)) * 16 + n16) * 4];
            D[t] = mfma_f4(*reinterpret_cast<const v4i*>(src), qop, dseed);
        }
        if (i < N) {
            int32_t* row = a.scores + ((int64_t)bh * N + i) * N;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    const int j = j0 + 16 * g + 4 * t + r2;
                    if (j < N) row[j] = (int32_t)D[t][r2];
                }
        }
        __syncthreads();
    }
}

// QK-tile probe: D_ij for every (query, key) by one of two methods, reduced per query row to
// max_j D_ij and sum_j D_ij (fp32, exact for these integer ranges), so that the cost of the
// tile itself is measured rather than the N^2 score writes.
//   METHOD 0: the forward's tile, fp4 MFMA on LDS-staged fp4 K operands;
//   METHOD 1: VALU XOR + v_bcnt on LDS-staged sign words, D = d - 2 popcount(q XOR k).
// Both hand D to the softmax stage as fp32 in the same lane layout (query n, keys 16g..16g+15).
template <int NT, int METHOD>
__global__ __launch_bounds__(256) void binattn_qk_stats_kernel(FwdArgs a, float* rowmax, float* rowsum) {
    constexpr int W = (NT + 1) / 2;
    typedef TileRegs<NT, 4> Regs;
    typedef TileLds<NT, 4> Lds;
    __shared__ Lds lds;
    __shared__ __attribute__((aligned(16))) uint32_t kraw[kBC * W];
    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int lb = xcd_logical_block(blockIdx.x, a.B * a.H * nqb);
    const int bh = lb / nqb, qb = lb % nqb;
    const int tid = threadIdx.x, wave = tid >> 6, g = (tid & 63) >> 4, n16 = tid & 15;
    const int i = qb * kBR + wave * 16 + n16;
    const bool live = i < N;
    const uint32_t* qrow = a.qbits + ((int64_t)bh * N + (live ? i : N - 1)) * W;
    v4i qop;
    v4f dseed = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t qw[W];
    if (METHOD == 0) {
        const float seed = load_q<W>(qrow, live, d, g, qop);
        dseed = v4f{seed, seed, seed, seed};
    } else {
#pragma unroll
        for (int w = 0; w < W; ++w) qw[w] = live ? qrow[w] : 0u;
    }
    const uint32_t* kbh = a.kbits + (int64_t)bh * N * W;
    const int ntiles = (N + kBC - 1) / kBC;
    float mloc = -INFINITY, ssum = 0.0f;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int j0 = tile * kBC, jg = j0 + 16 * g;
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbh + j0 * W, (N - j0) * W * 4);
        if (METHOD == 0) {
            Regs r;
#pragma unroll
            for (int u = 0; u < Regs::KT; ++u) r.kw[u] = __builtin_amdgcn_raw_buffer_load_b32(kr, (tid + 256 * u) * 4, 0, 0);
#pragma unroll
            for (int u = 0; u < Regs::VCH; ++u) r.v[u] = make_uint4(0, 0, 0, 0);
            r.mu = 0.0f;
            store_tile<NT, 4>(r, lds, d);
        } else {
            if (tid < kBC * W) kraw[tid] = __builtin_amdgcn_raw_buffer_load_b32(kr, tid * 4, 0, 0);
        }
        __syncthreads();
        float D[16];
        if (METHOD == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t* src = &lds.k[((t * W + (g < W ? g : 0)) * 16 + n16) * 4];  // Q is 0 for g >= W
                const v4f x = mfma_f4(*reinterpret_cast<const v4i*>(src), qop, dseed);
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) D[4 * t + r2] = x[r2];
            }
        } else {
            uint32_t kw[16 * W];
#pragma unroll
            for (int u = 0; u < 4 * W; ++u) {
                const uint4 x = *reinterpret_cast<const uint4*>(&kraw[16 * g * W + 4 * u]);
                kw[4 * u] = x.x; kw[4 * u + 1] = x.y; kw[4 * u + 2] = x.z; kw[4 * u + 3] = x.w;
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                uint32_t c = 0;
#pragma unroll
                for (int w = 0; w < W; ++w) c += __builtin_popcount(qw[w] ^ kw[k * W + w]);  // v_xor + v_bcnt (accumulating)
                D[k] = (float)(d - 2 * (int)c);
            }
        }
        const int nvalid = N - jg;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const bool ok = k < nvalid;
            mloc = fmaxf(mloc, ok ? D[k] : -INFINITY);
            ssum += ok ? D[k] : 0.0f;
        }
        __syncthreads();
    }
    const float m = rows4_max(mloc), sm = rows4_sum(ssum);
    if (live && g == 0) {
        rowmax[(int64_t)bh * N + i] = m;
        rowsum[(int64_t)bh * N + i] = sm;
    }
}

template <int NT>
static hipError_t launch_fwd_nt(const FwdArgs& a, int bk, hipStream_t s) {
    switch (bk) {
        case BK_NONE: launch_fwd_bk<NT, BK_NONE>(a, s); break;
        case BK_DENSE_F16: launch_fwd_bk<NT, BK_DENSE_F16>(a, s); break;
        case BK_DENSE_F32: launch_fwd_bk<NT, BK_DENSE_F32>(a, s); break;
        default: launch_fwd_bk<NT, BK_RELPOS>(a, s); break;
    }
    return hipGetLastError();
}

bool forward_streams(const FwdArgs& a, int bias_kind) { return stream_picked(a, bias_kind == 2); }

hipError_t launch_forward(const FwdArgs& a, int bias_kind, hipStream_t s) {
    int bk = BK_NONE;
    if (bias_kind == 1) bk = a.bias_f32 ? BK_DENSE_F32 : BK_DENSE_F16;
    if (bias_kind == 2) {
        if (relpos_kind(a.gw) == BK_RELPOS_G) return launch_forward_gather(a, s);
        bk = BK_RELPOS;
    }
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
    switch ((a.d + 31) / 32) {
        case 1: hipLaunchKernelGGL(binattn_scores_kernel<2>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(binattn_scores_kernel<4>, grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL(binattn_scores_kernel<6>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(binattn_scores_kernel<8>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int NTV>
static void launch_qk_stats_nt(const FwdArgs& a, int method, float* rowmax, float* rowsum, dim3 grid, hipStream_t s) {
    if (method)
        hipLaunchKernelGGL((binattn_qk_stats_kernel<NTV, 1>), grid, dim3(256), 0, s, a, rowmax, rowsum);
    else
        hipLaunchKernelGGL((binattn_qk_stats_kernel<NTV, 0>), grid, dim3(256), 0, s, a, rowmax, rowsum);
}

hipError_t launch_qk_stats(const FwdArgs& a, int method, float* rowmax, float* rowsum, hipStream_t s) {
    const int nqb = (a.N + kBR - 1) / kBR;
    const dim3 grid((unsigned)(a.B * a.H * nqb));
    switch ((a.d + 31) / 32) {
        case 1: launch_qk_stats_nt<2>(a, method, rowmax, rowsum, grid, s); break;
        case 2: launch_qk_stats_nt<4>(a, method, rowmax, rowsum, grid, s); break;
        case 3: launch_qk_stats_nt<6>(a, method, rowmax, rowsum, grid, s); break;
        default: launch_qk_stats_nt<8>(a, method, rowmax, rowsum, grid, s); break;
    }
    return hipGetLastError();
}

// Whether the relative-position window any tile of a streamed launch stages fits on chip
// (an upper bound on the table rows one query block and one key tile touch).
bool relpos_window_fits(int gw) {
    const int rows = (kBR - 1) / gw + 1 + (kBC - 1) / gw + 1 + 1;
    return rows * (2 * gw - 1) <= kRelposWin;
}

int keep_plan_max_blocks() { return kLongTiles; }

void keep_plan_host(int64_t nheads, int nqb, int slots, bool fused, int plan[4]) {
    const KeepPlan p = keep_plan(nheads, nqb, slots, fused ? 3.0 : 0.5);
    plan[0] = p.a;
    plan[1] = p.f;
    plan[2] = p.b;
    plan[3] = p.r;
}

}  // namespace binattn
