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
//    rows add them per tile as two more MFMAs (B = 64) into the same accumulator.
//  * Epilogue: O = acc * s_c / sum(p), s_c = a_c / 127 from the channel absmax a_c.
#include <type_traits>

#include "tile.h"

namespace binattn {

// ---------------------------------------------------------------------------------------------
// Longer rows: key tiles streamed through a two-stage LDS ring, FlashAttention-2 running max.
// DEFER: keep the PV sums in int32 across tiles and fold them into fp32 only when some row
// max of the wave moves (long rows, where that becomes rare).  TF32: the relative-position
// table is fp32 (else fp16).
//
// Relative position: the window staged for a tile holds the table rows its queries and keys
// touch, from row dr_lo = ri_min - rjm + gh - 1 (ri_min: grid row of the block's first query,
// rjm: grid row of the tile's last key).  The entry of query (ri, ci) and key (rj, cj) sits at
// (ri - ri_min + rjm - rj) row_len + ci - cj + gw - 1: a query part fixed per lane, a tile part
// rjm row_len, and a key part rj row_len + cj that moves by a whole tile of keys per step --
// all stepped from tile to tile without a division.
template <int NT, int BIAS, bool DEFER, bool TF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT <= 4 && (BIAS == BK_RELPOS || BIAS == BK_NONE) ? 4 : 1))) void binattn_fwd_stream_kernel(FwdArgs a) {
    constexpr int TW = BIAS == BK_RELPOS ? kRelposWin : 4;
    typedef TileRegs<NT, TW> Regs;
    typedef TileLds<NT, TW> Lds;
    __shared__ Lds lds[2];
    __shared__ __attribute__((aligned(16))) float sScale[128];

    const int N = a.N, d = a.d;
    int bh, q0;
    block_coords<BIAS>(a, bh, q0);
    const int h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntiles = (N + kBC - 1) / kBC;
    const int nfull = N / kBC;  // tiles whose 64 keys are all < N

    HeadPtrs hp;
    hp.kb = a.kbits + (int64_t)bh * N * ((NT + 1) / 2);
    hp.kmu = a.kmu + (int64_t)bh * N;
    hp.vq = a.vq + (int64_t)bh * d * a.ldv;
    hp.table = nullptr;
    if (BIAS == BK_RELPOS) {
        const int64_t tsz = (int64_t)(2 * a.gh - 1) * (2 * a.gw - 1);
        hp.table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz)
                              : (const void*)((const _Float16*)a.bias + h * tsz);
    }
    stage_common(a, bh, sScale);

    const int qw0 = q0 + wave * 16;
    const bool wave_live = qw0 < N;
    const LaneQ lq = lane_query<NT>(a, bh, qw0, g, n16);

    // relative position (see above): per lane the query part aq and the key part kk (kcol: the
    // key's grid column); uniform, the grid position (lrow, lcol) of the last key of the last
    // tile loaded, and rjm_ld, the window's key row for that tile
    const int gw = a.gw, row_len = 2 * gw - 1;
    const int dcol = BIAS == BK_RELPOS ? kBC % gw : 0, drow = BIAS == BK_RELPOS ? kBC / gw : 0;
    int aq = 0, kk = 0, kcol = 0, ri_min = 0, lrow = 0, lcol = 0, rjm_ld = 0;
    if (BIAS == BK_RELPOS) {
        ri_min = q0 / gw;
        const int ri = lq.qi / gw, ci = lq.qi - ri * gw;
        aq = (ri - ri_min) * row_len + ci + gw - 1;
        const int rj = (16 * g) / gw;
        kcol = 16 * g - rj * gw;
        kk = rj * row_len + kcol;
        lrow = (kBC - 1) / gw;
        lcol = kBC - 1 - lrow * gw;
        rjm_ld = min(lrow, a.gh - 1);
    }
    auto window_off = [&](int rjm) { return (ri_min - rjm + a.gh - 1) * row_len; };

    // dense bias rows of this wave: row (h, qw0 + r) at offset r*ld elements; rows >= N read 0
    const int esz = BIAS == BK_DENSE_F32 ? 4 : 2;
    const char* brow = nullptr;
    int brow_bytes = 0;
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
        const int r0 = min(qw0, N);
        brow = (const char*)a.bias + ((int64_t)h * N + r0) * a.bias_ld * esz;
        brow_bytes = min(N - r0, 16) * (int)a.bias_ld * esz;
    }
    const int bvoff = (n16 * (int)a.bias_ld + 16 * g) * esz;

    float mrun = -INFINITY, lsum = 0.0f;
    v4i acci[NT];
    float accf[NT][4];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        acci[ct] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[ct][r] = 0.0f;
    }

    Regs regs;
    BiasRegs<BIAS> b0, b1;
    load_tile<NT, TW>(regs, a, hp, 0, window_off(rjm_ld));
    load_bias<BIAS>(b0, buffer_rsrc(brow, brow_bytes), bvoff);

    // One pipeline step: stage tile `tile` into LDS, issue the loads of tile+1, compute tile.
    // TAIL: the last tile, whose keys past N are masked (compiled separately, so that the steps
    // over whole tiles carry no masking).  The two bias register sets alternate without copies.
    auto step = [&](int tile, BiasRegs<BIAS>& bcur, BiasRegs<BIAS>& bnext, auto tail_c) {
        constexpr bool TAIL = decltype(tail_c)::value;
        Lds& s = lds[tile & 1];
        store_tile<NT, TW, false, TF32>(regs, s, d);
        __syncthreads();
        const int rjm = rjm_ld;  // window key row of this tile
        if (tile + 1 < ntiles) {
            const int jn = (tile + 1) * kBC;
            if (BIAS == BK_RELPOS) {  // the last key of tile + 1, one tile of keys on
                lcol += dcol;
                lrow += drow;
                if (lcol >= gw) lcol -= gw, ++lrow;
                rjm_ld = min(lrow, a.gh - 1);
            }
            load_tile<NT, TW>(regs, a, hp, jn, window_off(rjm_ld));
            load_bias<BIAS>(bnext, buffer_rsrc(brow + jn * esz, brow_bytes - jn * esz), bvoff);
        }
        // (a wave wholly past N computes on clamped inputs and stores nothing: no per-tile test)
        const int jg = tile * kBC + 16 * g;
        int idx0 = 15;
        if (BIAS == BK_RELPOS) {
            idx0 = aq + rjm * row_len - kk;
            if (TAIL && jg >= N) idx0 = 15;  // a run wholly past N is masked; its reads stay in the window
            kcol += dcol;                    // this lane's keys in the next tile
            kk += drow * row_len + dcol;
            if (kcol >= gw) kcol -= gw, kk += row_len - gw;
        }
        float S[16], mloc = -INFINITY;
        tile_scores<NT, BIAS>(s.k, s.mu, lq, bcur, s.tw + idx0 - 15, TAIL, N - jg, S, mloc);
        const float mnew = fmaxf(mrun, rows4_max(mloc));
        if (__any(mnew > mrun)) {
            const float alpha = fast_exp2((mrun - mnew) * kLog2e);  // 0 on the first tile
            lsum *= alpha;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accf[ct][r] = DEFER ? (accf[ct][r] + (float)acci[ct][r]) * alpha : accf[ct][r] * alpha;
                if (DEFER) acci[ct] = v4i{0, 0, 0, 0};
            }
        }
        mrun = mnew;
        const v4i pw = tile_probs(S, kLog2_255 - mnew * kLog2e, lsum);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const v4i vop = *reinterpret_cast<const v4i*>(&s.v[(ct * kWave + lane) * 4]);
            if (DEFER) {
                v4i x = mfma_i8(vop, pw, acci[ct]);
                x = mfma_i8(vop, kC64, x);
                acci[ct] = mfma_i8(vop, kC64, x);
            } else {
                v4i x = mfma_i8(vop, pw, v4i{0, 0, 0, 0});
                x = mfma_i8(vop, kC64, x);
                x = mfma_i8(vop, kC64, x);
#pragma unroll
                for (int r = 0; r < 4; ++r) accf[ct][r] += (float)x[r];
            }
        }
    };
    const std::false_type whole;
    const std::true_type tail;
    int tile = 0;
    for (; tile + 2 <= nfull; tile += 2) {
        step(tile, b0, b1, whole);
        step(tile + 1, b1, b0, whole);
    }
    // at most one whole tile and the ragged last tile remain; bias set b0 is the current one
    if (tile < nfull) {
        step(tile, b0, b1, whole);
        if (tile + 1 < ntiles) step(tile + 1, b1, b0, tail);
    } else if (tile < ntiles) {
        step(tile, b0, b1, tail);
    }

    if (!wave_live) return;
    if (DEFER) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) accf[ct][r] += (float)acci[ct][r];
    }
    store_out<NT>(a, bh, lq, sScale, accf, rows4_sum(lsum));
}

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

template <int NT, int BK, bool TF32>
static void launch_stream(const FwdArgs& a, int ntiles, dim3 grid, hipStream_t s) {
    if (ntiles >= kDeferTiles)
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, true, TF32>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, false, TF32>), grid, dim3(256), 0, s, a);
}

template <int NT, int BK>
static void launch_fwd_bk(const FwdArgs& a, hipStream_t s) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    const int nqb = (a.N + kBR - 1) / kBR;
    if (ntiles <= kKeepTiles && (BK != BK_RELPOS || keep_window_fits(a))) {
        launch_keep<NT, BK, false>(a, s);
        return;
    }
    if constexpr (NT <= 4 && BK != BK_RELPOS) {
        if (ntiles <= kLongTiles) {
            launch_keep_long<NT, BK>(a, s);
            return;
        }
    }
    const dim3 grid((unsigned)(a.B * a.H * nqb));
    if constexpr (BK == BK_RELPOS) {
        if (a.bias_f32) {
            launch_stream<NT, BK, true>(a, ntiles, grid, s);
            return;
        }
    }
    launch_stream<NT, BK, false>(a, ntiles, grid, s);
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
