// stream.h -- the forward for rows too long to stage whole: key tiles streamed through a
// two-stage LDS ring with the FlashAttention-2 running max ("BinaryAttention" paper notes,
// CVPR 2026, hardware-implementation bullet), and the dispatch of a forward launch between it and
// the head-resident kernel of tile.h.  Shared by forward.hip and forward_gather.hip (the
// relative-position bias on grids whose width is not a multiple of 16).
#pragma once

#include <type_traits>

#include "tile.h"

namespace binattn {

// ---------------------------------------------------------------------------------------------
// Longer rows: key tiles streamed through a two-stage LDS ring, FlashAttention-2 running max.
// DEFER: keep the PV sums in int32 across tiles and fold them into fp32 only when some row
// max of the wave moves (long rows, where that becomes rare).  TF32: the relative-position
// table is fp32 (else fp16).  QX: the queries arrive unpacked (a.qx) and are packed in the
// prologue (a separate instantiation, so that its launches are told apart in profiles).
//
// Relative position: the window staged for a tile holds the table rows its queries and keys
// touch, from row dr_lo = ri_min - rjm + gh - 1 (ri_min: grid row of the block's first query,
// rjm: grid row of the tile's last key).  The entry of query (ri, ci) and key (rj, cj) sits at
// (ri - ri_min + rjm - rj) row_len + ci - cj + gw - 1: a query part fixed per lane, a tile part
// rjm row_len, and a key part rj row_len + cj that moves by a whole tile of keys per step --
// all stepped from tile to tile without a division.
template <int NT, int BIAS, bool DEFER, bool TF32, bool QX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT <= 4 && (BIAS == BK_RELPOS || BIAS == BK_NONE) ? 4 : 1))) void binattn_fwd_stream_kernel(FwdArgs a) {
    constexpr int TW = is_relpos(BIAS) ? kRelposWin : 4;
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
    if (is_relpos(BIAS)) {
        const int64_t tsz = (int64_t)(2 * a.gh - 1) * (2 * a.gw - 1);
        hp.table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz)
                              : (const void*)((const _Float16*)a.bias + h * tsz);
    }
    stage_common(a, bh, sScale);

    const int qw0 = q0 + wave * 16;
    const bool wave_live = qw0 < N;
    const int vrow = lane ^ ((lane >> 3) & 6);  // the lane's V^ operand row as store_tile<.., SWZ> stores it
    LaneQ lq;
    if constexpr (QX)
        lq = lane_query_raw<NT>(a, bh, qw0, g, n16);
    else
        lq = lane_query<NT>(a, bh, qw0, g, n16);

    // relative position (see above): per lane the query part aq and the key part kk (kcol: the
    // key's grid column); uniform, the grid position (lrow, lcol) of the last key of the last
    // tile loaded, and rjm_ld, the window's key row for that tile.  RELPOS_G (any grid width): in
    // place of the lane's run, thread tid < 64 steps the grid position (tr, tc) of key tid of each
    // tile and stages that key's part for every lane to gather (keys past N take key N - 1's).
    const int gw = a.gw, row_len = 2 * gw - 1;
    const int dcol = is_relpos(BIAS) ? kBC % gw : 0, drow = is_relpos(BIAS) ? kBC / gw : 0;
    int aq = 0, kk = 0, kcol = 0, ri_min = 0, lrow = 0, lcol = 0, rjm_ld = 0, tr = 0, tc = 0, klast = 0;
    if (is_relpos(BIAS)) {
        ri_min = q0 / gw;
        const int ri = lq.qi / gw, ci = lq.qi - ri * gw;
        aq = 4 * ((ri - ri_min) * row_len + ci + gw - 1);  // (in bytes: one form of it stays live)
        lrow = (kBC - 1) / gw;
        lcol = kBC - 1 - lrow * gw;
        rjm_ld = min(lrow, a.gh - 1);
    }
    if (BIAS == BK_RELPOS) {
        const int rj = (16 * g) / gw;
        kcol = 16 * g - rj * gw;
        kk = rj * row_len + kcol;
    }
    if (BIAS == BK_RELPOS_G) {
        tr = tid / gw;
        tc = tid - tr * gw;
        const int rl = (N - 1) / gw;
        klast = rl * row_len + (N - 1 - rl * gw);
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
        store_tile<NT, TW, false, TF32, true>(regs, s, d);
        if (BIAS == BK_RELPOS_G && tid < kBC) {
            s.kk[tid] = -4 * (tile * kBC + tid < N ? tr * row_len + tc : klast);
            tc += dcol;  // key tid of the next tile
            tr += drow;
            if (tc >= gw) tc -= gw, ++tr;
        }
        __syncthreads();
        const int rjm = rjm_ld;  // window key row of this tile
        if (tile + 1 < ntiles) {
            const int jn = (tile + 1) * kBC;
            if (is_relpos(BIAS)) {  // the last key of tile + 1, one tile of keys on
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
        const char* twb = reinterpret_cast<const char*>(s.tw);
        const float* wrun = s.tw;  // window entry of the run's key jg (+15 entries: its last key)
        if (BIAS == BK_RELPOS) {
            int off = aq + 4 * (rjm * row_len - kk - 15);
            if (TAIL && jg >= N) off = 0;  // a run wholly past N is masked; its reads stay in the window
            wrun = reinterpret_cast<const float*>(twb + off);
            kcol += dcol;  // this lane's keys in the next tile
            kk += drow * row_len + dcol;
            if (kcol >= gw) kcol -= gw, kk += row_len - gw;
        }
        if (BIAS == BK_RELPOS_G)  // the keys' parts are gathered from s.kk
            wrun = reinterpret_cast<const float*>(twb + aq + 4 * rjm * row_len);
        float S[16], mloc = -INFINITY;
        tile_scores<NT, BIAS, true>(s.k, s.mu, lq, bcur, wrun, TAIL, N - jg, S, mloc, s.kk + 16 * g);
        // The row max moves only if some lane's own max exceeds it: the cross-lane reduction and
        // the fold run only then (a row whose max stays gets alpha = 1).
        if (__any(mloc > mrun)) {
            const float mnew = fmaxf(mrun, rows4_max(mloc));
            const float alpha = fast_exp2((mrun - mnew) * kLog2e);  // 0 on the first tile
            lsum *= alpha;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accf[ct][r] = DEFER ? (accf[ct][r] - (float)acci[ct][r]) * alpha : accf[ct][r] * alpha;
                if (DEFER) acci[ct] = v4i{0, 0, 0, 0};
            }
            mrun = mnew;
        }
        const float mnew = mrun;
        // PV on the signed int8 MFMA with the bytes 127 - P^ and one constant MFMA (B = -127):
        // sum_j (127 - P^_j) V^_j - 127 sum_j V^_j = -sum_j P^_j V^_j, so the accumulators hold
        // the negated sums (one constant MFMA per channel tile instead of two for +128 sum V^)
        const v4i pw = tile_probs<0x7F7F7F7Fu>(S, kLog2_255 - mnew * kLog2e, lsum);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const v4i vop = *reinterpret_cast<const v4i*>(&s.v[(ct * kWave + vrow) * 4]);
            if (DEFER) {
                acci[ct] = mfma_i8(vop, kCm127, mfma_i8(vop, pw, acci[ct]));
            } else {
                const v4i x = mfma_i8(vop, kCm127, mfma_i8(vop, pw, v4i{0, 0, 0, 0}));
#pragma unroll
                for (int r = 0; r < 4; ++r) accf[ct][r] -= (float)x[r];
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
            for (int r = 0; r < 4; ++r) accf[ct][r] -= (float)acci[ct][r];
    }
    store_out<NT>(a, bh, lq, sScale, accf, rows4_sum(lsum));
}

template <int NT, int BK, bool TF32>
inline void launch_stream(const FwdArgs& a, int ntiles, dim3 grid, hipStream_t s) {
    const bool defer = ntiles >= kDeferTiles;
    if (a.qx) {
        if (defer)
            hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, true, TF32, true>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, false, TF32, true>), grid, dim3(256), 0, s, a);
    } else if (defer) {
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, true, TF32, false>), grid, dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, false, TF32, false>), grid, dim3(256), 0, s, a);
    }
}

// The kernel launch_fwd_bk picks: the head-resident kernel for rows of <= 4 tiles (relative
// position: when the whole row's window fits) and, at d <= 64 without the relative-position bias,
// for rows of <= 10 tiles; the streaming kernel otherwise.
inline bool stream_picked(const FwdArgs& a, bool relpos) {
    const int ntiles = (a.N + kBC - 1) / kBC, nt = (a.d + 15) / 16;
    if (ntiles <= kKeepTiles && (!relpos || keep_window_fits(a))) return false;
    if (nt <= 4 && !relpos && ntiles <= kLongTiles) return false;
    return true;
}

template <int NT, int BK>
inline void launch_fwd_bk(const FwdArgs& a, hipStream_t s) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    const int nqb = (a.N + kBR - 1) / kBR;
    if (ntiles <= kKeepTiles && (!is_relpos(BK) || keep_window_fits(a))) {
        launch_keep<NT, BK, false>(a, s);
        return;
    }
    if constexpr (NT <= 4 && !is_relpos(BK)) {
        if (ntiles <= kLongTiles) {
            launch_keep_long<NT, BK>(a, s);
            return;
        }
    }
    const dim3 grid((unsigned)(a.B * a.H * nqb));
    if constexpr (is_relpos(BK)) {
        if (a.bias_f32) {
            launch_stream<NT, BK, true>(a, ntiles, grid, s);
            return;
        }
    }
    launch_stream<NT, BK, false>(a, ntiles, grid, s);
}

}  // namespace binattn
