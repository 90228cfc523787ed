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
//  * QK^T on the fp8 MFMA (v_mfma_f32_16x16x128_f8f6f4; one instruction covers d <= 128).
//    With s = +-1 query signs and b = 0/1 key bits, s.t = sum s (2b - 1) = 2 s.b - sum(s):
//    the K operand is the bits as fp8 {0, 1}, the Q operand is fp8 {+-2}, and the
//    accumulator is seeded with -sum(s) of the lane's query.  Every product and partial
//    sum is a small integer, so the fp32 result is D exactly, already in float.
//  * The tile is computed transposed (keys are MFMA rows, queries columns) and the
//    key rows are permuted so that lane (query n, group g) holds the 16 consecutive
//    keys 16g..16g+15 of the tile for query n -- exactly the A-operand layout of the
//    int8 PV MFMA, so P never leaves registers, and the per-lane bias run is contiguous.
//  * K bits are unpacked once per workgroup per tile into LDS in MFMA-operand order
//    (each lane reads 32 consecutive bytes); V^ (channel-major in HBM) is staged the
//    same way.  LDS is double-buffered and the loads of tile t+1 are issued before
//    tile t is computed: one barrier per tile.  All global reads go through buffer
//    resources rebased per tile on the scalar unit, so addresses cost no vector ALU
//    and reads past a head's end return zero.
//  * Online softmax in fp32 with the running max reduced over the 4 lanes that
//    share a query (row-swap permutes).  p = 255 exp(S - m) =
//    exp2(S log2e - m log2e + log2 255), P^ = rint(p) via v_cvt_pk_u8_f32.
//  * PV with signed int8 MFMA: sum P^ V^ = sum (P^-128) V^ + 2 * sum 64 V^; the two
//    64-weighted column sums are two more MFMAs into the same accumulator.
//    Short rows fold each tile's int32 result into the fp32 accumulator (with the
//    running-max rescale); long rows keep accumulating in int32 across tiles and
//    fold only when some row max in the wave moves.
//  * Epilogue: O = acc * s_c / sum(p), s_c = a_c / 127 from the channel absmax a_c.
#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kWaves = 4;
constexpr int kBR = kWaves * 16;            // queries per workgroup (16 per wave)
constexpr int kBC = 64;                     // keys per tile
constexpr int kRelposWin = 1024;            // fp32 entries of the per-tile relative-position window
constexpr int kDeferTiles = 16;             // rows of at least this many tiles accumulate in int32
constexpr int kResTiles = 4;                // rows of at most this many tiles are staged whole in the prologue
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.99435343685886f;

enum { BK_NONE = 0, BK_DENSE_F16 = 1, BK_DENSE_F32 = 2, BK_RELPOS = 3 };

// Keys of one 64-key tile as A-operand rows: MFMA tile t, row m <-> key 16*(m/4) + 4t + (m%4).
// After the MFMA, lane (n, g) register r of tile t holds key 16g + 4t + r.
__device__ __forceinline__ int key_slot(int j, int& t) {
    t = (j & 15) >> 2;
    return 4 * (j >> 4) + (j & 3);
}

// Raw global data of one tile held in registers between its load and its LDS store.
template <int NT, int BIAS>
struct TileRegs {
    static constexpr int W = (NT + 1) / 2;                 // sign words per key
    static constexpr int KT = (kBC * W + 255) / 256;       // K word tasks per thread
    static constexpr int VCH = (NT * 64 + 255) / 256;      // 16-byte V^ chunks per thread
    static constexpr int TW = BIAS == BK_RELPOS ? kRelposWin / 256 : 1;
    uint32_t kw[KT];
    uint4 v[VCH];
    float mu;
    float tw[TW];
};

// LDS of one pipeline stage (a multiple of 16 bytes, so both stages keep 16-byte alignment).
template <int NT, int BIAS>
struct alignas(16) TileLds {
    static constexpr int W = (NT + 1) / 2;
    uint32_t k[4 * W * 16 * 8];            // [t][group][row] x 32 B: A operand of QK MFMA t, lane (row, group)
    uint32_t v[NT * kWave * 4];            // [ct][lane] x 16 B: B operand of PV MFMA ct
    float mu[kBC];
    float tw[BIAS == BK_RELPOS ? kRelposWin : 4];
};

struct RelposWin {
    int dr_lo, row_len, count;
};

// Rows of the relative-position table touched by queries [q0, q0+kBR) and keys [j0, j0+kBC).
__device__ __forceinline__ RelposWin relpos_window(int q0, int j0, int N, int gh, int gw) {
    const int ri_min = q0 / gw, ri_max = (min(q0 + kBR, N) - 1) / gw;
    const int rj_min = j0 / gw, rj_max = (min(j0 + kBC, N) - 1) / gw;
    RelposWin w;
    w.dr_lo = ri_min - rj_max + gh - 1;
    w.row_len = 2 * gw - 1;
    w.count = ((ri_max - ri_min) + (rj_max - rj_min) + 1) * w.row_len;
    return w;
}

// Per-workgroup pointers of one (b, h).
struct HeadPtrs {
    const uint32_t* kb;
    const float* kmu;
    const int8_t* vq;
    const void* table;  // relative-position table of head h
};

template <int NT, int BIAS>
__device__ __forceinline__ void load_tile(TileRegs<NT, BIAS>& r, const FwdArgs& a, const HeadPtrs& hp, int q0,
                                          int j0) {
    typedef TileRegs<NT, BIAS> R;
    const int tid = threadIdx.x, N = a.N, d = a.d;
    // sign words of keys j0.. (keys >= N read as 0)
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(hp.kb + j0 * R::W, (N - j0) * R::W * 4);
#pragma unroll
    for (int i = 0; i < R::KT; ++i)
        r.kw[i] = __builtin_amdgcn_raw_buffer_load_b32(kr, (tid + 256 * i) * 4, 0, 0);
    // V^ columns j0 .. j0+63 of every channel (channels >= d read as 0)
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(hp.vq + j0, d * (int)a.ldv - j0);
#pragma unroll
    for (int i = 0; i < R::VCH; ++i) {
        const int id = tid + 256 * i;
        const int c = id >> 2, gg = id & 3;
        const v4i x = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(vr, (int)(c * a.ldv) + 16 * gg, 0, 0));
        r.v[i] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    const __amdgpu_buffer_rsrc_t mr = buffer_rsrc(hp.kmu + j0, (N - j0) * 4);
    r.mu = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, (tid & 63) * 4, 0, 0));
    if (BIAS == BK_RELPOS) {
        const RelposWin w = relpos_window(q0, j0, N, a.gh, a.gw);
        const int tsz = (2 * a.gh - 1) * w.row_len;
        const int off = w.dr_lo * w.row_len;
        if (a.bias_f32) {
            const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const float*)hp.table + off, (tsz - off) * 4);
#pragma unroll
            for (int i = 0; i < r.TW; ++i)
                r.tw[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tr, (tid + 256 * i) * 4, 0, 0));
        } else {
            const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const _Float16*)hp.table + off, (tsz - off) * 2);
#pragma unroll
            for (int i = 0; i < r.TW; ++i) {
                const uint16_t hbits = __builtin_amdgcn_raw_buffer_load_b16(tr, (tid + 256 * i) * 2, 0, 0);
                r.tw[i] = (float)__builtin_bit_cast(_Float16, hbits);
            }
        }
    }
}

template <int NT, int BIAS>
__device__ __forceinline__ void store_tile(const TileRegs<NT, BIAS>& r, TileLds<NT, BIAS>& s, int d) {
    typedef TileRegs<NT, BIAS> R;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R::KT; ++i) {
        const int id = tid + 256 * i;
        if (id < kBC * R::W) {
            const int j = id / R::W, w = id % R::W;
            uint32_t word = r.kw[i];
            const int left = d - 32 * w;  // channels >= d contribute nothing
            if (left < 32) word &= (1u << left) - 1u;
            uint32_t o[8];
            unpack_bits32_f8(word, o);
            int t;
            const int m = key_slot(j, t);
            uint32_t* dst = &s.k[((t * R::W + w) * 16 + m) * 8];
            *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint4*>(dst + 4) = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
#pragma unroll
    for (int i = 0; i < R::VCH; ++i) {
        const int id = tid + 256 * i;
        if (id < NT * 64) {
            const int c = id >> 2, gg = id & 3;
            *reinterpret_cast<uint4*>(&s.v[((c >> 4) * kWave + (c & 15) + 16 * gg) * 4]) = r.v[i];
        }
    }
    if (tid < kBC) s.mu[tid] = r.mu;
    if (BIAS == BK_RELPOS) {
#pragma unroll
        for (int i = 0; i < r.TW; ++i) s.tw[tid + 256 * i] = r.tw[i];
    }
}

// Q operand (B of the QK MFMA) for one lane: fp8 2*sign of channels 32g .. 32g+31 (0 past d);
// returns -sum of the query's d signs (the accumulator seed), 0 for a query past N.
template <int W>
__device__ __forceinline__ float load_q(const uint32_t* __restrict__ qrow, bool live, int d, int g, v8i& q) {
    uint32_t o[8];
    const uint32_t word = (live && g < W) ? qrow[g] : 0u;
    unpack_signs32_f8x2(word, o);
#pragma unroll
    for (int c = 0; c < 8; ++c) q[c] = (live && g < W && 32 * g + 4 * c < d) ? (int)o[c] : 0;
    int pos = 0;
    if (live) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int left = d - 32 * w;
            const uint32_t mask = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
            pos += __builtin_popcount(qrow[w] & mask);
        }
    }
    return live ? (float)(d - 2 * pos) : 0.0f;  // -(pos - (d - pos))
}

// Dense bias of one lane for one tile: its query row, keys jg .. jg+15 (raw fp16 or fp32 words).
template <int BIAS>
struct BiasRegs {
    static constexpr int NV = BIAS == BK_DENSE_F32 ? 4 : (BIAS == BK_DENSE_F16 ? 2 : 1);
    v4i w[NV];
};

// rows: buffer over this wave's 16 query rows starting at key column j0 (rows past N read 0).
template <int BIAS>
__device__ __forceinline__ void load_bias(BiasRegs<BIAS>& b, __amdgpu_buffer_rsrc_t rows, int voff) {
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
#pragma unroll
        for (int k = 0; k < BiasRegs<BIAS>::NV; ++k)
            b.w[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rows, voff + 16 * k, 0, 0));
    }
}

template <int BIAS>
__device__ __forceinline__ float bias_at(const BiasRegs<BIAS>& b, int k) {
    if (BIAS == BK_DENSE_F16) {
        const uint32_t word = (uint32_t)b.w[k >> 3][(k >> 1) & 3];
        const uint16_t bits16 = (k & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
        return (float)__builtin_bit_cast(_Float16, bits16);
    } else {
        return __int_as_float(b.w[k >> 2][k & 3]);
    }
}

// Per-wave state carried across key tiles.
template <int NT>
struct WaveState {
    v8i qop;
    v4f dseed;                 // accumulator seed: -sum of the query's signs
    float cq, mrun, lpart;
    int qi;
    bool live;                 // some query of this wave is < N (wave-uniform)
    v4i acci[NT];              // deferred int32 PV accumulators (long rows)
    v4f accf[NT];
};

// zk: 16 rows x 32 zero bytes, the A operand of lanes whose channel group is past d.
template <int NT, int BIAS, bool DEFER>
__device__ __forceinline__ void tile_body(const FwdArgs& a, TileLds<NT, BIAS>& s, const uint32_t* zk,
                                          WaveState<NT>& st, const BiasRegs<BIAS>& bcur, int tile, int ntiles,
                                          int q0) {
    constexpr int W = (NT + 1) / 2;
    const int N = a.N;
    const int lane = threadIdx.x & 63, g = lane >> 4, m16 = lane & 15;
    const int j0 = tile * kBC;
    const int jg = j0 + 16 * g;  // first key of this lane's run

    // ---- QK^T: D exactly, in fp32
    v4f D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t* src = g < W ? &s.k[((t * W + g) * 16 + m16) * 8] : zk + m16 * 8;
        const v4i lo = *reinterpret_cast<const v4i*>(src);
        const v4i hi = *reinterpret_cast<const v4i*>(src + 4);
        const v8i kop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        D[t] = mfma_f8(kop, st.qop, st.dseed);
    }
    // ---- scale + bias
    float muk[16];
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&s.mu[16 * g + k]);
        muk[k] = m4.x; muk[k + 1] = m4.y; muk[k + 2] = m4.z; muk[k + 3] = m4.w;
    }
    int idx0 = 0;
    if (BIAS == BK_RELPOS) {
        const RelposWin w = relpos_window(q0, j0, N, a.gh, a.gw);
        const int gw = a.gw;
        const int ri = st.qi / gw, ci = st.qi % gw;
        const int rj = jg / gw, cj = jg % gw;
        idx0 = (ri - rj + a.gh - 1 - w.dr_lo) * w.row_len + (ci - cj + gw - 1);
        if (jg >= N) idx0 = 15;  // the whole run is past N and masked below; keep reads in the window
    }
    float sc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float b = 0.0f;
        if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) b = bias_at<BIAS>(bcur, k);
        if (BIAS == BK_RELPOS) b = s.tw[idx0 - k];
        sc[k] = __builtin_fmaf(D[k >> 2][k & 3] * muk[k], st.cq, b);
    }
    if (tile == ntiles - 1) {  // ragged tail: keys >= N take no weight
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (jg + k >= N) sc[k] = -INFINITY;
    }
    // ---- running max over the 64 keys of the tile (4 lanes share a query)
    float mloc = sc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mloc = fmaxf(mloc, sc[k]);
    const float mnew = fmaxf(st.mrun, rows4_max(mloc));
    const bool up = __any(mnew > st.mrun);
    float ar[4] = {1.0f, 1.0f, 1.0f, 1.0f};  // rescale of the O rows this lane holds (queries 4g + r)
    if (up) {
        const float alpha = fast_exp2((st.mrun - mnew) * kLog2e);  // 0 on the first tile
        st.lpart *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
        if (DEFER) {
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r) st.accf[ct][r] = (st.accf[ct][r] + (float)st.acci[ct][r]) * ar[r];
                st.acci[ct] = v4i{0, 0, 0, 0};
            }
        }
    }
    st.mrun = mnew;

    // ---- P^ = rint(255 exp(S - m)) - 128 as int8, row sums, integer PV
    const float negm = kLog2_255 - mnew * kLog2e;
    v4i pw;
    float lsum = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t word = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(__builtin_fmaf(sc[4 * t + r], kLog2e, negm));
            lsum += p;
            word = __builtin_amdgcn_cvt_pk_u8_f32(p, r, word);
        }
        pw[t] = (int)(word ^ 0x80808080u);
    }
    st.lpart += lsum;
    const v4i c64 = v4i{0x40404040, 0x40404040, 0x40404040, 0x40404040};
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const v4i vop = *reinterpret_cast<const v4i*>(&s.v[(ct * kWave + lane) * 4]);
        if (DEFER) {
            v4i acc = mfma_i8(pw, vop, st.acci[ct]);
            acc = mfma_i8(c64, vop, acc);
            st.acci[ct] = mfma_i8(c64, vop, acc);
        } else {
            v4i acc = mfma_i8(pw, vop, v4i{0, 0, 0, 0});
            acc = mfma_i8(c64, vop, acc);
            acc = mfma_i8(c64, vop, acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) st.accf[ct][r] = __builtin_fmaf(st.accf[ct][r], ar[r], (float)acc[r]);
        }
    }
}

template <int NT, int BIAS, bool DEFER, bool RES>
__global__ __launch_bounds__(256) void binattn_fwd_kernel(FwdArgs a) {
    constexpr int W = (NT + 1) / 2;
    typedef TileRegs<NT, BIAS> Regs;
    typedef TileLds<NT, BIAS> Lds;
    // RES: one LDS stage per tile of the whole (short) row; otherwise a two-stage ring
    __shared__ Lds lds[RES ? kResTiles : 2];
    __shared__ __attribute__((aligned(16))) uint32_t zk[16 * 8];
    if (threadIdx.x < 16 * 8) zk[threadIdx.x] = 0u;

    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    int bh, qb;
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
        // the dense bias is shared over the batch: keep the batch items of one (h, query block) together
        const int b = lb % a.B, hq = lb / a.B;
        qb = hq % nqb;
        bh = b * a.H + hq / nqb;
    } else {
        bh = lb / nqb;
        qb = lb % nqb;
    }
    const int h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keeps row pointers scalar
    const int q0 = qb * kBR;

    HeadPtrs hp;
    hp.kb = a.kbits + (int64_t)bh * N * W;
    hp.kmu = a.kmu + (int64_t)bh * N;
    hp.vq = a.vq + (int64_t)bh * d * a.ldv;
    hp.table = nullptr;
    if (BIAS == BK_RELPOS) {
        const int64_t tsz = (int64_t)(2 * a.gh - 1) * (2 * a.gw - 1);
        hp.table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz)
                              : (const void*)((const _Float16*)a.bias + h * tsz);
    }

    WaveState<NT> st;
    const int qw0 = q0 + wave * 16;  // first query of this wave
    {
        const int i = qw0 + n16;
        const bool live = i < N;
        st.live = qw0 < N;
        st.qi = live ? i : N - 1;
        const float seed = load_q<W>(a.qbits + ((int64_t)bh * N + st.qi) * W, live, d, g, st.qop);
        st.dseed = v4f{seed, seed, seed, seed};
        st.cq = live ? a.qmu[(int64_t)bh * N + i] * a.qk_scale : 0.0f;
        st.mrun = -INFINITY;
        st.lpart = 0.0f;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            st.acci[ct] = v4i{0, 0, 0, 0};
            st.accf[ct] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    // dense bias rows of this wave: row (h, qw0 + r) at offset r*ld elements; rows >= N read 0
    const int esz = BIAS == BK_DENSE_F32 ? 4 : 2;
    const char* brow = nullptr;
    int brow_bytes = 0;
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
        const int r0 = min(qw0, N);
        brow = (const char*)a.bias + ((int64_t)h * N + r0) * a.bias_ld * esz;
        brow_bytes = min(N - r0, 16) * (int)a.bias_ld * esz;  // at most 16 rows: far below 2^31
    }
    const int bvoff = (n16 * (int)a.bias_ld + 16 * g) * esz;

    const int ntiles = (N + kBC - 1) / kBC;
    // the scales of this lane's output channels, needed only at the end
    float vsc[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int c = ct * 16 + n16;
        vsc[ct] = c < d ? a.vamax[(int64_t)bh * d + c] / 127.0f : 0.0f;  // dequantisation scale, as fp32 a/127
    }
    BiasRegs<BIAS> b0, b1;
    if (RES) {
        // whole row on chip: every tile's loads in flight at once, then one barrier
        Regs regs[kResTiles];
#pragma unroll
        for (int t = 0; t < kResTiles; ++t)
            if (t < ntiles) load_tile<NT, BIAS>(regs[t], a, hp, q0, t * kBC);
        load_bias<BIAS>(b0, buffer_rsrc(brow, brow_bytes), bvoff);
#pragma unroll
        for (int t = 0; t < kResTiles; ++t)
            if (t < ntiles) store_tile<NT, BIAS>(regs[t], lds[t], d);
        __syncthreads();
        if (st.live) {
            // compute, with the next tile's bias in flight (two register sets, no copies)
            auto body = [&](int tile, BiasRegs<BIAS>& bcur, BiasRegs<BIAS>& bnext) {
                if (tile + 1 < ntiles) {
                    const int jn = (tile + 1) * kBC;
                    load_bias<BIAS>(bnext, buffer_rsrc(brow + jn * esz, brow_bytes - jn * esz), bvoff);
                }
                tile_body<NT, BIAS, DEFER>(a, lds[tile], zk, st, bcur, tile, ntiles, q0);
            };
#pragma unroll
            for (int tile = 0; tile < kResTiles; tile += 2) {
                if (tile < ntiles) body(tile, b0, b1);
                if (tile + 1 < ntiles) body(tile + 1, b1, b0);
            }
        }
    } else {
        Regs regs;
        load_tile<NT, BIAS>(regs, a, hp, q0, 0);
        load_bias<BIAS>(b0, buffer_rsrc(brow, brow_bytes), bvoff);

        // One pipeline step: stage tile `tile` into LDS, issue the loads of tile+1, compute tile.
        // Unrolled by two so the two bias register sets alternate without copies.
        auto step = [&](int tile, BiasRegs<BIAS>& bcur, BiasRegs<BIAS>& bnext) {
            Lds& s = lds[tile & 1];
            store_tile<NT, BIAS>(regs, s, d);
            __syncthreads();
            if (tile + 1 < ntiles) {
                const int jn = (tile + 1) * kBC;
                load_tile<NT, BIAS>(regs, a, hp, q0, jn);
                load_bias<BIAS>(bnext, buffer_rsrc(brow + jn * esz, brow_bytes - jn * esz), bvoff);
            }
            if (st.live) tile_body<NT, BIAS, DEFER>(a, s, zk, st, bcur, tile, ntiles, q0);
        };
        for (int tile = 0; tile < ntiles; tile += 2) {
            step(tile, b0, b1);
            if (tile + 1 < ntiles) step(tile + 1, b1, b0);
        }
    }

    // ---- epilogue: O = acc * s_c / sum(p)
    if (!st.live) return;
    const float L = rows4_sum(st.lpart);
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) inv[r] = fast_rcp(__shfl(L, 4 * g + r));
    const int ibase = qw0 + 4 * g;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int c = ct * 16 + n16;
        if (c >= d) continue;
        const float sv = vsc[ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ibase + r;
            if (i >= N) continue;
            const float acc = DEFER ? st.accf[ct][r] + (float)st.acci[ct][r] : st.accf[ct][r];
            const float o = acc * sv * inv[r];
            const int64_t off = ((int64_t)bh * N + i) * d + c;
            if (a.out_f32)
                ((float*)a.out)[off] = o;
            else
                ((_Float16*)a.out)[off] = (_Float16)o;
        }
    }
}

// Integer score export through the same K staging, Q operand and QK tile as the forward kernel.
template <int NT>
__global__ __launch_bounds__(256) void binattn_scores_kernel(FwdArgs a) {
    constexpr int W = (NT + 1) / 2;
    typedef TileRegs<NT, BK_NONE> Regs;
    typedef TileLds<NT, BK_NONE> Lds;
    __shared__ Lds lds;
    __shared__ __attribute__((aligned(16))) uint32_t zk[16 * 8];
    if (threadIdx.x < 16 * 8) zk[threadIdx.x] = 0u;
    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    const int bh = lb / nqb, qb = lb % nqb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int q0 = qb * kBR;
    v8i qop;
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
        store_tile<NT, BK_NONE>(r, lds, d);
        __syncthreads();
        v4f D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t* src = g < W ? &lds.k[((t * W + g) * 16 + n16) * 8] : zk + n16 * 8;
            const v4i lo = *reinterpret_cast<const v4i*>(src);
            const v4i hi = *reinterpret_cast<const v4i*>(src + 4);
            const v8i kop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            D[t] = mfma_f8(kop, qop, dseed);
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

template <int NT, int BK>
static void launch_fwd_bk(const FwdArgs& a, dim3 grid, hipStream_t s) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    if (ntiles <= kResTiles)
        hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK, false, true>), grid, dim3(256), 0, s, a);
    else if (ntiles >= kDeferTiles)
        hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK, true, false>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((binattn_fwd_kernel<NT, BK, false, false>), grid, dim3(256), 0, s, a);
}

template <int NT>
static hipError_t launch_fwd_nt(const FwdArgs& a, int bk, hipStream_t s) {
    const int nqb = (a.N + kBR - 1) / kBR;
    const dim3 grid((unsigned)(a.B * a.H * nqb));
    switch (bk) {
        case BK_NONE: launch_fwd_bk<NT, BK_NONE>(a, grid, s); break;
        case BK_DENSE_F16: launch_fwd_bk<NT, BK_DENSE_F16>(a, grid, s); break;
        case BK_DENSE_F32: launch_fwd_bk<NT, BK_DENSE_F32>(a, grid, s); break;
        default: launch_fwd_bk<NT, BK_RELPOS>(a, grid, s); break;
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

// Whether the relative-position window any tile of a forward launch stages fits on chip
// (an upper bound on the table rows one query block and one key tile touch).
bool relpos_window_fits(int gw) {
    const int rows = (kBR - 1) / gw + 1 + (kBC - 1) / gw + 1 + 1;
    return rows * (2 * gw - 1) <= kRelposWin;
}

}  // namespace binattn
