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
//  * Rows of at most four tiles (N <= 256) take the exact row max: every tile is staged in
//    LDS at once, pass 1 computes the scores into registers and the max, pass 2 quantises
//    exp(S - max) and accumulates P^ V^ in int32 with no rescaling.  Longer rows stream
//    the tiles through a two-stage LDS ring with the FlashAttention-2 running max.
//  * p = 255 exp(S - m) = exp2(S log2e - m log2e + log2 255), P^ = rint(p) via
//    v_cvt_pk_u8_f32; the row sum is taken over the unquantised p.
//  * PV with signed int8 MFMA: sum P^ V^ = sum (P^-128) V^ + 2 * sum 64 V^; the two
//    64-weighted column sums are two more MFMAs into the same accumulator.
//  * Epilogue: O = acc * s_c / sum(p), s_c = a_c / 127 from the channel absmax a_c.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace binattn {

constexpr int kWaves = 4;
constexpr int kBR = kWaves * 16;            // queries per workgroup (16 per wave)
constexpr int kBC = 64;                     // keys per tile
constexpr int kRelposWin = 1024;            // fp32 entries of a staged relative-position window
constexpr int kKeepTiles = 4;               // rows of at most this many tiles: exact max, scores in registers
constexpr int kDeferTiles = 16;             // streamed rows of at least this many tiles accumulate in int32
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.99435343685886f;

enum { BK_NONE = 0, BK_DENSE_F16 = 1, BK_DENSE_F32 = 2, BK_RELPOS = 3 };

// Keys of one 64-key tile as A-operand rows: MFMA tile t, row m <-> key 16*(m/4) + 4t + (m%4).
// After the MFMA, lane (n, g) register r of tile t holds key 16g + 4t + r.
__device__ __forceinline__ int key_slot(int j, int& t) {
    t = (j & 15) >> 2;
    return 4 * (j >> 4) + (j & 3);
}

// V^ channels as A-operand rows of the PV MFMA: tile ct, row m <-> channel 4*NT*(m/4) + 4*ct + (m%4).
// After the MFMA, lane (query n, group g) register r of tile ct holds channel 4*NT*g + 4*ct + r.
template <int NT>
__device__ __forceinline__ int chan_slot(int c, int& ct) {
    const int q = c / (4 * NT), rem = c - q * (4 * NT);
    ct = rem >> 2;
    return 4 * q + (rem & 3);
}

// Raw global data of one tile held in registers between its load and its LDS store.
template <int NT, int TW>
struct TileRegs {
    static constexpr int W = (NT + 1) / 2;                 // sign words per key
    static constexpr int KT = (kBC * W + 255) / 256;       // K word tasks per thread
    static constexpr int VCH = (NT * 64 + 255) / 256;      // 16-byte V^ chunks per thread
    uint32_t kw[KT];
    uint4 v[VCH];
    float mu;
    float tw[TW / 256 > 0 ? TW / 256 : 1];
};

// LDS of one tile (a multiple of 16 bytes, so consecutive tiles keep 16-byte alignment).
// TW: fp32 entries of the tile's relative-position window (streamed rows), else 4.
template <int NT, int TW>
struct alignas(16) TileLds {
    static constexpr int W = (NT + 1) / 2;
    uint32_t k[4 * W * 16 * 8];            // [t][group][row] x 32 B: A operand of QK MFMA t, lane (row, group)
    uint32_t v[NT * kWave * 4];            // [ct][lane] x 16 B: A operand of PV MFMA ct
    float mu[kBC];
    float tw[TW];
};

struct RelposWin {
    int dr_lo, row_len, count;
};

// Rows of the relative-position table touched by queries [q0, q0+kBR) and keys [j0, j1).
__device__ __forceinline__ RelposWin relpos_window(int q0, int j0, int j1, int N, int gh, int gw) {
    const int ri_min = q0 / gw, ri_max = (min(q0 + kBR, N) - 1) / gw;
    const int rj_min = j0 / gw, rj_max = (min(j1, N) - 1) / gw;
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

// Loads PER window entries per thread (entry tid + 256 i) of a head's relative-position table,
// starting at element off, as fp32.  Entries past the table read as 0.
template <int PER>
__device__ __forceinline__ void load_window(float (&dst)[PER], const FwdArgs& a, const void* table, int off) {
    const int tid = threadIdx.x;
    const int tsz = (2 * a.gh - 1) * (2 * a.gw - 1);
    if (a.bias_f32) {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const float*)table + off, (tsz - off) * 4);
#pragma unroll
        for (int i = 0; i < PER; ++i)
            dst[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tr, (tid + 256 * i) * 4, 0, 0));
    } else {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const _Float16*)table + off, (tsz - off) * 2);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint16_t hbits = __builtin_amdgcn_raw_buffer_load_b16(tr, (tid + 256 * i) * 2, 0, 0);
            dst[i] = (float)__builtin_bit_cast(_Float16, hbits);
        }
    }
}

template <int NT, int TW>
__device__ __forceinline__ void load_tile(TileRegs<NT, TW>& r, const FwdArgs& a, const HeadPtrs& hp, int q0,
                                          int j0) {
    typedef TileRegs<NT, TW> R;
    const int tid = threadIdx.x, N = a.N, d = a.d;
    // sign words of keys j0.. (keys >= N read as 0)
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(hp.kb + j0 * R::W, (N - j0) * R::W * 4);
#pragma unroll
    for (int i = 0; i < R::KT; ++i)
        r.kw[i] = __builtin_amdgcn_raw_buffer_load_b32(kr, (tid + 256 * i) * 4, 0, 0);
    // V^ keys j0 .. j0+63 of every channel slot (channels >= d read as 0)
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
    if constexpr (TW >= 256) {
        const RelposWin w = relpos_window(q0, j0, j0 + kBC, N, a.gh, a.gw);
        load_window<TW / 256>(r.tw, a, hp.table, w.dr_lo * w.row_len);
    }
}

template <int NT, int TW>
__device__ __forceinline__ void store_tile(const TileRegs<NT, TW>& r, TileLds<NT, TW>& s, int d) {
    typedef TileRegs<NT, TW> R;
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
            int ct;
            const int m = chan_slot<NT>(c, ct);
            *reinterpret_cast<uint4*>(&s.v[(ct * kWave + m + 16 * gg) * 4]) = r.v[i];
        }
    }
    if (tid < kBC) s.mu[tid] = r.mu;
    if constexpr (TW >= 256) {
#pragma unroll
        for (int i = 0; i < TW / 256; ++i) s.tw[tid + 256 * i] = r.tw[i];
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

// The lane's query: Q operand, accumulator seed and scale.
struct LaneQ {
    v8i qop;
    v4f dseed;  // -sum of the query's signs
    float cq;   // mu_q / sqrt(d); 0 for a query past N
    int qi;     // query index (clamped to N-1)
    bool live;  // query < N
};

// Workgroup coordinates: (b*H + h, first query), with the XCD-aware block order.
template <int BIAS>
__device__ __forceinline__ void block_coords(const FwdArgs& a, int& bh, int& q0) {
    const int N = a.N;
    const int nqb = (N + kBR - 1) / kBR;
    const int nblk = a.B * a.H * nqb;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    int qb;
    if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) {
        // the dense bias is shared over the batch: keep the batch items of one (h, query block) together
        const int b = lb % a.B, hq = lb / a.B;
        qb = hq % nqb;
        bh = b * a.H + hq / nqb;
    } else {
        bh = lb / nqb;
        qb = lb % nqb;
    }
    q0 = qb * kBR;
}

template <int NT>
__device__ __forceinline__ LaneQ lane_query(const FwdArgs& a, int bh, int qw0, int g, int n16) {
    constexpr int W = (NT + 1) / 2;
    LaneQ lq;
    const int N = a.N;
    const int i = qw0 + n16;
    lq.live = i < N;
    lq.qi = lq.live ? i : N - 1;
    const float seed = load_q<W>(a.qbits + ((int64_t)bh * N + lq.qi) * W, lq.live, a.d, g, lq.qop);
    lq.dseed = v4f{seed, seed, seed, seed};
    lq.cq = lq.live ? a.qmu[(int64_t)bh * N + i] * a.qk_scale : 0.0f;
    return lq;
}

// Scores of one tile for one lane: S[k] for keys jg + k, k = 0..15, in natural units, keys >= N
// (k >= nvalid on the tail tile) set to -inf, and the running lane max mloc over them.
// sk/smu: the staged tile; zk: 16 rows x 32 zero bytes, the K operand of lanes whose channel
// group is past d.  win/idx0: relative-position window and the lane's index of key jg in it
// (the run's bias is win[idx0 - k]).
template <int NT, int BIAS>
__device__ __forceinline__ void tile_scores(const uint32_t* __restrict__ sk, const float* __restrict__ smu,
                                            const uint32_t* zk, const LaneQ& lq, const BiasRegs<BIAS>& bias,
                                            const float* win, int idx0, bool tail, int nvalid, float (&S)[16],
                                            float& mloc) {
    constexpr int W = (NT + 1) / 2;
    const int lane = threadIdx.x & 63, g = lane >> 4, m16 = lane & 15;
    v4f D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t* src = g < W ? &sk[((t * W + g) * 16 + m16) * 8] : zk + m16 * 8;
        const v4i lo = *reinterpret_cast<const v4i*>(src);
        const v4i hi = *reinterpret_cast<const v4i*>(src + 4);
        const v8i kop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        D[t] = mfma_f8(kop, lq.qop, lq.dseed);
    }
    float muk[16];
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&smu[16 * g + k]);
        muk[k] = m4.x; muk[k + 1] = m4.y; muk[k + 2] = m4.z; muk[k + 3] = m4.w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float b = 0.0f;
        if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) b = bias_at<BIAS>(bias, k);
        if (BIAS == BK_RELPOS) b = win[idx0 - k];
        S[k] = __builtin_fmaf(D[k >> 2][k & 3] * muk[k], lq.cq, b);
    }
    // The max is taken separately on the two paths: on the common one every S is an fma
    // result and needs no NaN canonicalisation before v_max3.
    if (tail) {  // ragged end: keys >= N take no weight
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (k >= nvalid) S[k] = -INFINITY;
#pragma unroll
        for (int k = 15; k > 0; k -= 2) mloc = fmaxf(fmaxf(mloc, S[k]), S[k - 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 16; k += 2) mloc = fmaxf(fmaxf(mloc, S[k]), S[k + 1]);
    }
}

// Quantised probabilities of one tile as the B operand of the PV MFMA (bytes P^ - 128) and
// their unquantised sum: p = 255 exp(S - m) with negm = log2(255) - m log2(e).
__device__ __forceinline__ v4i tile_probs(const float (&S)[16], float negm, float& lsum) {
    v4i pw;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t word = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(__builtin_fmaf(S[4 * t + r], kLog2e, negm));
            lsum += p;
            word = __builtin_amdgcn_cvt_pk_u8_f32(p, r, word);
        }
        pw[t] = (int)(word ^ 0x80808080u);
    }
    return pw;
}

constexpr v4i kC64 = v4i{0x40404040, 0x40404040, 0x40404040, 0x40404040};

// Dequantise, normalise and store the lane's 4*NT channels of its query.
template <int NT>
__device__ __forceinline__ void store_out(const FwdArgs& a, int bh, const LaneQ& lq, const float* sScale,
                                          const float (&acc)[NT][4], float L) {
    if (!lq.live) return;
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const int d = a.d, c0 = 4 * NT * g;
    const float inv = fast_rcp(L);
    const int64_t row = ((int64_t)bh * a.N + lq.qi) * d;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int c = c0 + 4 * ct;
        if (c >= d) continue;
        const float4 s4 = *reinterpret_cast<const float4*>(&sScale[c]);
        const float o0 = acc[ct][0] * s4.x * inv, o1 = acc[ct][1] * s4.y * inv;
        const float o2 = acc[ct][2] * s4.z * inv, o3 = acc[ct][3] * s4.w * inv;
        if (a.out_f32) {
            *reinterpret_cast<float4*>((float*)a.out + row + c) = make_float4(o0, o1, o2, o3);
        } else {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const h4 hv = h4{(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
            *reinterpret_cast<h4*>((_Float16*)a.out + row + c) = hv;
        }
    }
}

// Per-workgroup set-up shared by both kernels: the K zero block and the dequantisation
// scales s_c = a_c / 127 (IEEE division, as the oracle), 0 for channel slots past d.
__device__ __forceinline__ void stage_common(const FwdArgs& a, int bh, uint32_t* zk, float* sScale) {
    const int tid = threadIdx.x;
    if (tid < 16 * 8) zk[tid] = 0u;
    if (tid < 128) sScale[tid] = tid < a.d ? a.vamax[(int64_t)bh * a.d + tid] / 127.0f : 0.0f;
}

// ---------------------------------------------------------------------------------------------
// Rows of NTL <= kKeepTiles tiles (N <= 256): exact row max in two passes over register-resident
// scores.  A workgroup stages the K bits, mu_k and V^ of one (b, h) once and then loops over the
// query blocks [qb_lo, qb_hi) of that head (nsplit workgroups per head).  The next block's query
// words, dense-bias rows and relative-position window are loaded while the current block is
// computed, into registers the current block no longer needs.
template <int NT, int BIAS, int NTL>
__global__ __launch_bounds__(256) void binattn_fwd_keep_kernel(FwdArgs a, int nsplit) {
    constexpr int W = (NT + 1) / 2;
    constexpr bool DENSE = BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32;
    typedef TileRegs<NT, 4> Regs;
    typedef TileLds<NT, 4> Lds;
    __shared__ Lds lds[NTL];
    __shared__ __attribute__((aligned(16))) float sWin[BIAS == BK_RELPOS ? kRelposWin : 4];
    __shared__ __attribute__((aligned(16))) float sScale[128];
    __shared__ __attribute__((aligned(16))) uint32_t zk[16 * 8];

    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int lb = xcd_logical_block(blockIdx.x, a.B * a.H * nsplit);
    const int bh = lb / nsplit, split = lb % nsplit;
    const int qb_lo = split * nqb / nsplit, qb_hi = (split + 1) * nqb / nsplit;
    const int h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keeps row pointers scalar

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
    const int esz = BIAS == BK_DENSE_F32 ? 4 : 2;
    const int bvoff = (n16 * (int)a.bias_ld + 16 * g) * esz;

    // Per-block inputs of this lane: word g of its query's signs (0 past d or N) and mu_q.
    auto load_query = [&](int qb, uint32_t& qword, float& qmu) {
        const int i = qb * kBR + wave * 16 + n16;
        const bool live = i < N;
        qword = (live && g < W) ? a.qbits[((int64_t)bh * N + i) * W + g] : 0u;
        qmu = live ? a.qmu[(int64_t)bh * N + i] : 0.0f;
    };
    // Dense bias rows of this wave's 16 queries of block qb, every tile (rows >= N read 0).
    auto load_bias_rows = [&](int qb, BiasRegs<BIAS> (&bias)[NTL]) {
        const int r0 = min(qb * kBR + wave * 16, N);
        const char* brow = (const char*)a.bias + ((int64_t)h * N + r0) * a.bias_ld * esz;
        const int brow_bytes = min(N - r0, 16) * (int)a.bias_ld * esz;  // at most 16 rows: far below 2^31
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int j0 = t * kBC;
            load_bias<BIAS>(bias[t], buffer_rsrc(brow + j0 * esz, brow_bytes - j0 * esz), bvoff);
        }
    };
    // First table row of the relative-position window of block qb (every key touched).
    auto window_lo = [&](int qb) { return relpos_window(qb * kBR, 0, N, N, a.gh, a.gw).dr_lo; };

    // ---- stage the head once (all loads in flight together), then the first block's inputs
    {
        Regs regs[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) load_tile<NT, 4>(regs[t], a, hp, 0, t * kBC);
        stage_common(a, bh, zk, sScale);
#pragma unroll
        for (int t = 0; t < NTL; ++t) store_tile<NT, 4>(regs[t], lds[t], d);
    }
    float wv[kRelposWin / 256];
    if (BIAS == BK_RELPOS) {
        load_window<kRelposWin / 256>(wv, a, hp.table, window_lo(qb_lo) * (2 * a.gw - 1));
#pragma unroll
        for (int i = 0; i < kRelposWin / 256; ++i) sWin[tid + 256 * i] = wv[i];
    }
    uint32_t qword;
    float qmu;
    load_query(qb_lo, qword, qmu);
    BiasRegs<BIAS> bias[NTL];
    if (DENSE) load_bias_rows(qb_lo, bias);
    __syncthreads();

    for (int qb = qb_lo; qb < qb_hi; ++qb) {
        const int q0 = qb * kBR, qw0 = q0 + wave * 16;
        const bool live = qw0 < N;  // some query of this wave is < N (wave-uniform)
        const bool more = qb + 1 < qb_hi;
        if (BIAS == BK_RELPOS && more) load_window<kRelposWin / 256>(wv, a, hp.table, window_lo(qb + 1) * (2 * a.gw - 1));

        // the lane's query: Q operand (fp8 2*sign of channels 32g..32g+31, 0 past d) and seed
        LaneQ lq;
        {
            const int i = qw0 + n16;
            lq.live = i < N;
            lq.qi = lq.live ? i : N - 1;
            uint32_t o[8];
            unpack_signs32_f8x2(qword, o);
#pragma unroll
            for (int c = 0; c < 8; ++c) lq.qop[c] = (lq.live && g < W && 32 * g + 4 * c < d) ? (int)o[c] : 0;
            const float pos = rows4_sum((float)__builtin_popcount(qword));  // sign bits set over the query
            const float seed = lq.live ? (float)d - 2.0f * pos : 0.0f;
            lq.dseed = v4f{seed, seed, seed, seed};
            lq.cq = qmu * a.qk_scale;
        }
        int ri = 0, ci = 0, win_lo = 0;
        if (BIAS == BK_RELPOS) {
            ri = lq.qi / a.gw;
            ci = lq.qi % a.gw;
            win_lo = window_lo(qb);
        }

        // ---- pass 1: scores, row max, and the V^ column-sum term (128 * sum V^ per channel)
        float S[NTL][16];
        float mloc = -INFINITY;
        v4i acc[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
        if (live) {
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                const int jg = t * kBC + 16 * g;
                int idx0 = 0;
                if (BIAS == BK_RELPOS) {
                    const int rj = jg / a.gw, cj = jg % a.gw;
                    idx0 = (ri - rj + a.gh - 1 - win_lo) * (2 * a.gw - 1) + (ci - cj + a.gw - 1);
                    if (jg >= N) idx0 = 15;  // the whole run is past N and masked; keep reads in the window
                }
                tile_scores<NT, BIAS>(lds[t].k, lds[t].mu, zk, lq, bias[t], sWin, idx0, t == NTL - 1, N - jg,
                                      S[t], mloc);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const v4i vop = *reinterpret_cast<const v4i*>(&lds[t].v[(ct * kWave + lane) * 4]);
                    acc[ct] = mfma_i8(vop, kC64, acc[ct]);
                    acc[ct] = mfma_i8(vop, kC64, acc[ct]);
                }
                __builtin_amdgcn_sched_barrier(0);  // one tile's operands live at a time
            }
        }
        // the next block's query words and bias rows, into registers pass 1 has released
        if (more) {
            load_query(qb + 1, qword, qmu);
            if (DENSE) load_bias_rows(qb + 1, bias);
        }
        if (BIAS == BK_RELPOS) {
            __syncthreads();  // every wave is done with this block's window
            if (more) {
#pragma unroll
                for (int i = 0; i < kRelposWin / 256; ++i) sWin[tid + 256 * i] = wv[i];
            }
        }

        // ---- pass 2: P^ = rint(255 exp(S - m)), row sums, integer PV (no rescaling)
        if (live) {
            const float m = rows4_max(mloc);
            const float negm = kLog2_255 - m * kLog2e;
            float lsum = 0.0f;
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                const v4i pw = tile_probs(S[t], negm, lsum);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const v4i vop = *reinterpret_cast<const v4i*>(&lds[t].v[(ct * kWave + lane) * 4]);
                    acc[ct] = mfma_i8(vop, pw, acc[ct]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            float accf[NT][4];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) accf[ct][r] = (float)acc[ct][r];
            store_out<NT>(a, bh, lq, sScale, accf, rows4_sum(lsum));
        }
        if (BIAS == BK_RELPOS) __syncthreads();  // the next block's window is in place
    }
}

// ---------------------------------------------------------------------------------------------
// Longer rows: key tiles streamed through a two-stage LDS ring, FlashAttention-2 running max.
// DEFER: keep the PV sums in int32 across tiles and fold them into fp32 only when some row
// max of the wave moves (long rows, where that becomes rare).
template <int NT, int BIAS, bool DEFER>
__global__ __launch_bounds__(256) void binattn_fwd_stream_kernel(FwdArgs a) {
    constexpr int TW = BIAS == BK_RELPOS ? kRelposWin : 4;
    typedef TileRegs<NT, TW> Regs;
    typedef TileLds<NT, TW> Lds;
    __shared__ Lds lds[2];
    __shared__ __attribute__((aligned(16))) float sScale[128];
    __shared__ __attribute__((aligned(16))) uint32_t zk[16 * 8];

    const int N = a.N, d = a.d;
    int bh, q0;
    block_coords<BIAS>(a, bh, q0);
    const int h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntiles = (N + kBC - 1) / kBC;

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
    stage_common(a, bh, zk, sScale);

    const int qw0 = q0 + wave * 16;
    const bool wave_live = qw0 < N;
    const LaneQ lq = lane_query<NT>(a, bh, qw0, g, n16);
    int ri = 0, ci = 0;
    if (BIAS == BK_RELPOS) {
        ri = lq.qi / a.gw;
        ci = lq.qi % a.gw;
    }

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
    load_tile<NT, TW>(regs, a, hp, q0, 0);
    load_bias<BIAS>(b0, buffer_rsrc(brow, brow_bytes), bvoff);

    // One pipeline step: stage tile `tile` into LDS, issue the loads of tile+1, compute tile.
    // Unrolled by two so the two bias register sets alternate without copies.
    auto step = [&](int tile, BiasRegs<BIAS>& bcur, BiasRegs<BIAS>& bnext) {
        Lds& s = lds[tile & 1];
        store_tile<NT, TW>(regs, s, d);
        __syncthreads();
        if (tile + 1 < ntiles) {
            const int jn = (tile + 1) * kBC;
            load_tile<NT, TW>(regs, a, hp, q0, jn);
            load_bias<BIAS>(bnext, buffer_rsrc(brow + jn * esz, brow_bytes - jn * esz), bvoff);
        }
        if (!wave_live) return;
        const int j0 = tile * kBC, jg = j0 + 16 * g;
        int idx0 = 0;
        if (BIAS == BK_RELPOS) {
            const RelposWin w = relpos_window(q0, j0, j0 + kBC, N, a.gh, a.gw);
            const int rj = jg / a.gw, cj = jg % a.gw;
            idx0 = (ri - rj + a.gh - 1 - w.dr_lo) * w.row_len + (ci - cj + a.gw - 1);
            if (jg >= N) idx0 = 15;
        }
        float S[16], mloc = -INFINITY;
        tile_scores<NT, BIAS>(s.k, s.mu, zk, lq, bcur, s.tw, idx0, tile == ntiles - 1, N - jg, S, mloc);
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
    for (int tile = 0; tile < ntiles; tile += 2) {
        step(tile, b0, b1);
        if (tile + 1 < ntiles) step(tile + 1, b1, b0);
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
        store_tile<NT, 4>(r, lds, d);
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

// QK-tile probe: D_ij for every (query, key) by one of two methods, reduced per query row to
// max_j D_ij and sum_j D_ij (fp32, exact for these integer ranges), so that the cost of the
// tile itself is measured rather than the N^2 score writes.
//   METHOD 0: the forward's tile, fp8 MFMA on LDS-staged fp8 K operands;
//   METHOD 1: VALU XOR + v_bcnt on LDS-staged sign words, D = d - 2 popcount(q XOR k).
// Both hand D to the softmax stage as fp32 in the same lane layout (query n, keys 16g..16g+15).
template <int NT, int METHOD>
__global__ __launch_bounds__(256) void binattn_qk_stats_kernel(FwdArgs a, float* rowmax, float* rowsum) {
    constexpr int W = (NT + 1) / 2;
    typedef TileRegs<NT, 4> Regs;
    typedef TileLds<NT, 4> Lds;
    __shared__ Lds lds;
    __shared__ __attribute__((aligned(16))) uint32_t kraw[kBC * W];
    __shared__ __attribute__((aligned(16))) uint32_t zk[16 * 8];
    if (threadIdx.x < 16 * 8) zk[threadIdx.x] = 0u;
    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int lb = xcd_logical_block(blockIdx.x, a.B * a.H * nqb);
    const int bh = lb / nqb, qb = lb % nqb;
    const int tid = threadIdx.x, wave = tid >> 6, g = (tid & 63) >> 4, n16 = tid & 15;
    const int i = qb * kBR + wave * 16 + n16;
    const bool live = i < N;
    const uint32_t* qrow = a.qbits + ((int64_t)bh * N + (live ? i : N - 1)) * W;
    v8i qop;
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
                const uint32_t* src = g < W ? &lds.k[((t * W + g) * 16 + n16) * 8] : zk + n16 * 8;
                const v4i lo = *reinterpret_cast<const v4i*>(src);
                const v4i hi = *reinterpret_cast<const v4i*>(src + 4);
                const v4f x = mfma_f8(v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, qop, dseed);
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

// Whether the relative-position window of a whole short row (queries of one block, every key)
// fits the staged window; false sends the launch to the streaming kernel.
static bool keep_window_fits(const FwdArgs& a) {
    const int N = a.N, gw = a.gw, gh = a.gh;
    for (int q0 = 0; q0 < N; q0 += kBR) {
        const int ri_min = q0 / gw, ri_max = (min(q0 + kBR, N) - 1) / gw;
        if ((ri_max - ri_min + gh) * (2 * gw - 1) > kRelposWin) return false;
    }
    return true;
}

// Compute units of the current device (cached per device; 256 on MI355X).
static int device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int NT, int BK>
static void launch_fwd_bk(const FwdArgs& a, hipStream_t s) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    const int nqb = (a.N + kBR - 1) / kBR;
    if (ntiles <= kKeepTiles && (BK != BK_RELPOS || keep_window_fits(a))) {
        // enough workgroups for about three per compute unit, each looping over several query blocks
        const int64_t heads = (int64_t)a.B * a.H;
        const int64_t want = 3 * (int64_t)device_cus();
        const int nsplit = (int)std::min<int64_t>(nqb, std::max<int64_t>(1, (want + heads - 1) / heads));
        const dim3 grid((unsigned)(heads * nsplit));
        switch (ntiles) {
            case 1: hipLaunchKernelGGL((binattn_fwd_keep_kernel<NT, BK, 1>), grid, dim3(256), 0, s, a, nsplit); break;
            case 2: hipLaunchKernelGGL((binattn_fwd_keep_kernel<NT, BK, 2>), grid, dim3(256), 0, s, a, nsplit); break;
            case 3: hipLaunchKernelGGL((binattn_fwd_keep_kernel<NT, BK, 3>), grid, dim3(256), 0, s, a, nsplit); break;
            default: hipLaunchKernelGGL((binattn_fwd_keep_kernel<NT, BK, 4>), grid, dim3(256), 0, s, a, nsplit); break;
        }
        return;
    }
    const dim3 grid((unsigned)(a.B * a.H * nqb));
    if (ntiles >= kDeferTiles)
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((binattn_fwd_stream_kernel<NT, BK, false>), grid, dim3(256), 0, s, a);
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

}  // namespace binattn
