// tile.h -- device building blocks of the BinaryAttention forward kernels (tile staging,
// Q operand, bias, score tile, quantised probabilities, epilogue), the head-resident kernel and
// its launch plan, shared by the forward from packed inputs and the whole-attention path.
#pragma once

#include <algorithm>
#include <functional>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"
#include "prep.h"

namespace binattn {

constexpr int kWaves = 4;
constexpr int kBR = kWaves * 16;            // queries per workgroup (16 per wave)
constexpr int kBC = 64;                     // keys per tile
constexpr int kRelposWin = 1024;            // fp32 entries of a staged relative-position window
constexpr int kKeepTiles = 4;               // rows of at most this many tiles: exact max, scores in registers
constexpr int kLongTiles = 10;              // d <= 64: rows of up to this many tiles take the same kernel
constexpr int kDeferTiles = 16;             // streamed rows of at least this many tiles accumulate in int32
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.99435343685886f;

// Bias kinds of the kernels: none, dense fp16 / fp32, relative position on grids whose width
// is a multiple of 16 (a lane's 16-key run lies in one grid row, so its table entries are
// consecutive), and relative position on any other grid (RELPOS_G: each key's table offset is
// staged in LDS and gathered per element).
enum { BK_NONE = 0, BK_DENSE_F16 = 1, BK_DENSE_F32 = 2, BK_RELPOS = 3, BK_RELPOS_G = 4 };
constexpr bool is_relpos(int bk) { return bk == BK_RELPOS || bk == BK_RELPOS_G; }
inline int relpos_kind(int gw) { return gw % 16 == 0 ? BK_RELPOS : BK_RELPOS_G; }

// How the short-row kernel splits the query blocks of a head over workgroups: `a` segments of f
// blocks, then `b` segments of r blocks (the last segment of each kind clipped to the row).
struct KeepPlan {
    int a, f, b, r;
};

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
    uint32_t tw[TW / 256 > 0 ? TW / 256 : 1];  // raw table bits (fp16 or fp32), converted when stored
};

// LDS of one tile (a multiple of 16 bytes, so consecutive tiles keep 16-byte alignment).
// TW: fp32 entries of the tile's relative-position window (streamed rows), else 4.
template <int NT, int TW>
struct alignas(16) TileLds {
    static constexpr int W = (NT + 1) / 2;
    uint32_t k[4 * W * 16 * 4];            // [t][group][row] x 16 B: fp4 A operand of QK MFMA t, lane (row, group)
    uint32_t v[NT * kWave * 4];            // [ct][lane] x 16 B: A operand of PV MFMA ct
    float mu[kBC];
    float tw[TW];
    int kk[TW >= 256 ? kBC : 4];           // streamed relative position, any grid: per key, its window byte offset
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

// Loads entries off + eo[i] (i < PER) of a head's relative-position table as fp32; entries past
// the table read as 0.
template <int PER>
__device__ __forceinline__ void load_window_at(float (&dst)[PER], const FwdArgs& a, const void* table, int off,
                                               const int (&eo)[PER]) {
    const int tsz = (2 * a.gh - 1) * (2 * a.gw - 1);
    if (a.bias_f32) {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const float*)table + off, (tsz - off) * 4);
#pragma unroll
        for (int i = 0; i < PER; ++i)
            dst[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tr, eo[i] * 4, 0, 0));
    } else {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const _Float16*)table + off, (tsz - off) * 2);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint16_t hbits = __builtin_amdgcn_raw_buffer_load_b16(tr, eo[i] * 2, 0, 0);
            dst[i] = (float)__builtin_bit_cast(_Float16, hbits);
        }
    }
}

// Raw bits of PER window entries per thread (entry tid + 256 i) of a head's relative-position
// table from element off; entries past the table read as 0.  Left unconverted so that no wait
// for these loads sits where they are issued.
template <int PER>
__device__ __forceinline__ void load_window_raw(uint32_t (&dst)[PER], const FwdArgs& a, const void* table, int off) {
    const int tsz = (2 * a.gh - 1) * (2 * a.gw - 1);
    if (a.bias_f32) {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const float*)table + off, (tsz - off) * 4);
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b32(tr, (threadIdx.x + 256 * i) * 4, 0, 0);
    } else {
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const _Float16*)table + off, (tsz - off) * 2);
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b16(tr, (threadIdx.x + 256 * i) * 2, 0, 0);
    }
}

template <bool F32>
__device__ __forceinline__ float table_value(uint32_t raw) {
    return F32 ? __uint_as_float(raw) : (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
}

// Loads of key tile j0 into registers: sign words, V^ chunks, mu_k and (TW >= 256) the
// relative-position window starting at table element woff.
template <int NT, int TW>
__device__ __forceinline__ void load_tile(TileRegs<NT, TW>& r, const FwdArgs& a, const HeadPtrs& hp, int j0,
                                          int woff) {
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
    if constexpr (TW >= 256) load_window_raw<TW / 256>(r.tw, a, hp.table, woff);
}

// NARROW: the tile holds at most 16 valid keys (the last tile of a row) and is staged for the
// narrow score tile: key j is K operand row j of MFMA 0, and the V^ dword of keys 4q..4q+3 is the
// first dword of operand lane (slot, q) -- those lanes' other bytes meet zero P^ bytes.
// TF32: the relative-position table (TW >= 256) is fp32, else fp16.
// SWZ (streamed tiles, staged once per tile by the whole workgroup): the 16-byte operand rows are
// stored with their index XOR-swizzled within each aligned group of eight -- K rows of sign word w
// at row ^ 4 (w & 1), V^ rows of key chunk gg at row ^ 2 gg -- so that every eight lanes of a
// staging store hit eight different bank groups (the readers apply the same XOR to their rows).
template <int NT, int TW, bool NARROW = false, bool TF32 = false, bool SWZ = false>
__device__ __forceinline__ void store_tile(const TileRegs<NT, TW>& r, TileLds<NT, TW>& s, int d) {
    typedef TileRegs<NT, TW> R;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R::KT; ++i) {
        const int id = tid + 256 * i;
        if (id < (NARROW ? 16 : kBC) * R::W) {
            const int j = id / R::W, w = id % R::W;
            uint32_t word = r.kw[i];
            const int left = d - 32 * w;  // channels >= d contribute nothing
            if (left < 32) word &= (1u << left) - 1u;
            uint32_t o[4];
            unpack_bits32_f4(word, o);
            int t = 0, m = j;
            if (!NARROW) m = key_slot(j, t);
            if (SWZ) m ^= 4 * (w & 1);
            *reinterpret_cast<uint4*>(&s.k[((t * R::W + w) * 16 + m) * 4]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < R::VCH; ++i) {
        const int id = tid + 256 * i;
        if (id < NT * 64) {
            const int c = id >> 2, gg = id & 3;
            int ct;
            const int m = chan_slot<NT>(c, ct);
            if (!NARROW) {
                *reinterpret_cast<uint4*>(&s.v[(ct * kWave + ((m + 16 * gg) ^ (SWZ ? 2 * gg : 0))) * 4]) = r.v[i];
            } else if (gg == 0) {
                const uint4 x = r.v[i];
                s.v[(ct * kWave + m) * 4] = x.x;
                s.v[(ct * kWave + m + 16) * 4] = x.y;
                s.v[(ct * kWave + m + 32) * 4] = x.z;
                s.v[(ct * kWave + m + 48) * 4] = x.w;
            }
        }
    }
    if (tid < kBC) s.mu[tid] = r.mu;
    if constexpr (TW >= 256) {
#pragma unroll
        for (int i = 0; i < TW / 256; ++i) s.tw[tid + 256 * i] = table_value<TF32>(r.tw[i]);
    }
}

// Column sums of V^ for the u8 offset of P^: sum_j P^_j V^_jc = sum_j (P^_j - 128) V^_jc +
// 128 sum_j V^_jc, and the second term does not depend on the query.  colsum_add adds the
// sums of the 16-key chunks a thread stages (one channel slot per chunk); colsum_store
// reduces the four chunks of a slot (four consecutive lanes) and writes 128 * sum per slot.
template <int NT, int TW>
__device__ __forceinline__ void colsum_add(const TileRegs<NT, TW>& r, int (&cs)[TileRegs<NT, TW>::VCH]) {
#pragma unroll
    for (int i = 0; i < TileRegs<NT, TW>::VCH; ++i) {
        const uint4 x = r.v[i];
        int sum = __builtin_amdgcn_sdot4((int)x.x, 0x01010101, 0, false);
        sum = __builtin_amdgcn_sdot4((int)x.y, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)x.z, 0x01010101, sum, false);
        cs[i] += __builtin_amdgcn_sdot4((int)x.w, 0x01010101, sum, false);
    }
}

template <int NT, int VCH>
__device__ __forceinline__ void colsum_store(const int (&cs)[VCH], int* sCol) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
        const int id = threadIdx.x + 256 * i;
        int v = cs[i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if (id < NT * 64 && (id & 3) == 0) sCol[id >> 2] = 128 * v;
    }
}

// Q operand (B of the QK MFMA) for one lane from word g of its query's signs: fp4 2*sign of
// channels 32g .. 32g+31; all zero for a group wholly past d (whose lanes read group 0's K rows).
// Channels past d inside the last group keep a nonzero code: their K codes are 0 (the K words
// are masked to d before unpacking), so those products vanish.
__device__ __forceinline__ v4i q_operand(uint32_t word, bool live, int d, int g) {
    uint32_t o[4];
    unpack_signs32_f4x2(word, o);
    v4i q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (live && 32 * g < d) ? (int)o[i] : 0;
    return q;
}

// Q operand of one lane read from its packed row; returns -sum of the query's d signs (the
// accumulator seed), 0 for a query past N.
template <int W>
__device__ __forceinline__ float load_q(const uint32_t* __restrict__ qrow, bool live, int d, int g, v4i& q) {
    q = q_operand((live && g < W) ? qrow[g] : 0u, live && g < W, d, g);
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
    v4i qop;
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

// The lane's query packed in the kernel's own prologue from fp16 / fp32 Q (a.qx): its sign word g
// and mu_q with pack_wave's arithmetic -- the same sign test, the same per-chunk partial |x| sums,
// added in channel order (lanes g = 0, 1, .. add theirs in turn) -- so that the packed path and
// this one agree bit for bit ("BinaryAttention" paper notes, key design 1).
template <int NT>
__device__ __forceinline__ LaneQ lane_query_raw(const FwdArgs& a, int bh, int qw0, int g, int n16) {
    constexpr int W = (NT + 1) / 2;
    LaneQ lq;
    const int N = a.N, d = a.d, cpt = d >> 3;
    const int i = qw0 + n16;
    lq.live = i < N;
    lq.qi = lq.live ? i : N - 1;
    const int64_t row = ((int64_t)bh * N + lq.qi) * d;
    uint4 v[8];  // chunks 4 g .. 4 g + 3 (fp16: one 16-byte load each; fp32: two)
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (4 * g + c < cpt) {
            if (a.qx_f32) {
                const float* x = static_cast<const float*>(a.qx) + row + 8 * (4 * g + c);
                v[2 * c] = *reinterpret_cast<const uint4*>(x);
                v[2 * c + 1] = *reinterpret_cast<const uint4*>(x + 4);
            } else {
                v[c] = *reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.qx) + row + 8 * (4 * g + c));
            }
        }
    }
    uint32_t word = 0;
    float psum[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint32_t byte = 0;
        float sum = 0.0f;
        if (a.qx_f32) {
            const uint32_t w8[8] = {v[2 * c].x, v[2 * c].y, v[2 * c].z, v[2 * c].w,
                                    v[2 * c + 1].x, v[2 * c + 1].y, v[2 * c + 1].z, v[2 * c + 1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = __uint_as_float(w8[e]);
                byte |= (f >= 0.0f ? 1u : 0u) << e;  // -0.0 >= 0 holds: zero counts as +1
                sum += fabsf(f);
            }
        } else {
            chunk_sign_abs(__builtin_bit_cast(h8, v[c]), byte, sum);
        }
        psum[c] = sum;
        if (4 * g + c < cpt) word |= byte << (8 * c);
    }
    float acc = 0.0f;
#pragma unroll
    for (int gg = 0; gg < W; ++gg) {
        if (g == gg) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * g + c < cpt) acc += psum[c];
        }
        acc = __shfl(acc, 16 * gg + n16);
    }
    lq.qop = q_operand(word, lq.live && g < W, d, g);
    const float pos = rows4_sum((float)__builtin_popcount(g < W ? word : 0u));  // sign bits set over the query
    const float seed = lq.live ? (float)d - 2.0f * pos : 0.0f;
    lq.dseed = v4f{seed, seed, seed, seed};
    lq.cq = lq.live ? acc / (float)d * a.qk_scale : 0.0f;
    return lq;
}

// Scores of one tile for one lane: S[k] for keys jg + k, k = 0..15, in natural units, keys >= N
// (k >= nvalid on the tail tile) set to -inf, and the running lane max mloc over them.
// sk/smu: the staged tile.  Lanes whose channel group g is past d read the operand rows of group
// 0: their Q operand is zero, so those products vanish whatever the K codes are (every fp4 code
// is finite).  wrun: relative-position window entry of key jg + 15 (the run's bias for key jg + k
// is wrun[15 - k]: a grid row holds whole runs, and the column offset falls as the key rises).
// RELPOS_G: wrun is the window entry of the lane's query part, and kk (LDS) holds the byte
// offsets from it of the entries of keys jg .. jg + 15 (any grid width).
template <int NT, int BIAS, bool SWZ = false>
__device__ __forceinline__ void tile_scores(const uint32_t* __restrict__ sk, const float* __restrict__ smu,
                                            const LaneQ& lq, const BiasRegs<BIAS>& bias, const float* wrun,
                                            bool tail, int nvalid, float (&S)[16], float& mloc,
                                            const int* kk = nullptr) {
    constexpr int W = (NT + 1) / 2;
    const int lane = threadIdx.x & 63, g = lane >> 4, m16 = lane & 15;
    const int gw = g < W ? g : 0;
    const int koff = (gw * 16 + (SWZ ? m16 ^ (4 * (gw & 1)) : m16)) * 4;  // lane-constant
    v4f D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) D[t] = mfma_f4(*reinterpret_cast<const v4i*>(&sk[t * W * 64 + koff]), lq.qop, lq.dseed);
    // the run's window entries through one base register and immediate offsets (the window's own
    // LDS offset is beyond the reach of the read-pair offsets, and folded into it every pair
    // would take an address add)
    typedef const float __attribute__((address_space(3)))* lds_cfptr;
    lds_cfptr wl = (lds_cfptr)wrun;
    if (BIAS == BK_RELPOS) asm volatile("" : "+v"(wl));
    float muk[16];
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&smu[16 * g + k]);
        muk[k] = m4.x; muk[k + 1] = m4.y; muk[k + 2] = m4.z; muk[k + 3] = m4.w;
    }
    int koffs[BIAS == BK_RELPOS_G ? 16 : 1];
    if constexpr (BIAS == BK_RELPOS_G) {
#pragma unroll
        for (int k = 0; k < 16; k += 4) {
            const int4 o4 = *reinterpret_cast<const int4*>(&kk[k]);
            koffs[k] = o4.x; koffs[k + 1] = o4.y; koffs[k + 2] = o4.z; koffs[k + 3] = o4.w;
        }
    }
    typedef const char __attribute__((address_space(3)))* lds_ccptr;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float b = 0.0f;
        if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) b = bias_at<BIAS>(bias, k);
        if (BIAS == BK_RELPOS) b = wl[15 - k];
        if constexpr (BIAS == BK_RELPOS_G) b = *(lds_cfptr)((lds_ccptr)wrun + koffs[k]);
        S[k] = __builtin_fmaf(D[k >> 2][k & 3] * muk[k], lq.cq, b);
    }
    // The max is taken separately on the two paths: on the common one every S is an fma
    // result and needs no NaN canonicalisation before v_max3.
    if (tail) {  // ragged end: keys >= N take no weight
        // (the empty asm keeps this a branch of its own: without it the compiler turns the
        // masking of every tile into selects on lane masks it hoists out of the block loop)
        int nv = nvalid;
        asm volatile("" : "+v"(nv));
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (k >= nv) S[k] = -INFINITY;
#pragma unroll
        for (int k = 15; k > 0; k -= 2) mloc = fmaxf(fmaxf(mloc, S[k]), S[k - 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 16; k += 2) mloc = fmaxf(fmaxf(mloc, S[k]), S[k + 1]);
    }
}

// Quantised probabilities of one tile as the B operand of the PV MFMA and their unquantised sum:
// p = 255 exp(S - m) with negm = log2(255) - m log2(e).  Bytes P^ ^ FLIP as int8: FLIP = 0x80
// gives P^ - 128; FLIP = 0x7F gives 127 - P^ (for every P^ in 0..255).
template <uint32_t FLIP = 0x80808080u>
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
        pw[t] = (int)(word ^ FLIP);
    }
    return pw;
}

// The narrow last tile (at most 16 valid keys, staged by store_tile<..., true>): one MFMA, lane
// (query n, group g) holds keys jg + r, jg = j0 + 4g, r = 0..3; keys >= N (r >= nvalid) get -inf.
// bias: loaded at key column jg (bias_at r < 4); wrun: window entry of key jg + 3.
template <int NT, int BIAS>
__device__ __forceinline__ void tile_scores4(const uint32_t* __restrict__ sk, const float* __restrict__ smu,
                                             const LaneQ& lq, const BiasRegs<BIAS>& bias, const float* wrun,
                                             int nvalid, float (&S)[4], float& mloc) {
    constexpr int W = (NT + 1) / 2;
    const int lane = threadIdx.x & 63, g = lane >> 4, m16 = lane & 15;
    const int koff = ((g < W ? g : 0) * 16 + m16) * 4;
    const v4f D = mfma_f4(*reinterpret_cast<const v4i*>(&sk[koff]), lq.qop, lq.dseed);
    typedef const float __attribute__((address_space(3)))* lds_cfptr;
    lds_cfptr wl = (lds_cfptr)wrun;
    if (BIAS == BK_RELPOS) asm volatile("" : "+v"(wl));
    const float4 m4 = *reinterpret_cast<const float4*>(&smu[4 * g]);
    const float muk[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float b = 0.0f;
        if (BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32) b = bias_at<BIAS>(bias, r);
        if (BIAS == BK_RELPOS) b = wl[3 - r];
        S[r] = r < nvalid ? __builtin_fmaf(D[r] * muk[r], lq.cq, b) : -INFINITY;
    }
    mloc = fmaxf(fmaxf(mloc, S[0]), S[1]);
    mloc = fmaxf(fmaxf(mloc, S[2]), S[3]);
}

// P^ - 128 of the narrow tile in the first dword of the lane's PV operand, zeros after it.
__device__ __forceinline__ v4i tile_probs4(const float (&S)[4], float negm, float& lsum) {
    uint32_t word = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(S[r], kLog2e, negm));
        lsum += p;
        word = __builtin_amdgcn_cvt_pk_u8_f32(p, r, word);
    }
    return v4i{(int)(word ^ 0x80808080u), 0, 0, 0};
}

constexpr v4i kCm127 = v4i{(int)0x81818181, (int)0x81818181, (int)0x81818181, (int)0x81818181};  // int8 -127

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

// Per-workgroup set-up shared by both kernels: the dequantisation scales s_c = a_c / 127
// (IEEE division, as the oracle), 0 for channel slots past d.
__device__ __forceinline__ void stage_common(const FwdArgs& a, int bh, float* sScale) {
    const int tid = threadIdx.x;
    if (tid < 128) sScale[tid] = tid < a.d ? a.vamax[(int64_t)bh * a.d + tid] / 127.0f : 0.0f;
}

// Whole-attention staging of one (b, h) from fp16 Q, K, V, done by the short-row kernel itself:
// K -> sign bits as fp4 operand rows and mu_k (one key per thread); V -> channel absmax,
// dequantisation scales and int8 V^ written straight into the operand rows (V held in
// registers in groups of 4 tokens, transposed with v_perm); the Q of the workgroup's query
// blocks -> sign word g and mu_q per lane (sQw, sQmu).  The arithmetic is that of
// pack_wave and quant_head_regs -- the same comparisons, the same fp32 summation order for
// mu, the same IEEE 127/a and rint -- so the results equal the separate path bit for bit.
// sRed: 2048 floats; sInv, sAmx: 128 words; sCol: 128 * sum_j V^_jc per channel slot (16 NT).
// The per-channel reductions (absmax, column sum) take 256/d threads per channel, which meet in
// an LDS max / add.
template <int NT, int NTL, bool NARROW>
__device__ __forceinline__ void fused_stage(const FwdArgs& a, int bh, int qb_lo, int nitems, TileLds<NT, 4>* lds,
                                            float* sScale, uint32_t* sQw, float* sQmu, float* sRed,
                                            float* sInv, uint32_t* sAmx, int* sCol) {
    constexpr int W = (NT + 1) / 2;
    constexpr int MAXCK = 2 * NT;  // 8-channel chunks of one key (d <= 16 NT)
    constexpr int MAXC = 16;       // V chunks per thread: 4 * ceil(64 / G) with G = 256 / (d/8) >= 16
    const int N = a.N, d = a.d, tid = threadIdx.x;
    const int cpt = d >> 3;
    // operand padding (keys >= N, channel slots >= d) stays zero
    for (int id = tid; id < NTL * NT * 64; id += 256)
        reinterpret_cast<uint4*>(lds[id / (NT * 64)].v)[id % (NT * 64)] = make_uint4(0, 0, 0, 0);
    if (tid < 128) {
        sAmx[tid] = 0u;  // max of non-negative floats, compared as bit patterns
        sCol[tid] = 0;
    }

    // ---- the K and V loads of the head in flight together.  Buffer loads: rows past N read
    // as zero and no load sits under a lane-dependent branch (so no load is waited for early).
    const int hbytes = N * d * 2;  // at most 256 * 128 * 2
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(a.k_raw + (int64_t)bh * N * d, hbytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(a.v_raw + (int64_t)bh * N * d, hbytes);
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(a.q_raw + (int64_t)bh * N * d, hbytes);
    auto load16 = [](__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    };
    const int j = tid;  // this thread's key
    h8 kx[MAXCK];
#pragma unroll
    for (int c = 0; c < MAXCK; ++c)
        if (c < cpt) kx[c] = load16(kr, j * d * 2 + 16 * c);  // uniform condition
    const int P = cpt, G = 256 / P;
    const int part = tid % P, grp = tid / P;
    h8 vx[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int n = 4 * (grp + G * (i >> 2)) + (i & 3);
        vx[i] = load16(vr, grp < G ? n * d * 2 + part * 16 : hbytes);  // past N (or idle thread): 0
    }
    const int lane = tid & 63, g = lane >> 4, n16 = lane & 15, wave = tid >> 6;
    __syncthreads();  // the zero fill is complete before any operand row is written

    // ---- K: sign bytes and partial |x| sums per chunk, words, mu_k (pack_wave's order)
    if (j < NTL * kBC) {
        uint32_t words[W];
#pragma unroll
        for (int w = 0; w < W; ++w) words[w] = 0u;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < MAXCK; ++c) {
            if (c < cpt) {
                uint32_t byte;
                float sum;
                chunk_sign_abs(kx[c], byte, sum);
                acc += sum;
                words[c >> 2] |= byte << (8 * (c & 3));
            }
        }
        const bool live = j < N;
        const int jj = j & (kBC - 1);
        const bool narrow = NARROW && j / kBC == NTL - 1;  // the last tile, staged narrow
        int t = 0, m = jj;
        if (!narrow) m = key_slot(jj, t);
        TileLds<NT, 4>& s = lds[j / kBC];
        if (!narrow || jj < 16) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                uint32_t o[4];
                unpack_bits32_f4(live ? words[w] : 0u, o);
                *reinterpret_cast<uint4*>(&s.k[((t * W + w) * 16 + m) * 4]) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        s.mu[jj] = live ? acc / (float)d : 0.0f;
    }

    // the Q loads, issued once K has released its registers, arrive while V is processed
    h8 qx[kKeepTiles][4];
#pragma unroll
    for (int it = 0; it < kKeepTiles; ++it) {
        const int i = (qb_lo + it) * kBR + wave * 16 + n16;
#pragma unroll
        for (int c = 0; c < 4; ++c)  // chunks past d belong to the next query: masked where used
            if (it < nitems) qx[it][c] = load16(qr, min(i, N) * d * 2 + 64 * g + 16 * c);
    }

    // ---- V: channel absmax (input precision), scales, quantise, transpose, scatter
    h8 mv;
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = (_Float16)0;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) mv = __builtin_elementwise_max(mv, __builtin_elementwise_abs(vx[i]));
    if (grp < G) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sRed[grp * d + part * 8 + e] = (float)mv[e];
    }
    __syncthreads();
    const int K = 256 / d;  // threads per channel in the reductions
    if (tid < K * d) {
        const int c = tid % d;
        float av = 0.0f;
        for (int gi = tid / d; gi < G; gi += K) av = fmaxf(av, sRed[gi * d + c]);
        atomicMax(&sAmx[c], __float_as_uint(av));
    }
    __syncthreads();
    if (tid < 128) {
        const float av = __uint_as_float(sAmx[tid]);
        sScale[tid] = tid < d ? av / 127.0f : 0.0f;  // dequantisation scale, as fp32 a/127
        sInv[tid] = av > 0.0f ? 127.0f / av : 0.0f;
    }
    __syncthreads();
    // V^ = rint(v * fl32(127/a)), |v| <= a keeping it within +-127 (no clamp needed).  d <= 64:
    // through t + 1.5 * 2^23, which for |t| < 2^22 rounds t to the nearest integer (ties to even,
    // as rint) and holds it in the low mantissa bits, so its low byte is V^ as int8 and its bit
    // pattern minus that of 1.5 * 2^23 is V^ -- a channel's four token bytes go straight into one
    // dword (byte t = token t) with three v_perm.  Wider heads keep rint, v_cvt_pk_u8 and a 4x4
    // transpose, which hold fewer registers at once (the three-waves-per-SIMD budget).
    constexpr float kRound = 12582912.0f;
    uint32_t vsum[8];  // d <= 64: sum of those bit patterns per channel (wraps; minus cnt times kRound's)
    float vsumf[8];    // wider: sum of V^ per channel (exact integers)
#pragma unroll
    for (int e = 0; e < 8; ++e) vsum[e] = 0u, vsumf[e] = 0.0f;
    uint32_t cnt = 0;
    if (grp < G) {
        float inv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) inv[e] = sInv[part * 8 + e];
#pragma unroll
        for (int u = 0; u < MAXC / 4; ++u) {
            const int n0 = 4 * (grp + G * u);
            if (n0 < N) {
                cnt += 4;
                const int t = n0 >> 6, jj = n0 & (kBC - 1);
                const bool narrow = NARROW && t == NTL - 1;  // keys 4q..4q+3 -> first dword of lane q
                const int gg = narrow ? jj >> 2 : jj >> 4, ii = narrow ? 0 : jj & 15;
                char* vbase = reinterpret_cast<char*>(lds[t].v);
                if constexpr (NT <= 4) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {  // channel part * 8 + e of the four tokens
                        uint32_t ub[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
#pragma clang fp contract(off)
                            const float x = (float)vx[4 * u + r][e] * inv[e];  // product and sum round separately
                            ub[r] = __float_as_uint(x + kRound);
                            vsum[e] += ub[r];
                        }
                        const uint32_t lo = __builtin_amdgcn_perm(ub[1], ub[0], 0x0c0c0400u);  // t0 t1 0 0
                        const uint32_t hi = __builtin_amdgcn_perm(ub[3], ub[2], 0x0c0c0400u);  // t2 t3 0 0
                        int ct;
                        const int m = chan_slot<NT>(part * 8 + e, ct);
                        *reinterpret_cast<uint32_t*>(vbase + ((ct * kWave + m + 16 * gg) * 16 + ii)) =
                            __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    }
                } else {
                    uint32_t qb[4][2];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            uint32_t word = 0;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const float q = __builtin_rintf((float)vx[4 * u + r][4 * w + b] * inv[4 * w + b]);
                                vsumf[4 * w + b] += q;
                                word = __builtin_amdgcn_cvt_pk_u8_f32(q + 128.0f, b, word);  // exact: q is an integer
                            }
                            qb[r][w] = word ^ 0x80808080u;
                        }
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        const uint32_t in[4] = {qb[0][w], qb[1][w], qb[2][w], qb[3][w]};
                        uint32_t out[4];
                        transpose4x4(in, out);
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) {
                            int ct;
                            const int m = chan_slot<NT>(part * 8 + 4 * w + cc, ct);
                            *reinterpret_cast<uint32_t*>(vbase + ((ct * kWave + m + 16 * gg) * 16 + ii)) = out[cc];
                        }
                    }
                }
            }
        }
    }

    // column sums: partial sums through sRed (the absmax pass is done with it); integers, so the
    // order of the additions does not matter
    int* sRedI = reinterpret_cast<int*>(sRed);
    if (grp < G) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sRedI[grp * d + part * 8 + e] = NT <= 4 ? (int)(vsum[e] - cnt * __float_as_uint(kRound)) : (int)vsumf[e];
    }
    __syncthreads();
    if (tid < K * d) {
        const int c = tid % d;
        int cs = 0;
        for (int gi = tid / d; gi < G; gi += K) cs += sRedI[gi * d + c];
        atomicAdd(&sCol[c], 128 * cs);
    }

    // ---- Q of every query block of this workgroup: word g of the signs and mu_q per lane
#pragma unroll
    for (int it = 0; it < kKeepTiles; ++it) {
        if (it >= nitems) break;
        const int i = (qb_lo + it) * kBR + wave * 16 + n16;
        const bool live = i < N;
        uint32_t word = 0;
        float psum[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t byte;
            float sum;
            chunk_sign_abs(qx[it][c], byte, sum);
            psum[c] = sum;
            if (4 * g + c < cpt) word |= byte << (8 * c);
        }
        // mu = (sum over the query's chunks in channel order) / d: lanes g = 0, 1, .. add theirs in turn
        float acc = 0.0f;
#pragma unroll
        for (int gg = 0; gg < W; ++gg) {
            if (g == gg) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (4 * g + c < cpt) acc += psum[c];
            }
            acc = __shfl(acc, 16 * gg + n16);
        }
        sQw[(it * kWaves + wave) * kWave + lane] = (live && g < W) ? word : 0u;
        if (g == 0) sQmu[(it * kWaves + wave) * 16 + n16] = live ? acc / (float)d : 0.0f;
    }
}

// ---------------------------------------------------------------------------------------------
// Head-resident kernel: exact row max in two passes over register-resident scores.  A workgroup
// stages the K operand rows, mu_k, V^ and the V^ column sums of one (b, h) once and then loops
// over its segment [qb_lo, qb_hi) of that head's query blocks (segments per the KeepPlan).  The
// next block's query words, dense-bias rows and relative-position window are loaded while the
// current block is computed, into registers the current block no longer needs.  FUSED: the
// staging reads fp16 Q, K, V and packs / quantises them itself (fused_stage).
// TAIL: 0 when N is a multiple of the tile; 1 when the last tile masks the keys >= N; 2 when the
// last tile (tile NTL - 1) holds at most 16 keys and is computed as the narrow tile.
// NTL > kKeepTiles (long rows): NTL is the capacity and ceil(N / 64) <= NTL tiles are used; the
// dense bias is then fetched one tile ahead instead of a whole query block ahead.
template <int NT, int BIAS, int NTL, bool FUSED, int TAIL>
__global__ __launch_bounds__(256) void binattn_fwd_keep_kernel(FwdArgs a, KeepPlan plan) {
    constexpr int W = (NT + 1) / 2;
    constexpr bool DENSE = BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32;
    constexpr bool LONG = NTL > kKeepTiles;
    constexpr bool RAGGED = TAIL != 0, NARROW = TAIL == 2;
    static_assert(!(LONG && FUSED), "the whole-attention staging covers short rows only");
    typedef TileRegs<NT, 4> Regs;
    typedef TileLds<NT, 4> Lds;
    __shared__ Lds lds[NTL];
    __shared__ __attribute__((aligned(16))) float sWin[is_relpos(BIAS) ? kRelposWin : 4];
    // RELPOS_G: per key of the head, the byte offset of its part of the window index
    __shared__ __attribute__((aligned(16))) int sKk[BIAS == BK_RELPOS_G ? NTL * kBC : 4];
    __shared__ __attribute__((aligned(16))) float sScale[128];
    __shared__ __attribute__((aligned(16))) int sCol[128];  // 128 * sum_j V^_jc per channel slot
    // whole-attention path only: the prepared Q of every query block, and staging scratch
    __shared__ __attribute__((aligned(16))) uint32_t sQw[FUSED ? kKeepTiles * kWaves * kWave : 1];
    __shared__ __attribute__((aligned(16))) float sQmu[FUSED ? kKeepTiles * kWaves * 16 : 1];
    __shared__ __attribute__((aligned(16))) float sRed[FUSED ? 2048 : 1];
    __shared__ __attribute__((aligned(16))) float sInv[FUSED ? 128 : 1];
    __shared__ __attribute__((aligned(16))) uint32_t sAmx[FUSED ? 128 : 1];

    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int nt = LONG ? (N + kBC - 1) / kBC : NTL;  // tiles in use
    // This workgroup's segment of the query blocks of one head.  Workgroup b runs on XCD b % 8;
    // each XCD owns a contiguous range of heads and lays its workgroups out by the plan (first
    // the `a` segments of f blocks of each head, then the `b` segments of r blocks).
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int64_t nheads = (int64_t)a.B * a.H;
    const int hx0 = (int)(nheads * xcd / 8), hx = (int)(nheads * (xcd + 1) / 8) - hx0;
    int bh, qb_lo, qb_len;
    if (slot < hx * plan.a) {
        bh = hx0 + slot / plan.a;
        qb_lo = (slot % plan.a) * plan.f;
        qb_len = plan.f;
    } else {
        const int s2 = slot - hx * plan.a;
        if (s2 >= hx * plan.b) return;  // this XCD has fewer heads than the grid allows for
        bh = hx0 + s2 / plan.b;
        qb_lo = plan.a * plan.f + (s2 % plan.b) * plan.r;
        qb_len = plan.r;
    }
    const int qb_hi = min(nqb, qb_lo + qb_len);
    if (qb_lo >= qb_hi) return;
    if (DENSE) {  // heads in (h, b) order: the batch items of one head share its bias rows in the XCD's L2
        const int hh = bh / a.B, bb = bh - hh * a.B;
        bh = bb * a.H + hh;
    }
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keeps row pointers scalar
    const int h = bh % a.H;

    HeadPtrs hp;
    hp.kb = a.kbits + (int64_t)bh * N * W;
    hp.kmu = a.kmu + (int64_t)bh * N;
    hp.vq = a.vq + (int64_t)bh * d * a.ldv;
    hp.table = nullptr;
    if (is_relpos(BIAS)) {
        const int64_t tsz = (int64_t)(2 * a.gh - 1) * (2 * a.gw - 1);
        hp.table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz)
                              : (const void*)((const _Float16*)a.bias + h * tsz);
    }
    const int esz = BIAS == BK_DENSE_F32 ? 4 : 2;
    const int bvoff = (n16 * (int)a.bias_ld + 16 * g) * esz;

    // Per-block inputs of this lane: word g of its query's signs (0 past d or N) and mu_q.
    auto load_query = [&](int qb, uint32_t& qword, float& qmu) {
        if constexpr (FUSED) {
            const int it = qb - qb_lo;
            qword = sQw[(it * kWaves + wave) * kWave + lane];
            qmu = sQmu[(it * kWaves + wave) * 16 + n16];
        } else {
            const int i = qb * kBR + wave * 16 + n16;
            const bool live = i < N;
            qword = (live && g < W) ? a.qbits[((int64_t)bh * N + i) * W + g] : 0u;
            qmu = live ? a.qmu[(int64_t)bh * N + i] : 0.0f;
        }
    };
    // Dense bias rows of this wave's 16 queries of block qb, key tile t (rows >= N read 0); the
    // narrow last tile reads its lane's four keys.
    auto load_bias_tile = [&](int qb, int t, BiasRegs<BIAS>& bias_t) {
        const int r0 = min(qb * kBR + wave * 16, N);
        const char* brow = (const char*)a.bias + ((int64_t)h * N + r0) * a.bias_ld * esz;
        const int brow_bytes = min(N - r0, 16) * (int)a.bias_ld * esz;  // at most 16 rows: far below 2^31
        const int j0 = t * kBC;
        const int voff = NARROW && t == NTL - 1 ? (n16 * (int)a.bias_ld + 4 * g) * esz : bvoff;
        load_bias<BIAS>(bias_t, buffer_rsrc(brow + j0 * esz, brow_bytes - j0 * esz), voff);
    };
    // First table row of the relative-position window of block qb (every key touched).
    auto window_lo = [&](int qb) { return relpos_window(qb * kBR, 0, N, N, a.gh, a.gw).dr_lo; };

    // ---- stage the head once (all loads in flight together), then the first block's inputs
    if constexpr (FUSED) {
        fused_stage<NT, NTL, NARROW>(a, bh, qb_lo, qb_hi - qb_lo, lds, sScale, sQw, sQmu, sRed, sInv, sAmx, sCol);
        __syncthreads();  // the prepared query words are read by load_query below
    } else {
        Regs regs[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t)
            if (!LONG || t < nt) load_tile<NT, 4>(regs[t], a, hp, t * kBC, 0);
        stage_common(a, bh, sScale);
        int cs[Regs::VCH];
#pragma unroll
        for (int i = 0; i < Regs::VCH; ++i) cs[i] = 0;
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            if (!LONG || t < nt) {
                if (NARROW && t == NTL - 1)
                    store_tile<NT, 4, true>(regs[t], lds[t], d);
                else
                    store_tile<NT, 4>(regs[t], lds[t], d);
                colsum_add(regs[t], cs);
            }
        }
        colsum_store<NT>(cs, sCol);
    }
    // window slot tid + 256 i holds table row r, column c of the window (row stride a.wrs; the
    // slots past a row's 2 gw - 1 entries are padding, loaded but never read)
    float wv[kRelposWin / 256];
    int weo[kRelposWin / 256];
    if (BIAS == BK_RELPOS_G) {  // key j at grid (rj, cj): (gh - 1 - rj) row stride + gw - 1 - cj, in bytes
        for (int j = tid; j < NTL * kBC; j += 256) {
            const int jj = min(j, N - 1);  // keys past N are masked: any in-window offset will do
            const int rj = jj / a.gw, cj = jj - rj * a.gw;
            sKk[j] = 4 * ((a.gh - 1 - rj) * a.wrs + a.gw - 1 - cj);
        }
    }
    if (is_relpos(BIAS)) {
#pragma unroll
        for (int i = 0; i < kRelposWin / 256; ++i) {
            const int slot = tid + 256 * i, r = slot / a.wrs;
            weo[i] = r * (2 * a.gw - 1) + (slot - r * a.wrs);
        }
        load_window_at<kRelposWin / 256>(wv, a, hp.table, window_lo(qb_lo) * (2 * a.gw - 1), weo);
#pragma unroll
        for (int i = 0; i < kRelposWin / 256; ++i) sWin[tid + 256 * i] = wv[i];
    }
    uint32_t qword;
    float qmu;
    load_query(qb_lo, qword, qmu);
    // short rows: every tile's bias rows of the block, fetched a block ahead; long rows: two
    // tile buffers, each tile fetched while the one before it is computed
    BiasRegs<BIAS> bias[LONG ? 2 : NTL];
    if (DENSE) {
#pragma unroll
        for (int t = 0; t < (LONG ? 1 : NTL); ++t) load_bias_tile(qb_lo, t, bias[t]);
    }
    __syncthreads();

    // relative position: the key part of each tile's window offset for this lane's key run
    // (keys 64 t + 16 g ..), so a block adds only its query's part
    int krel[BIAS == BK_RELPOS ? NTL : 1];
    if (BIAS == BK_RELPOS) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int jg = t * kBC + 16 * g, rj = jg / a.gw, cj = jg % a.gw;
            krel[t] = (a.gh - 1 - rj) * a.wrs + (a.gw - 1 - cj);
        }
    }

    for (int qb = qb_lo; qb < qb_hi; ++qb) {
        // The staged tiles do not change across query blocks; reading them through an offset the
        // compiler cannot see is zero keeps it from hoisting every tile's operands out of this
        // loop (which would hold them all in registers and halve the occupancy).
        Lds* const L = lds + opaque_zero();
        const int q0 = qb * kBR, qw0 = q0 + wave * 16;
        const bool live = qw0 < N;  // some query of this wave is < N (wave-uniform)
        const bool more = qb + 1 < qb_hi;
        if (is_relpos(BIAS) && more)
            load_window_at<kRelposWin / 256>(wv, a, hp.table, window_lo(qb + 1) * (2 * a.gw - 1), weo);

        // the lane's query: Q operand (fp4 2*sign of channels 32g..32g+31, 0 past d) and seed
        LaneQ lq;
        {
            const int i = qw0 + n16;
            lq.live = i < N;
            lq.qi = lq.live ? i : N - 1;
            lq.qop = q_operand(qword, lq.live && g < W, d, g);
            const float pos = rows4_sum((float)__builtin_popcount(qword));  // sign bits set over the query
            const float seed = lq.live ? (float)d - 2.0f * pos : 0.0f;
            lq.dseed = v4f{seed, seed, seed, seed};
            lq.cq = qmu * a.qk_scale;
        }
        int qrel = 0;  // relative position: the query's part of the window offsets
        if (is_relpos(BIAS)) {
            const int ri = lq.qi / a.gw, ci = lq.qi % a.gw;
            qrel = (ri - window_lo(qb)) * a.wrs + ci;
        }

        // ---- pass 1: scores and row max
        float S[NTL][16];
        float S4[4];  // the narrow last tile
        float mloc = -INFINITY;
        if (live) {
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                if (!LONG || t < nt) {  // (a uniform skip, not a break: the loop must unroll to keep S in registers)
                    if (LONG && DENSE && t + 1 < nt) load_bias_tile(qb, t + 1, bias[(t + 1) & 1]);
                    const bool nar = NARROW && t == NTL - 1;
                    const int run = nar ? 4 : 16;  // keys per lane
                    const int jg = t * kBC + run * g;
                    int idx0 = run - 1;
                    if (BIAS == BK_RELPOS)  // (a run wholly past N is masked; its reads stay in the window)
                        idx0 = jg >= N ? run - 1 : qrel + krel[t];
                    if (BIAS == BK_RELPOS_G) idx0 = qrel + 15;  // window base of the query; keys via sKk
                    if (nar)
                        tile_scores4<NT, BIAS>(L[t].k, L[t].mu, lq, bias[LONG ? (t & 1) : t], sWin + idx0 - 3, N - jg,
                                               S4, mloc);
                    else
                        tile_scores<NT, BIAS>(L[t].k, L[t].mu, lq, bias[LONG ? (t & 1) : t], sWin + idx0 - 15,
                                              TAIL == 1 && t == nt - 1, N - jg, S[t], mloc, sKk + jg);
                }
                __builtin_amdgcn_sched_barrier(0);  // one tile's operands live at a time
            }
        }
        // the next block's query words and bias rows, into registers pass 1 has released
        if (more) {
            load_query(qb + 1, qword, qmu);
            if (DENSE) {
#pragma unroll
                for (int t = 0; t < (LONG ? 1 : NTL); ++t) load_bias_tile(qb + 1, t, bias[t]);
            }
        }
        if (is_relpos(BIAS)) {
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
            v4i acc[NT];  // starts at the column-sum term of the lane's channels
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acc[ct] = *reinterpret_cast<const v4i*>(&sCol[4 * NT * g + 4 * ct]);
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                if (!LONG || t < nt) {
                    const v4i pw = NARROW && t == NTL - 1 ? tile_probs4(S4, negm, lsum) : tile_probs(S[t], negm, lsum);
#pragma unroll
                    for (int ct = 0; ct < NT; ++ct) {
                        const v4i vop = *reinterpret_cast<const v4i*>(&L[t].v[(ct * kWave + lane) * 4]);
                        acc[ct] = mfma_i8(vop, pw, acc[ct]);
                    }
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
        if (is_relpos(BIAS)) __syncthreads();  // the next block's window is in place
    }
}

// LDS row stride (fp32 entries) of the relative-position window the head-resident kernel stages
// for a whole short row (the queries of one block, every key), or 0 when it does not fit (the
// launch then goes to the streaming kernel).  A wave's 16 queries share a grid row, and so do the
// 16 keys of lane group g (the grid width is a multiple of 16), so group g reads 16 consecutive
// window entries from an offset that moves by -(rj stride + cj) with its first key (rj, cj).  The
// smallest stride >= the table row 2 gw - 1 that puts the four groups' runs on disjoint banks
// (their starts 16 apart modulo 32 within each half-wave and at least 16 apart modulo 64 across
// the wave) makes every window read free of bank conflicts; 2 gw - 1 itself when none fits.
inline int keep_window_stride(const FwdArgs& a) {
    const int N = a.N, gw = a.gw, gh = a.gh, row = 2 * gw - 1;
    int rows = 0;  // table rows of the largest window
    for (int q0 = 0; q0 < N; q0 += kBR) {
        const int ri_min = q0 / gw, ri_max = (min(q0 + kBR, N) - 1) / gw;
        rows = max(rows, ri_max - ri_min + gh);
    }
    if (gw % 16 != 0) return rows * row <= kRelposWin ? row : 0;  // gathered per key: no run layout to place
    auto conflict_free = [&](int rs) {
        for (int j0 = 0; j0 < N; j0 += kBC) {
            int st[4];
            for (int g = 0; g < 4; ++g) {
                const int j = j0 + 16 * g;
                st[g] = (((-(j / gw) * rs - j % gw) % 64) + 64) % 64;
            }
            for (int g = 0; g < 4; ++g)
                for (int h = g + 1; h < 4 && j0 + 16 * h < N; ++h) {  // groups past N are masked
                    const int dist = (st[h] - st[g] + 64) % 64;
                    if (dist < 16 || dist > 48) return false;
                    if (h == g + 1 && (g & 1) == 0 && dist % 32 != 16) return false;
                }
        }
        return true;
    };
    for (int rs = row; rs < row + 64; ++rs)
        if (rows * rs <= kRelposWin && conflict_free(rs)) return rs;
    return rows * row <= kRelposWin ? row : 0;
}
inline bool keep_window_fits(const FwdArgs& a) { return keep_window_stride(a) > 0; }

// Compute units of the current device (cached per device; 256 on MI355X).
inline int device_cus() {
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

// Resident 256-thread workgroups of `kernel` per compute unit (registers and LDS permitting).
template <typename K>
inline int resident_per_cu(K kernel) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 256, 0) != hipSuccess || nb < 1) nb = 1;
    return nb;
}

// Makespan, in units of one query block's work, of one XCD's workgroups under `plan`, dispatched
// in order onto `slots` resident slots as they free up (each workgroup also stages its head,
// `stage` units).
inline double keep_plan_makespan(int heads, int nqb, int slots, double stage, KeepPlan p) {
    std::vector<double> free_at((size_t)std::max(slots, 1), 0.0);
    std::make_heap(free_at.begin(), free_at.end(), std::greater<double>());
    double end = 0.0;
    auto run = [&](int len) {
        std::pop_heap(free_at.begin(), free_at.end(), std::greater<double>());
        const double t = free_at.back() + stage + len;
        free_at.back() = t;
        std::push_heap(free_at.begin(), free_at.end(), std::greater<double>());
        end = std::max(end, t);
    };
    for (int h = 0; h < heads; ++h)
        for (int k = 0; k < p.a; ++k) run(std::max(0, std::min(p.f, nqb - k * p.f)));
    for (int h = 0; h < heads; ++h)
        for (int k = 0; k < p.b; ++k) run(std::max(0, std::min(p.r, nqb - p.a * p.f - k * p.r)));
    return end;
}

// The plan with the shortest modelled makespan for B*H heads of nqb query blocks on a device
// with `slots` resident workgroups (all XCDs); remembered per shape.
inline KeepPlan keep_plan(int64_t nheads, int nqb, int slots, double stage) {
    struct Entry {
        int64_t nheads;
        int nqb, slots, stage_milli;
        KeepPlan plan;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    const int stage_milli = (int)(stage * 1000.0);
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry& e : cache)
            if (e.nheads == nheads && e.nqb == nqb && e.slots == slots && e.stage_milli == stage_milli) return e.plan;
    }
    const int heads = (int)((nheads + 7) / 8), xslots = std::max(1, slots / 8);  // the busiest XCD
    KeepPlan best{1, nqb, 0, 1};
    double best_t = keep_plan_makespan(heads, nqb, xslots, stage, best);
    for (int f = 1; f <= nqb; ++f)
        for (int na = 1; na * f <= nqb + f - 1; ++na) {
            const int rest = nqb - na * f;
            for (int r = 1; r <= (rest > 0 ? f : 1); ++r) {
                const KeepPlan p{na, f, rest > 0 ? (rest + r - 1) / r : 0, r};
                const double t = keep_plan_makespan(heads, nqb, xslots, stage, p);
                if (t < best_t - 1e-9) best_t = t, best = p;
            }
        }
    // equal segments all go first: the workgroups of one head are then launched next to each
    // other (same XCD, consecutive slots) and the later ones find its inputs in L2
    if (best.b > 0 && best.r == best.f) best.a += best.b, best.b = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() > 64) cache.clear();
    cache.push_back(Entry{nheads, nqb, slots, stage_milli, best});
    return best;
}

// Staging a head costs about half a query block's work (plain), three (whole attention).
template <int NT, int BK, int NTL, bool FUSED, int TAIL>
inline void launch_keep_inst(const FwdArgs& a, hipStream_t s) {
    static const int per_cu = resident_per_cu(binattn_fwd_keep_kernel<NT, BK, NTL, FUSED, TAIL>);
    const int64_t nheads = (int64_t)a.B * a.H;
    const int nqb = (a.N + kBR - 1) / kBR;
    const KeepPlan p = keep_plan(nheads, nqb, per_cu * device_cus(), FUSED ? 3.0 : 0.5);
    const int64_t grid = 8 * ((nheads + 7) / 8) * (p.a + p.b);
    FwdArgs ka = a;
    if (is_relpos(BK)) ka.wrs = keep_window_stride(a);
    hipLaunchKernelGGL((binattn_fwd_keep_kernel<NT, BK, NTL, FUSED, TAIL>), dim3((unsigned)grid), dim3(256), 0, s,
                       ka, p);
}

// Kind of the last tile: 0 whole, 2 at most 16 keys (narrow), 1 otherwise.
inline int keep_tail(int N) {
    const int r = N % kBC;
    return r == 0 ? 0 : (r <= 16 ? 2 : 1);
}

// The head-resident kernel for rows of kKeepTiles < ceil(N / 64) <= kLongTiles tiles (d <= 64);
// the narrow last tile only where it is tile kLongTiles - 1.
template <int NT, int BK>
inline void launch_keep_long(const FwdArgs& a, hipStream_t s) {
    static_assert(NT <= 4, "long rows are staged whole for d <= 64 only");
    const int ntiles = (a.N + kBC - 1) / kBC, tail = keep_tail(a.N);
    if (tail == 0)
        launch_keep_inst<NT, BK, kLongTiles, false, 0>(a, s);
    else if (tail == 2 && ntiles == kLongTiles)
        launch_keep_inst<NT, BK, kLongTiles, false, 2>(a, s);
    else
        launch_keep_inst<NT, BK, kLongTiles, false, 1>(a, s);
}

template <int NT, int BK, bool FUSED, int TAIL>
inline void launch_keep_tail(const FwdArgs& a, int ntiles, hipStream_t s) {
    switch (ntiles) {
        case 1: launch_keep_inst<NT, BK, 1, FUSED, TAIL>(a, s); break;
        case 2: launch_keep_inst<NT, BK, 2, FUSED, TAIL>(a, s); break;
        case 3: launch_keep_inst<NT, BK, 3, FUSED, TAIL>(a, s); break;
        default: launch_keep_inst<NT, BK, 4, FUSED, TAIL>(a, s); break;
    }
}

// The short-row kernel for rows of ceil(N / 64) <= kKeepTiles tiles.
template <int NT, int BK, bool FUSED>
inline void launch_keep(const FwdArgs& a, hipStream_t s) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    const int tail = keep_tail(a.N);
    if (tail == 0) {
        launch_keep_tail<NT, BK, FUSED, 0>(a, ntiles, s);
        return;
    }
    if constexpr (!is_relpos(BK)) {  // relative position: the last tile is masked, never narrow
        if (tail == 2) {
            launch_keep_tail<NT, BK, FUSED, 2>(a, ntiles, s);
            return;
        }
    }
    launch_keep_tail<NT, BK, FUSED, 1>(a, ntiles, s);
}

}  // namespace binattn
