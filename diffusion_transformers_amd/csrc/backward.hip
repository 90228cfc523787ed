// backward.hip -- gradients of the quantisation-aware BinaryAttention forward.
//
// "BinaryAttention" paper notes (CVPR 2026), Method details, key design 4 and the section on the
// loss and training strategy: the model is fine-tuned with quantisation-aware training, the
// forward keeps sign(Q), sign(K) and the backward passes the gradient through sign with a
// straight-through estimator.  Readings where the pages are silent (the same as the CPU oracle):
//   - sign: d sign(x)/dx := 1, or 1{|x| <= clip} when a clip > 0 is given;
//   - mu = mean|x| is differentiated exactly (d mu/dx_c = sgn(x_c)/d, sgn(0) = 0);
//   - the P (u8, 1/255) and V (int8, per channel) quantisers are straight-through: their forward
//     values are the quantised ones, their gradients those of the identity;
//   - the row max is a constant; the row sum l = sum exp(S - m) is differentiated.
// With P = exp(S - m) / l, A = P^/255 / l (the weights the forward applies), Vt = s V^:
//   dV_j = sum_i A_ij dO_i,   Delta_i = dO_i . O_i,   dP_ij = dO_i . Vt_j,
//   dS_ij = P_ij (dP_ij - Delta_i) = db_ij (summed over the batch, or into the table entry (i, j)
//   indexes),   ds_i = sum_j dS_ij t_j / sqrt(d),   dt_j = sum_i dS_ij s_i / sqrt(d)
//   (s = mu_q sign(q), t = mu_k sign(k)),   dq_ic = mu_q ds_ic ste(q_ic) + sgn(q_ic)/d sum_e ds_ie
//   sign(q_ie) (likewise dk), dv = dV.
//
// gfx950 design (one workgroup = 4 waves x 16 rows; tiles of 64 keys or queries).  The four
// dense products run on the bf16 MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  bf16
// keeps fp32's exponent range, so gradients of any scale enter without overflow or underflow;
// every operand that is not exact in bf16 (V^ and P^ are integers below 256, the signs are +-1)
// is split into two bf16 terms x = hi + lo (hi = bf16(x), lo = bf16(x - hi), about 16
// significant bits) and multiplied as two MFMAs, so that the products keep near-fp32 accuracy:
//   dP_ij = sum_c (dO_ic s_c) V^_jc                      (dO s split, V^ exact)
//   dV_j  = sum_i (dO_i / (255 l_i)) P^_ij               (dO / (255 l) split, P^ exact)
//   dQ_i  = sum_j (dS_ij mu_kj / sqrt(d)) sign(k_j)      (dS mu split, sign exact)
//   dK_j  = sum_i (dS_ij mu_qi / sqrt(d)) sign(q_i)
// (rows of dS sum to about zero, so rounding dS and mu k separately to 8 bits would cancel badly
// for short rows; the split keeps that cancellation exact to ~2^-16).
//  * bw_rows_kernel<STATS = true> (a workgroup per 64 queries): the exact row max and row sum
//    over all key tiles (scores by the forward's fp4 QK tile) and Delta = dO . O.
//  * bw_prep_kernel writes, from the packed Q/K and int8 V of the forward's preparation and the
//    row sums, the bf16 operand arrays in the layouts the lanes read (rows of channels, or
//    channels by 64-row tile), so that tiles are staged in LDS by 16-byte copies and every
//    operand read is one ds_read_b128.
//  * Every staging step issues all of a tile's global loads before its first LDS store (a loop of
//    load, wait, store pays one memory latency per iteration, and the kernels are bound by them).
//  * bw_rows_kernel<STATS = false> (a workgroup per 64 queries): per key tile the scores, P, dP,
//    dS, dQ and the bias gradient (dense: each batch item's dS stored in bf16 and summed over the
//    batch in fp32 afterwards -- a sum of independent terms, so the rounding (relative 2^-9 per
//    term) does not cancel into the result the way it would inside dQ's row sums; relative
//    position: the table's entries accumulated in LDS).
//  * bw_k_kernel (a workgroup per 64 keys): per query tile the transposed score tile (queries as
//    MFMA rows, the lane's key as the column), P and P^, dP, dS, then dV and dK.
#include <utility>

#include "tile.h"

namespace binattn {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

struct BwArgs {
    const void* q;        // [B,H,N,d] input dtype
    const void* k;
    const void* o;        // forward output, grad dtype
    const void* dout;     // grad dtype
    int in_f32, g_f32;
    const uint32_t* qbits;
    const float* qmu;
    const uint32_t* kbits;
    const float* kmu;
    const int8_t* vq;
    const float* vamax;
    int64_t ldv;
    const void* bias;
    int64_t bias_ld;
    int bias_f32;
    int gh, gw;
    int B, H, N, d, W, Np;  // Np: N rounded up to a multiple of 64; channels padded to CP = 32 W
    float qk_scale;
    float clip;
    // bf16 operand arrays; "row" arrays are [BH][Np][CP], "tile" arrays [BH][Np/64][CP][64]
    __bf16* vh;      // row: V^ (exact)
    __bf16* dos_hi;  // row: dO_ic s_c, two terms
    __bf16* dos_lo;
    __bf16* sk;      // tile: sign(k_c) (+-1; 0 past N and d)
    __bf16* sq;      // tile: sign(q_c)
    __bf16* dot_hi;  // tile: dO_ic / (255 l_i), two terms
    __bf16* dot_lo;
    float* m;        // [BH][N] row max, row sum, Delta
    float* l;
    float* delta;
    float* dq;       // [B,H,N,d] fp32
    float* dk;
    float* dv;
    float* db;       // dense [H,N,N] or table [H,(2gh-1)(2gw-1)], fp32; may be null
    __bf16* dsb;     // dense bias gradient: dS of every batch item [B][H][N][Np] in bf16, summed over B afterwards
    float* dtp;      // table gradient of each query-block workgroup [B H nqb][kTabMax] when the table has
                     // at most kTabMax entries (else null: the entries go to db by atomics per key tile)
};

constexpr int kTabMax = 4096;  // table entries a workgroup accumulates whole in LDS

__device__ __forceinline__ v4f mfma_b(bf8 a, bf8 b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

__device__ __forceinline__ float ld_any(const void* p, int64_t i, int f32) {
    return f32 ? static_cast<const float*>(p)[i] : (float)static_cast<const _Float16*>(p)[i];
}

__device__ __forceinline__ float ste_grad(float x, float clip) { return (clip > 0.0f && fabsf(x) > clip) ? 0.0f : 1.0f; }

__device__ __forceinline__ float sgn0(float x) { return x > 0.0f ? 1.0f : (x < 0.0f ? -1.0f : 0.0f); }

__device__ __forceinline__ bool sign_bit(const uint32_t* bits, int64_t tok, int W, int c) {
    return (bits[tok * W + (c >> 5)] >> (c & 31)) & 1u;
}

// Row (query or key) slot of MFMA t's A operand row m: after the MFMA, lane (n, g) register r of
// tile t holds row 16 g + 4 t + r (the forward's key_slot order).
__device__ __forceinline__ int slot_row(int t, int m) { return 16 * (m >> 2) + 4 * t + (m & 3); }

// x = hi + lo in bf16 (hi rounded to nearest, lo the rounded remainder).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// The 8 values x[8 s2 .. 8 s2 + 7] as bf16 MFMA operands (step s2 covers rows 16 g + 8 s2 + i).
__device__ __forceinline__ bf8 pack_exact(const float (&x)[16], int s2) {
    bf8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[8 * s2 + i];
    return r;
}

__device__ __forceinline__ void pack_split(const float (&x)[16], int s2, bf8& hi, bf8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __bf16 h, l;
        split_bf16(x[8 * s2 + i], h, l);
        hi[i] = h;
        lo[i] = l;
    }
}

// db[h][i][j] = sum over b of dS[b][h][i][j] (stored in bf16), in fp32 and batch order
// (deterministic).  A thread takes four consecutive keys (one 8-byte load per batch item; the
// stored rows are padded to Np keys with zeros).
__global__ __launch_bounds__(256) void bw_dbias_kernel(const __bf16* __restrict__ dsb, float* __restrict__ db, int B,
                                                       int H, int N, int Np) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nq = Np / 4;
    const int64_t hn = (int64_t)H * N;
    if (e >= hn * nq) return;
    const int64_t r = e / nq;  // r = h N + i
    const int j = 4 * (int)(e - r * nq);
    const int64_t stride = hn * Np;
    const __bf16* p = dsb + r * Np + j;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = 0; b < B; ++b) {
        typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
        const bf4 x = *reinterpret_cast<const bf4*>(p + b * stride);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] += (float)x[t];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (j + t < N) db[r * N + j + t] = acc[t];
}

// Table gradient: db[h][e] = sum of the partial tables of the query-block workgroups of head h
// (stored at logical block (b H + h) nqb + query block), in a fixed order (deterministic): a
// workgroup takes 64 entries, its 4 waves sum every 4th partial (8 running sums each), and the
// 4 wave sums are added in wave order.
__global__ __launch_bounds__(256) void bw_dtable_kernel(const float* __restrict__ dtp, float* __restrict__ db, int B,
                                                        int H, int nqb, int tsz) {
    __shared__ float part[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 64 + lane;
    const bool ok = e < (int64_t)H * tsz;
    const int h = ok ? (int)(e / tsz) : 0, t = ok ? (int)(e - (int64_t)h * tsz) : 0;
    const int np = B * nqb;  // partials of head h: (b H + h) nqb + qb for b < B, qb < nqb
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
        int n = wv, u = 0;
        for (; n < np; n += 4, u = (u + 1) & 7) {
            const int b = n / nqb, qb = n - b * nqb;
            acc[u] += dtp[((int64_t)(b * H + h) * nqb + qb) * kTabMax + t];
        }
    }
    part[wv][lane] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    if (wv == 0 && ok) db[e] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

__global__ __launch_bounds__(256) void bw_zero_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Calls f(std::integral_constant<int, K>) for K = 0 .. N-1, so that register arrays are indexed
// by constants from the start (an array indexed in a loop can be left in scratch memory).
template <typename F, int... K>
__device__ __forceinline__ void for_each_k(F&& f, std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    for_each_k(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------------------------
// bf16 operand arrays, 64 rows of one head per workgroup; rows >= N and channels >= d are zero
// (needs the row sums).  Every load of the tile (dO rows, V^ channel rows, sign words) is issued
// before the first LDS store; the tile is gathered into LDS along each source's layout, then
// written out in 16-byte stores in each destination layout.
template <int CP, bool G32>
__global__ __launch_bounds__(256) void bw_prep_kernel(BwArgs a) {
    constexpr int TP = CP + 1;  // odd LDS row pitch: column walks are conflict-free
    constexpr int W = CP / 32, DIT = 8 * CP / 256, VIT = (4 * CP + 255) / 256;
    __shared__ float sv[kBC * TP], sd[kBC * TP];
    __shared__ float ssc[CP], sil[kBC];
    __shared__ uint32_t skb[kBC * 4], sqb[kBC * 4];
    const int nb = a.Np / kBC;
    const int64_t bh = blockIdx.x / nb;
    const int j0 = (blockIdx.x % nb) * kBC;
    const int N = a.N, d = a.d, tid = threadIdx.x;
    // ---- loads: dO chunks (row tid % 64, channels 8 (i / 64) ..+7), V^ chunks (channel t % CP,
    // tokens 16 (t / CP) ..+15), sign words, scales, row sums
    uint4 dv[DIT], dv2[G32 ? DIT : 1], vv[VIT];
    static_for<DIT>([&](auto k) {
        const int i = tid + 256 * k, r = i & 63, c0 = 8 * (i >> 6), j = j0 + r;
        dv[k] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (G32) dv2[k] = make_uint4(0u, 0u, 0u, 0u);
        if (j < N && c0 < d) {
            const int64_t e = (bh * N + j) * d + c0;
            if constexpr (G32) {
                dv[k] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.dout) + e);
                dv2[k] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.dout) + e + 4);
            } else {
                dv[k] = *reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.dout) + e);
            }
        }
    });
    static_for<VIT>([&](auto k) {
        const int t = tid + 256 * k, c = t % CP, q = t / CP;
        vv[k] = make_uint4(0u, 0u, 0u, 0u);  // (V^ past N is zero in its padded rows)
        if (t < 4 * CP && c < d) vv[k] = *reinterpret_cast<const uint4*>(a.vq + (bh * d + c) * a.ldv + j0 + 16 * q);
    });
    const int bw = tid >> 6, br = tid & 63;
    const bool bok = tid < kBC * W && j0 + br < N;
    const uint32_t kword = bok ? a.kbits[(bh * N + j0 + br) * W + bw] : 0u;
    const uint32_t qword = bok ? a.qbits[(bh * N + j0 + br) * W + bw] : 0u;
    const float sc = tid < CP && tid < d ? a.vamax[bh * d + tid] / 127.0f : 0.0f;
    const float lrow = tid < kBC && j0 + tid < N ? a.l[bh * N + j0 + tid] : 0.0f;
    // ---- LDS
    if (tid < CP) ssc[tid] = sc;
    if (tid < kBC) sil[tid] = j0 + tid < N ? 1.0f / (255.0f * lrow) : 0.0f;
    if (tid < kBC * W) {
        skb[br * 4 + bw] = kword;
        sqb[br * 4 + bw] = qword;
    }
    static_for<DIT>([&](auto k) {
        const int i = tid + 256 * k, r = i & 63, c0 = 8 * (i >> 6);
        if constexpr (G32) {
            const uint32_t w8[8] = {dv[k].x, dv[k].y, dv[k].z, dv[k].w, dv2[k].x, dv2[k].y, dv2[k].z, dv2[k].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sd[r * TP + c0 + e] = __uint_as_float(w8[e]);
        } else {
            const h8 hv = __builtin_bit_cast(h8, dv[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) sd[r * TP + c0 + e] = (float)hv[e];
        }
    });
    static_for<VIT>([&](auto k) {
        const int t = tid + 256 * k, c = t % CP, q = t / CP;
        if (t < 4 * CP) {
            const uint32_t w4[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
#pragma unroll
            for (int e = 0; e < 16; ++e) sv[(16 * q + e) * TP + c] = (float)(int)(int8_t)(w4[e >> 2] >> (8 * (e & 3)));
        }
    });
    __syncthreads();
    const int64_t t0 = (bh * a.Np + j0) * CP;  // the tile's 64 CP values in either layout
    auto put = [](__bf16* dst, const __bf16 (&x)[8]) { *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(x); };
    for (int o8 = tid; o8 < kBC * CP / 8; o8 += 256) {  // [row][c], 8 channels per thread
        const int jl = o8 / (CP / 8), c0 = 8 * (o8 - jl * (CP / 8));
        alignas(16) __bf16 v[8], hi[8], lo[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            v[u] = (__bf16)sv[jl * TP + c0 + u];
            split_bf16(sd[jl * TP + c0 + u] * ssc[c0 + u], hi[u], lo[u]);
        }
        const int64_t o = t0 + jl * CP + c0;
        put(a.vh + o, v);
        put(a.dos_hi + o, hi);
        put(a.dos_lo + o, lo);
    }
    for (int o8 = tid; o8 < kBC * CP / 8; o8 += 256) {  // [c][row], 8 rows per thread
        const int c = o8 / (kBC / 8), r0 = 8 * (o8 - c * (kBC / 8));
        alignas(16) __bf16 xk[8], xq[8], hi[8], lo[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int jl = r0 + u;
            const bool ok = c < d && j0 + jl < N;
            const bool bk = (skb[jl * 4 + (c >> 5)] >> (c & 31)) & 1u, bq = (sqb[jl * 4 + (c >> 5)] >> (c & 31)) & 1u;
            xk[u] = (__bf16)(ok ? (bk ? 1.0f : -1.0f) : 0.0f);
            xq[u] = (__bf16)(ok ? (bq ? 1.0f : -1.0f) : 0.0f);
            split_bf16(sd[jl * TP + c] * sil[jl], hi[u], lo[u]);
        }
        const int64_t o = t0 + c * kBC + r0;
        put(a.sk + o, xk);
        put(a.sq + o, xq);
        put(a.dot_hi + o, hi);
        put(a.dot_lo + o, lo);
    }
}

// Staging in two phases, every global load of a tile issued before the first LDS store (a loop
// of load, wait, store would pay one memory latency per iteration): load() into registers,
// store() into LDS.

// ROWS rows of RL bf16 values (8 ROWS RL / 8 is a multiple of 256): thread tid holds the 16-byte
// chunks tid + 256 k of the row-major tile.
template <int ROWS, int RL>
struct BfTile {
    static constexpr int PER = RL / 8, TOT = ROWS * PER, IT = TOT / 256;
    static_assert(TOT % 256 == 0, "whole chunks per thread");
    uint4 v[IT];
    __device__ __forceinline__ void load(const __bf16* src) {
        static_for<IT>([&](auto k) {
            v[k] = *reinterpret_cast<const uint4*>(src + 8 * (threadIdx.x + 256 * k));
        });
    }
    template <int PITCH>
    __device__ __forceinline__ void store(__bf16* dst) const {
        static_for<IT>([&](auto k) {
            const int i = threadIdx.x + 256 * k, r = i / PER, c = i - r * PER;
            *reinterpret_cast<uint4*>(dst + r * PITCH + 8 * c) = v[k];
        });
    }
};

// Sign words of 64 rows starting at row r0 of a head, one word per thread (thread tid < 64 W: row
// tid % 64, word tid / 64), rows >= N zero, stored as the fp4 {0, 1} A-operand rows of the QK
// tile (the forward's K staging).
template <int W>
struct SignTile {
    uint32_t word;
    __device__ __forceinline__ void load(const uint32_t* bits, int r0, int N) {
        const int id = threadIdx.x, w = id >> 6, r = id & 63;
        word = id < kBC * W && r0 + r < N ? bits[(int64_t)(r0 + r) * W + w] : 0u;
    }
    __device__ __forceinline__ void store_fp4(uint32_t* dst, int d) const {
        const int id = threadIdx.x, w = id >> 6, r = id & 63;
        if (id < kBC * W) {
            uint32_t x = word;
            const int left = d - 32 * w;
            if (left < 32) x &= (1u << left) - 1u;
            uint32_t o[4];
            unpack_bits32_f4(x, o);
            const int t = (r & 15) >> 2, m = 4 * (r >> 4) + (r & 3);
            *reinterpret_cast<uint4*>(&dst[((t * W + w) * 16 + m) * 4]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
};

// Relative position on any grid: the table rows that queries [q0, q0 + 64) and keys [j0, j0 + 64)
// touch, from row ri_min - rjm + gh - 1 (rjm: grid row of the tile's last key), at row stride
// 2 gw - 1 (entries past the table read 0, through the buffer's range); off: that start's element
// offset in the head's table.
struct WinTile {
    uint32_t v[kRelposWin / 256];  // raw table bits (fp32, or fp16 in the low half), converted when stored
    int off, f32;
    __device__ __forceinline__ void load(const BwArgs& a, const void* table, int q0, int j0) {
        const int gw = a.gw, row_len = 2 * gw - 1, tsz = (2 * a.gh - 1) * row_len;
        const int ri_min = q0 / gw, rjm = min((j0 + kBC - 1) / gw, a.gh - 1);
        off = (ri_min - rjm + a.gh - 1) * row_len;
        f32 = a.bias_f32;
        const int esz = f32 ? 4 : 2;
        const __amdgpu_buffer_rsrc_t tr = buffer_rsrc((const char*)table + (int64_t)off * esz, (tsz - off) * esz);
#pragma unroll
        for (int i = 0; i < kRelposWin / 256; ++i) {
            const int o = (threadIdx.x + 256 * i) * esz;
            v[i] = f32 ? __builtin_amdgcn_raw_buffer_load_b32(tr, o, 0, 0) : __builtin_amdgcn_raw_buffer_load_b16(tr, o, 0, 0);
        }
    }
    __device__ __forceinline__ void store(float* win) const {
#pragma unroll
        for (int i = 0; i < kRelposWin / 256; ++i)
            win[threadIdx.x + 256 * i] = f32 ? __uint_as_float(v[i]) : (float)__builtin_bit_cast(_Float16, (uint16_t)v[i]);
    }
};

// Dense bias of queries [i0, i0 + 64) and keys [k0, k0 + 64) of head h as fp32 [query][key]
// (entries past N zero): 16-byte loads along the rows (row starts are 16-byte aligned), 2 per
// thread for fp16 and 4 for fp32.
template <bool F32>
struct DenseTile {
    static constexpr int EPC = F32 ? 4 : 8, CPR = kBC / EPC, IT = kBR * CPR / 256;  // elements per chunk, chunks per row
    uint4 v[IT];
    __device__ __forceinline__ void load(const BwArgs& a, int h, int i0, int k0) {
        const int N = a.N;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int i = threadIdx.x + 256 * k, r = i / CPR, c = i - r * CPR;
            v[k] = make_uint4(0u, 0u, 0u, 0u);
            if (i0 + r < N && k0 + EPC * c < N)  // the chunk then lies within the row's bias_ld entries
                v[k] = *reinterpret_cast<const uint4*>((const char*)a.bias +
                                                        (((int64_t)h * N + i0 + r) * a.bias_ld + k0 + EPC * c) * (F32 ? 4 : 2));
        }
    }
    __device__ __forceinline__ void store(float* dst, int k0, int N) const {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int i = threadIdx.x + 256 * k, r = i / CPR, c = i - r * CPR;
            float f[EPC];
            if constexpr (F32) {
                f[0] = __uint_as_float(v[k].x); f[1] = __uint_as_float(v[k].y);
                f[2] = __uint_as_float(v[k].z); f[3] = __uint_as_float(v[k].w);
            } else {
                const h8 x = __builtin_bit_cast(h8, v[k]);
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (float)x[e];
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if (k0 + EPC * c + e >= N) f[e] = 0.0f;  // padding columns past N
            }
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
                *reinterpret_cast<float4*>(&dst[r * kBC + EPC * c + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
        }
    }
};

// ---------------------------------------------------------------------------------------------
// (ST: the row statistics pass, which stages only the score operands)
template <int NT, int BIAS, bool ST = false>
struct alignas(16) BwQLds {
    static constexpr int W = (NT + 1) / 2, CP = 32 * W, RP = CP + 8, TPK = kBC + 8;
    uint32_t k[4 * W * 16 * 4];
    float mu[kBC];
    __bf16 vh[ST ? 8 : kBC * RP];  // V^ of the tile's keys [key][channel]
    __bf16 sk[ST ? 8 : CP * TPK];  // sign(k) [channel][key]
    float tw[BIAS == BK_RELPOS_G ? kRelposWin : 4];
    float dwin[BIAS == BK_RELPOS_G && !ST ? kTabMax : 4];  // the whole table's gradient, or one tile's window
    int kk[kBC];
};

// A workgroup per 64 queries.  STATS: the row max, row sum and Delta of its queries (a few KB of
// LDS, up to 8 waves per SIMD).  Otherwise: dS, the bias gradient and dq, from the row
// statistics and the prepared operand arrays (LDS allows at most 3 workgroups per CU: registers
// up to that occupancy hold a tile's staged loads without spilling).
// RUN16 (relative position on a grid whose width is a multiple of 16, d > 32): a wave's 16
// queries lie in one grid row and so do the 16 keys of a lane group, so the 256 dS values of a
// (wave, group) pair fall on the 31 table entries of their diagonals ci - cj: they are summed
// along those diagonals in LDS first (the V^ and sign tiles' space, free after dQ), and 2 LDS
// atomics per lane replace 16.
template <int NT, int BIAS, bool STATS, bool RUN16 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, STATS ? 8 : 3))) void bw_rows_kernel(BwArgs a) {
    typedef BwQLds<NT, BIAS, STATS> Lt;
    constexpr int W = Lt::W, CP = Lt::CP, RP = Lt::RP, TPK = Lt::TPK, NCB = 2 * W;
    static_assert(!RUN16 || 2 * (kBC * RP + CP * TPK) >= 4 * 4 * 16 * 17 * 4, "diagonal scratch fits the two tiles");
    constexpr bool DENSE = BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32;
    __shared__ Lt L;
    const int N = a.N, d = a.d;
    const int nqb = (N + kBR - 1) / kBR;
    const int lb = xcd_logical_block(blockIdx.x, a.B * a.H * nqb);
    const int bh = lb / nqb, q0 = (lb % nqb) * kBR, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntiles = (N + kBC - 1) / kBC;

    FwdArgs fa = {};
    fa.qbits = a.qbits; fa.qmu = a.qmu; fa.N = N; fa.d = d; fa.qk_scale = a.qk_scale;
    const int qw0 = q0 + wave * 16;
    const LaneQ lq = lane_query<NT>(fa, bh, qw0, g, n16);
    const int i = lq.qi;
    const int64_t tok = (int64_t)bh * N + i;

    const int gw = a.gw, row_len = 2 * gw - 1;
    const int64_t tsz = (int64_t)(2 * a.gh - 1) * row_len;
    const void* table = nullptr;
    int aq = 0;
    if (BIAS == BK_RELPOS_G) {
        table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz) : (const void*)((const _Float16*)a.bias + h * tsz);
        const int ri = i / gw, ci = i - ri * gw;
        aq = (ri - q0 / gw) * row_len + ci + gw - 1;
    }
    const int esz = BIAS == BK_DENSE_F32 ? 4 : 2;
    const char* brow = nullptr;
    int brow_bytes = 0;
    if (DENSE) {
        const int r0 = min(qw0, N);
        brow = (const char*)a.bias + ((int64_t)h * N + r0) * a.bias_ld * esz;
        brow_bytes = min(N - r0, 16) * (int)a.bias_ld * esz;
    }
    const int bvoff = (n16 * (int)a.bias_ld + 16 * g) * esz;

    // Stage key tile j0: fp4 K operand, mu_k, (relative position) window and key parts, and
    // (not STATS) the V^ and sign(k) tiles.  Returns the window's table offset.
    auto stage = [&](int j0) {
        SignTile<W> kst;
        kst.load(a.kbits + (int64_t)bh * N * W, j0, N);
        const float mu = tid < kBC && j0 + tid < N ? a.kmu[(int64_t)bh * N + j0 + tid] : 0.0f;
        WinTile win;
        if (BIAS == BK_RELPOS_G) win.load(a, table, q0, j0);
        BfTile<kBC, CP> tvh;
        BfTile<CP, kBC> tsk;
        const int64_t t0 = ((int64_t)bh * a.Np + j0) * CP;
        if (!STATS) {
            tvh.load(a.vh + t0);
            tsk.load(a.sk + t0);
        }
        // (every load above is issued before the stores below)
        kst.store_fp4(L.k, d);
        if (tid < kBC) L.mu[tid] = mu;
        int woff = 0;
        if (BIAS == BK_RELPOS_G) {
            win.store(L.tw);
            woff = win.off;
            if (tid < kBC) {
                const int j = min(j0 + tid, N - 1);  // keys past N are masked: any in-window entry
                const int rj = j / gw;
                L.kk[tid] = -4 * (rj * row_len + j - rj * gw);
            }
        }
        if (!STATS) {
            tvh.template store<RP>(L.vh);
            tsk.template store<TPK>(L.sk);
        }
        return woff;
    };
    // Scores of key tile j0 for the lane's query (keys >= N: -inf), the forward's tile code.
    // Dense bias rows of the lane's query for key tile j0 (fetched a tile ahead of their use).
    auto fetch_bias = [&](int j0, BiasRegs<BIAS>& br) {
        if (DENSE && j0 < N) load_bias<BIAS>(br, buffer_rsrc(brow + j0 * esz, brow_bytes - j0 * esz), bvoff);
    };
    auto scores = [&](int j0, float (&S)[16], float& mloc, const BiasRegs<BIAS>& br) {
        const int jg = j0 + 16 * g;
        const float* wrun = L.tw;
        if (BIAS == BK_RELPOS_G) {
            const int rjm = min((j0 + kBC - 1) / gw, a.gh - 1);
            wrun = L.tw + aq + rjm * row_len;  // the keys' parts (L.kk) are gathered from here
        }
        tile_scores<NT, BIAS>(L.k, L.mu, lq, br, wrun, true, N - jg, S, mloc, L.kk + 16 * g);
    };

    if (STATS) {  // exact row max and row sum (online over the tiles), Delta
        // tile t + 1's operands are loaded into registers before tile t's scores and stored to
        // LDS after them
        SignTile<W> kst;
        float kmu = 0.0f;
        WinTile win;
        auto load_ops = [&](int j0) {
            kst.load(a.kbits + (int64_t)bh * N * W, j0, N);
            kmu = tid < kBC && j0 + tid < N ? a.kmu[(int64_t)bh * N + j0 + tid] : 0.0f;
            if (BIAS == BK_RELPOS_G) win.load(a, table, q0, j0);
        };
        auto store_ops = [&](int j0) {
            kst.store_fp4(L.k, d);
            if (tid < kBC) L.mu[tid] = kmu;
            if (BIAS == BK_RELPOS_G) {
                win.store(L.tw);
                if (tid < kBC) {
                    const int j = min(j0 + tid, N - 1);  // keys past N are masked: any in-window entry
                    const int rj = j / gw;
                    L.kk[tid] = -4 * (rj * row_len + j - rj * gw);
                }
            }
        };
        float mrun = -INFINITY, lpart = 0.0f;
        BiasRegs<BIAS> bcur, bnext;
        fetch_bias(0, bcur);
        load_ops(0);
        for (int t = 0; t < ntiles; ++t) {
            store_ops(t * kBC);
            __syncthreads();
            if (t + 1 < ntiles) load_ops((t + 1) * kBC);
            fetch_bias((t + 1) * kBC, bnext);
            float S[16], mloc = -INFINITY;
            scores(t * kBC, S, mloc, bcur);
            bcur = bnext;
            const float mnew = fmaxf(mrun, rows4_max(mloc));
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) sum += fast_exp2((S[k] - mnew) * kLog2e);
            lpart = lpart * fast_exp2((mrun - mnew) * kLog2e) + sum;
            mrun = mnew;
            __syncthreads();
        }
        const float lrow = rows4_sum(lpart);
        // Delta = dO . O, the lane's share: 16-byte chunks g, g + 4, ... of the two rows (d is a
        // multiple of 8 and the rows 16-byte aligned)
        float dpart = 0.0f;
        if (a.g_f32) {
            const float4* pd = reinterpret_cast<const float4*>((const float*)a.dout + tok * d);
            const float4* po = reinterpret_cast<const float4*>((const float*)a.o + tok * d);
            for (int c = g; 4 * c < d; c += 4) {
                const float4 x = pd[c], y = po[c];
                dpart += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            }
        } else {
            const h8* pd = reinterpret_cast<const h8*>((const _Float16*)a.dout + tok * d);
            const h8* po = reinterpret_cast<const h8*>((const _Float16*)a.o + tok * d);
            for (int c = g; 8 * c < d; c += 4) {
                const h8 x = pd[c], y = po[c];
#pragma unroll
                for (int e = 0; e < 8; ++e) dpart += (float)x[e] * (float)y[e];
            }
        }
        const float delta = rows4_sum(dpart);
        if (lq.live && g == 0) {
            a.m[tok] = mrun;
            a.l[tok] = lrow;
            a.delta[tok] = delta;
        }
        return;
    }

    const float mrow = a.m[tok], delta = a.delta[tok];
    const float inv_l = lq.live ? 1.0f / a.l[tok] : 0.0f;
    // dO s of the lane's query, channels 32 s + 8 g .. + 7 (0 past d and N), two terms: the B
    // operand of dP
    bf8 dhi[W], dlo[W];
#pragma unroll
    for (int s = 0; s < W; ++s) {
        const int c0 = 32 * s + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c0 + e;
            const float x = lq.live && c < d ? ld_any(a.dout, tok * d + c, a.g_f32) * (a.vamax[(int64_t)bh * d + c] / 127.0f)
                                             : 0.0f;
            __bf16 h_, l_;
            split_bf16(x, h_, l_);
            dhi[s][e] = h_;
            dlo[s][e] = l_;
        }
    }

    const bool whole = BIAS == BK_RELPOS_G && a.db && a.dtp;  // the table's gradient accumulates in LDS
    if (BIAS == BK_RELPOS_G && a.db)
        for (int e = tid; e < (whole ? kTabMax : kRelposWin); e += 256) L.dwin[e] = 0.0f;
    BiasRegs<BIAS> bcur, bnext;
    fetch_bias(0, bcur);
    v4f dqacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dqacc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * kBC, jg = j0 + 16 * g;
        fetch_bias(j0 + kBC, bnext);
        const int woff = stage(j0);
        __syncthreads();
        float S[16], mloc = -INFINITY;
        scores(j0, S, mloc, bcur);
        bcur = bnext;
        // dP: keys as MFMA rows (the score tile's order), 32 channels per step
        float dS[16];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
            const __bf16* arow = &L.vh[slot_row(tt, n16) * RP + 8 * g];
#pragma unroll
            for (int s = 0; s < W; ++s) {
                const bf8 av = *reinterpret_cast<const bf8*>(arow + 32 * s);
                acc = mfma_b(av, dhi[s], acc);
                acc = mfma_b(av, dlo[s], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kx = 4 * tt + r;
                const float p = fast_exp2((S[kx] - mrow) * kLog2e) * inv_l;  // 0 for keys >= N and queries >= N
                dS[kx] = p * (acc[r] - delta);
            }
        }
        // the bias gradient: dS of this batch item stored whole (dense; summed over the batch by
        // bw_dbias_kernel), or into the table entries
        if (DENSE && a.db && lq.live) {
            __bf16* drow = a.dsb + ((int64_t)bh * N + i) * a.Np + jg;  // keys past N hold 0
            alignas(16) __bf16 hv[16];  // rounded to bf16 (relative 2^-9): halves the bytes stored and summed
#pragma unroll
            for (int k = 0; k < 16; ++k) hv[k] = (__bf16)dS[k];
#pragma unroll
            for (int k = 0; k < 16; k += 8)
                *reinterpret_cast<uint4*>(drow + k) = *reinterpret_cast<const uint4*>(hv + k);
        }
        if (BIAS == BK_RELPOS_G && a.db && !RUN16) {
            if (lq.live) {  // (keys past N add their dS = 0 at key N - 1's entry: no per-key test)
                const int rjm = min((j0 + kBC - 1) / gw, a.gh - 1);
                const int base = aq + rjm * row_len + (whole ? woff : 0);  // window index (+ its table offset)
                char* drow = reinterpret_cast<char*>(L.dwin) + 4 * base;   // L.kk: the keys' byte offsets from it
                int kb[16];
#pragma unroll
                for (int k = 0; k < 16; k += 4) {
                    const int4 o4 = *reinterpret_cast<const int4*>(&L.kk[16 * g + k]);
                    kb[k] = o4.x; kb[k + 1] = o4.y; kb[k + 2] = o4.z; kb[k + 3] = o4.w;
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) atomicAdd(reinterpret_cast<float*>(drow + kb[k]), dS[k]);
            }
        }
        // dQ: channels as MFMA rows, keys 16 g + 8 s2 + i as k; B = dS mu_k / sqrt(d) in two terms
        float w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = dS[k] * (L.mu[16 * g + k] * a.qk_scale);
        bf8 bh0, bl0, bh1, bl1;
        pack_split(w, 0, bh0, bl0);
        pack_split(w, 1, bh1, bl1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const __bf16* arow = &L.sk[(16 * cb + n16) * TPK + 16 * g];
            const bf8 a0 = *reinterpret_cast<const bf8*>(arow), a1 = *reinterpret_cast<const bf8*>(arow + 8);
            dqacc[cb] = mfma_b(a0, bh0, dqacc[cb]);
            dqacc[cb] = mfma_b(a0, bl0, dqacc[cb]);
            dqacc[cb] = mfma_b(a1, bh1, dqacc[cb]);
            dqacc[cb] = mfma_b(a1, bl1, dqacc[cb]);
        }
        if (RUN16 && a.db) {  // the table gradient by diagonals (see above)
            __syncthreads();  // every wave is done with the V^ and sign tiles
            float* dg = reinterpret_cast<float*>(L.vh) + (wave * 4 + g) * 16 * 17;  // [query col][key col], pitch 17
#pragma unroll
            for (int k = 0; k < 16; ++k) dg[n16 * 17 + k] = dS[k];  // (0 for queries past N)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int d0 = n16 - 15, d1 = n16 + 1;  // this lane's diagonals ci - cj
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t - d0 < 16) s0 += dg[t * 17 + t - d0];       // ci = t, cj = t - d0
                if (t + d1 < 16) s1 += dg[(t + d1) * 17 + t];     // ci = t + d1, cj = t
            }
            if (qw0 < N && jg < N) {  // (N is a multiple of the grid width: whole rows and runs)
                const int ri = qw0 / gw, ci0 = qw0 - ri * gw, rj = jg / gw, cj0 = jg - rj * gw;
                const int t0 = (ri - rj + a.gh - 1) * row_len + ci0 - cj0 + gw - 1 - (whole ? 0 : woff);
                atomicAdd(&L.dwin[t0 + d0], s0);
                if (d1 < 16) atomicAdd(&L.dwin[t0 + d1], s1);
            }
        }
        __syncthreads();
        // flush the window's entries once the next key tile moves it (tiles whose last keys share
        // a grid row share the window)
        const bool moves = t + 1 == ntiles || min((j0 + 2 * kBC - 1) / gw, a.gh - 1) != min((j0 + kBC - 1) / gw, a.gh - 1);
        if (BIAS == BK_RELPOS_G && a.db && !whole && moves) {
            float* dtab = a.db + h * tsz;
            for (int e = tid; e < kRelposWin; e += 256) {
                const float v = L.dwin[e];
                if (v != 0.0f && woff + e < tsz) atomicAdd(dtab + woff + e, v);
                L.dwin[e] = 0.0f;
            }
            __syncthreads();
        }
    }
    if (whole) {  // this workgroup's share of the table gradient, summed over workgroups afterwards
        float* dst = a.dtp + (int64_t)lb * kTabMax;  // logical block: (b H + h) nqb + query block
        for (int e = tid; e < (int)tsz; e += 256) dst[e] = L.dwin[e];
    }

    // ---- dq = mu_q ds ste(q) + sgn(q)/d sum_e ds_e sign(q_e); the lane has channels 16 cb + 4 g + r
    float gpart = 0.0f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g + r;
            if (c < d) gpart += dqacc[cb][r] * (sign_bit(a.qbits, tok, W, c) ? 1.0f : -1.0f);
        }
    const float gsum = rows4_sum(gpart);
    if (!lq.live) return;
    const float mu = a.qmu[tok];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g + r;
            if (c < d) {
                const float x = ld_any(a.q, tok * d + c, a.in_f32);
                a.dq[tok * d + c] = mu * dqacc[cb][r] * ste_grad(x, a.clip) + sgn0(x) / (float)d * gsum;
            }
        }
}

// ---------------------------------------------------------------------------------------------
template <int NT, int BIAS>
struct alignas(16) BwKLds {
    static constexpr int W = (NT + 1) / 2, CP = 32 * W, RP = CP + 8, TPQ = kBR + 8;
    uint32_t q[4 * W * 16 * 4];
    float cq[kBR], mx[kBR], il[kBR], dl[kBR];
    __bf16 dos_hi[kBR * RP], dos_lo[kBR * RP];  // dO s of the tile's queries [query][channel]
    __bf16 dot_hi[CP * TPQ], dot_lo[CP * TPQ];  // dO / (255 l) [channel][query]
    __bf16 sq[CP * TPQ];                        // sign(q) [channel][query]
    float bt[BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32 ? kBR * kBC : 4];  // dense bias tile [query][key]
    float tw[BIAS == BK_RELPOS_G ? kRelposWin : 4];
    int qq[kBR];
};

// (LDS allows at most 2 workgroups per CU: registers up to that occupancy hold a tile's staged
// loads without spilling.)
template <int NT, int BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void bw_k_kernel(BwArgs a) {
    typedef BwKLds<NT, BIAS> Lt;
    constexpr int W = Lt::W, CP = Lt::CP, RP = Lt::RP, TPQ = Lt::TPQ, NCB = 2 * W;
    constexpr bool DENSE = BIAS == BK_DENSE_F16 || BIAS == BK_DENSE_F32;
    __shared__ Lt L;
    const int N = a.N, d = a.d;
    const int nkb = (N + kBC - 1) / kBC;
    const int lb = xcd_logical_block(blockIdx.x, a.B * a.H * nkb);
    const int bh = lb / nkb, k0 = (lb % nkb) * kBC, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqt = (N + kBR - 1) / kBR;

    // the lane's key: fp4 sign operand (+-2) of word g, seed -sum sign(k), mu_k, V^ channels 32 s + 8 g
    const int jraw = k0 + wave * 16 + n16;
    const bool klive = jraw < N;
    const int j = klive ? jraw : N - 1;
    const int64_t tok = (int64_t)bh * N + j;
    v4i kop;
    const float seed = load_q<W>(a.kbits + tok * W, klive, d, g, kop);
    const v4f dseed = v4f{seed, seed, seed, seed};
    const float muk = a.kmu[tok];
    bf8 vreg[W];  // V^ of the lane's key (exact; 0 past d)
#pragma unroll
    for (int s = 0; s < W; ++s) vreg[s] = *reinterpret_cast<const bf8*>(a.vh + ((int64_t)bh * a.Np + j) * CP + 32 * s + 8 * g);

    const int gw = a.gw, row_len = 2 * gw - 1;
    const int64_t tsz = (int64_t)(2 * a.gh - 1) * row_len;
    const void* table = nullptr;
    int kpart = 0;
    if (BIAS == BK_RELPOS_G) {
        table = a.bias_f32 ? (const void*)((const float*)a.bias + h * tsz) : (const void*)((const _Float16*)a.bias + h * tsz);
        const int rjm = min((k0 + kBC - 1) / gw, a.gh - 1);
        const int rj = j / gw, cj = j - rj * gw;
        kpart = (rjm - rj) * row_len + gw - 1 - cj;
    }

    v4f dvacc[NCB], dkacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dvacc[cb] = dkacc[cb] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int qt = 0; qt < nqt; ++qt) {
        const int i0 = qt * kBR;
        // ---- stage the query tile: every load, then the LDS stores
        SignTile<W> qst;
        qst.load(a.qbits + (int64_t)bh * N * W, i0, N);
        float st_cq = 0.0f, st_mx = INFINITY, st_l = 1.0f, st_dl = 0.0f;  // queries >= N: P = 0
        const bool qok = tid < kBR && i0 + tid < N;
        if (qok) {
            const int64_t qt_ = (int64_t)bh * N + i0 + tid;
            st_cq = a.qmu[qt_];
            st_mx = a.m[qt_];
            st_l = a.l[qt_];
            st_dl = a.delta[qt_];
        }
        // (two batches of loads, each issued whole before its stores: one batch of every tile
        // would not fit the registers)
        const int64_t t0 = ((int64_t)bh * a.Np + i0) * CP;
        BfTile<kBR, CP> tdh, tdl;
        tdh.load(a.dos_hi + t0);
        tdl.load(a.dos_lo + t0);
        DenseTile<BIAS == BK_DENSE_F32> btile;
        if (DENSE) btile.load(a, h, i0, k0);
        WinTile win;
        if (BIAS == BK_RELPOS_G) win.load(a, table, i0, k0);
        // (loads above, stores below)
        qst.store_fp4(L.q, d);
        if (tid < kBR) {
            L.cq[tid] = st_cq * a.qk_scale;
            L.mx[tid] = st_mx;
            L.il[tid] = qok ? 1.0f / st_l : 0.0f;
            L.dl[tid] = st_dl;
            if (BIAS == BK_RELPOS_G) {
                const int ii = min(i0 + tid, N - 1), ri = ii / gw;
                L.qq[tid] = (ri - i0 / gw) * row_len + ii - ri * gw;
            }
        }
        tdh.template store<RP>(L.dos_hi);
        tdl.template store<RP>(L.dos_lo);
        if (DENSE) btile.store(L.bt, k0, N);
        if (BIAS == BK_RELPOS_G) win.store(L.tw);
        BfTile<CP, kBR> toh, tol, tsq;
        toh.load(a.dot_hi + t0);
        tol.load(a.dot_lo + t0);
        tsq.load(a.sq + t0);
        // (loads above, stores below)
        toh.template store<TPQ>(L.dot_hi);
        tol.template store<TPQ>(L.dot_lo);
        tsq.template store<TPQ>(L.sq);
        __syncthreads();

        // ---- scores: queries as MFMA rows (slot order), the lane's key as the column
        const int koff = ((g < W ? g : 0) * 16 + n16) * 4;
        float S[16], Pq[16], dS[16];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const v4f D = mfma_f4(*reinterpret_cast<const v4i*>(&L.q[tt * W * 64 + koff]), kop, dseed);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kx = 4 * tt + r, il = 16 * g + kx;  // query i0 + il
                float b = 0.0f;
                if (DENSE) b = L.bt[il * kBC + wave * 16 + n16];
                if (BIAS == BK_RELPOS_G) b = L.tw[L.qq[il] + kpart];
                S[kx] = __builtin_fmaf(D[r] * muk, L.cq[il], b);
            }
        }
        // ---- P, P^ (for dV), dP, dS
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
            const int ro = slot_row(tt, n16) * RP + 8 * g;
#pragma unroll
            for (int s = 0; s < W; ++s) {
                acc = mfma_b(*reinterpret_cast<const bf8*>(&L.dos_hi[ro + 32 * s]), vreg[s], acc);
                acc = mfma_b(*reinterpret_cast<const bf8*>(&L.dos_lo[ro + 32 * s]), vreg[s], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kx = 4 * tt + r, il = 16 * g + kx;
                const float p255 = fast_exp2(__builtin_fmaf(S[kx], kLog2e, kLog2_255 - L.mx[il] * kLog2e));
                Pq[kx] = __builtin_rintf(p255);  // P^; the 1 / (255 l) is in the dO operand
                dS[kx] = p255 * (1.0f / 255.0f) * L.il[il] * (acc[r] - L.dl[il]);
            }
        }
        // ---- dV (A = dO / (255 l), B = P^) and dK (A = sign(q), B = dS mu_q / sqrt(d) in two terms):
        // channels as MFMA rows, queries 16 g + 8 s2 + i as k
        float w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = dS[k] * L.cq[16 * g + k];
        const bf8 p0 = pack_exact(Pq, 0), p1 = pack_exact(Pq, 1);
        bf8 wh0, wl0, wh1, wl1;
        pack_split(w, 0, wh0, wl0);
        pack_split(w, 1, wh1, wl1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int ro = (16 * cb + n16) * TPQ + 16 * g;
            dvacc[cb] = mfma_b(*reinterpret_cast<const bf8*>(&L.dot_hi[ro]), p0, dvacc[cb]);
            dvacc[cb] = mfma_b(*reinterpret_cast<const bf8*>(&L.dot_lo[ro]), p0, dvacc[cb]);
            dvacc[cb] = mfma_b(*reinterpret_cast<const bf8*>(&L.dot_hi[ro + 8]), p1, dvacc[cb]);
            dvacc[cb] = mfma_b(*reinterpret_cast<const bf8*>(&L.dot_lo[ro + 8]), p1, dvacc[cb]);
            const bf8 a0 = *reinterpret_cast<const bf8*>(&L.sq[ro]), a1 = *reinterpret_cast<const bf8*>(&L.sq[ro + 8]);
            dkacc[cb] = mfma_b(a0, wh0, dkacc[cb]);
            dkacc[cb] = mfma_b(a0, wl0, dkacc[cb]);
            dkacc[cb] = mfma_b(a1, wh1, dkacc[cb]);
            dkacc[cb] = mfma_b(a1, wl1, dkacc[cb]);
        }
        __syncthreads();
    }

    // ---- dk = mu_k dt ste(k) + sgn(k)/d sum_e dt_e sign(k_e), dv; channels 16 cb + 4 g + r
    float gpart = 0.0f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g + r;
            if (c < d) gpart += dkacc[cb][r] * (sign_bit(a.kbits, tok, W, c) ? 1.0f : -1.0f);
        }
    const float gsum = rows4_sum(gpart);
    if (!klive) return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g + r;
            if (c < d) {
                const float x = ld_any(a.k, tok * d + c, a.in_f32);
                a.dk[tok * d + c] = muk * dkacc[cb][r] * ste_grad(x, a.clip) + sgn0(x) / (float)d * gsum;
                a.dv[tok * d + c] = dvacc[cb][r];
            }
        }
}

// ---------------------------------------------------------------------------------------------
template <int NT, int BK>
static void launch_bw_bk(const BwArgs& a, hipStream_t s) {
    const unsigned nb = (unsigned)((int64_t)a.B * a.H * ((a.N + kBC - 1) / kBC));
    const unsigned np = (unsigned)((int64_t)a.B * a.H * (a.Np / kBC));
    hipLaunchKernelGGL((bw_rows_kernel<NT, BK, true>), dim3(nb), dim3(256), 0, s, a);
    if (a.g_f32)
        hipLaunchKernelGGL((bw_prep_kernel<16 * NT, true>), dim3(np), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_prep_kernel<16 * NT, false>), dim3(np), dim3(256), 0, s, a);
    if (is_relpos(BK) && a.gw % 16 == 0 && a.W >= 2)
        hipLaunchKernelGGL((bw_rows_kernel<NT, BK, false, (NT > 2)>), dim3(nb), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_rows_kernel<NT, BK, false>), dim3(nb), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bw_k_kernel<NT, BK>), dim3(nb), dim3(256), 0, s, a);
}

// One instantiation per 32-channel width: NT = 2 W (the kernels use W = ceil(NT / 2) only).
template <int NT>
static void launch_bw_nt(const BwArgs& a, int bk, hipStream_t s) {
    switch (bk) {
        case BK_NONE: launch_bw_bk<NT, BK_NONE>(a, s); break;
        case BK_DENSE_F16: launch_bw_bk<NT, BK_DENSE_F16>(a, s); break;
        case BK_DENSE_F32: launch_bw_bk<NT, BK_DENSE_F32>(a, s); break;
        default: launch_bw_bk<NT, BK_RELPOS_G>(a, s); break;
    }
}

int64_t backward_arrays_bytes(int B, int H, int N, int d, int bias_kind) {
    const int64_t Np = ((int64_t)N + kBC - 1) / kBC * kBC, CP = 32 * ((d + 31) / 32), BH = (int64_t)B * H;
    const int64_t extra = bias_kind == 1 ? BH * N * Np * 2 : (bias_kind == 2 ? BH * (Np / kBR) * kTabMax * 4 : 0);
    return 7 * BH * Np * CP * 2 + 3 * BH * N * 4 + extra + 11 * 256;
}

hipError_t launch_backward(const BwLaunch& L, hipStream_t s) {
    BwArgs a = {};
    a.q = L.q; a.k = L.k; a.o = L.o; a.dout = L.dout; a.in_f32 = L.in_f32; a.g_f32 = L.g_f32;
    a.qbits = L.qbits; a.qmu = L.qmu; a.kbits = L.kbits; a.kmu = L.kmu; a.vq = L.vq; a.vamax = L.vamax;
    a.ldv = ((int64_t)L.N + 63) / 64 * 64;
    a.bias = L.bias; a.bias_ld = L.bias_ld; a.bias_f32 = L.bias_f32; a.gh = L.gh; a.gw = L.gw;
    a.B = L.B; a.H = L.H; a.N = L.N; a.d = L.d; a.W = (L.d + 31) / 32; a.Np = (int)(((int64_t)L.N + kBC - 1) / kBC * kBC);
    a.qk_scale = (float)(1.0 / sqrt((double)L.d));
    a.clip = L.clip;
    // arrays in the scratch region, each 256-byte aligned
    const int64_t BH = (int64_t)L.B * L.H, CP = 32 * a.W;
    auto up = [](int64_t bytes) { return (bytes + 255) / 256 * 256; };
    char* p = reinterpret_cast<char*>(L.scratch);
    const int64_t arr = up(BH * a.Np * CP * 2), vec = up(BH * L.N * 4);
    __bf16** arrays[7] = {&a.vh, &a.dos_hi, &a.dos_lo, &a.sk, &a.sq, &a.dot_hi, &a.dot_lo};
    for (__bf16** x : arrays) {
        *x = reinterpret_cast<__bf16*>(p);
        p += arr;
    }
    a.m = reinterpret_cast<float*>(p); p += vec;
    a.l = reinterpret_cast<float*>(p); p += vec;
    a.delta = reinterpret_cast<float*>(p); p += vec;
    a.dsb = L.bias_kind == 1 ? reinterpret_cast<__bf16*>(p) : nullptr;
    const int64_t tsz = (int64_t)(2 * L.gh - 1) * (2 * L.gw - 1);
    a.dtp = L.bias_kind == 2 && tsz <= kTabMax ? reinterpret_cast<float*>(p) : nullptr;
    a.dq = L.dq; a.dk = L.dk; a.dv = L.dv; a.db = L.db;
    if (L.db && L.db_count > 0 && L.bias_kind == 2 && !a.dtp)  // table entries collect atomics
        hipLaunchKernelGGL(bw_zero_kernel, dim3((unsigned)((L.db_count + 255) / 256)), dim3(256), 0, s, L.db, L.db_count);
    int bk = BK_NONE;
    if (L.bias_kind == 1) bk = L.bias_f32 ? BK_DENSE_F32 : BK_DENSE_F16;
    if (L.bias_kind == 2) bk = BK_RELPOS_G;
    switch (a.W) {
        case 1: launch_bw_nt<2>(a, bk, s); break;
        case 2: launch_bw_nt<4>(a, bk, s); break;
        case 3: launch_bw_nt<6>(a, bk, s); break;
        default: launch_bw_nt<8>(a, bk, s); break;
    }
    if (L.db && L.bias_kind == 1)
        hipLaunchKernelGGL(bw_dbias_kernel, dim3((unsigned)(((int64_t)L.H * L.N * (a.Np / 4) + 255) / 256)), dim3(256),
                           0, s, a.dsb, L.db, L.B, L.H, L.N, a.Np);
    if (L.db && a.dtp)
        hipLaunchKernelGGL(bw_dtable_kernel, dim3((unsigned)((L.db_count + 63) / 64)), dim3(256), 0, s, a.dtp, L.db,
                           L.B, L.H, a.Np / kBR, (int)tsz);
    return hipGetLastError();
}

}  // namespace binattn
