/*
 * binattn_oracle.c -- plain, slow CPU oracle for the BinaryAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU path is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or constant with the
 * HIP library, and it never reads anything the HIP library produced.
 *
 * Source of the method: "BinaryAttention: One-bit QK-Attention for Vision and
 * Diffusion Transformers" (CVPR 2026, arXiv 2603.09582), paper-notes page,
 * section "Method details":
 *   - Key design 1 (Scaled Binary Representations): Q and K keep only their sign,
 *     a per-token scale mu carries the magnitude; the sign dot product is computed
 *     with XNOR/XOR + popcount.
 *   - Key design 2 (Bias Enhancement): S_ij = mu_q mu_k s_i^T t_j / sqrt(d) + b_ij,
 *     with b a dense learnable matrix or a relative-position bias.
 *   - Key design 3 (Hybrid Quantization): the softmax output P is quantised to
 *     unsigned 8 bit with the static scale 1/255; V is quantised channel-wise to
 *     8 bit; PV is an integer product.
 *   - Loss and training strategy (hardware implementation bullet): the kernel is a
 *     FlashAttention2-style tiled kernel (softmax with running max and row sum).
 *
 * Arithmetic: fp64 throughout, except the V quantiser, which is defined in fp32
 * so that a GPU implementation can reproduce it bit for bit.  Readings of points
 * the pages leave open (all listed in the design notes of the repository):
 *   mu      = mean |x| over the d channels of one token, stored as fp32;
 *   sign    = +1 iff x >= 0 (so -0.0 -> +1), bit = 1 <=> +1, pad bits 0;
 *   softmax = FlashAttention2 reading: the quantised quantity is the unnormalised
 *             P~ = exp(S - rowmax) in (0,1]; the row sum l = sum P~ is kept in
 *             floating point and divides in the epilogue;
 *   P^      = round-half-even(255 * P~) in {0..255};
 *   V^      = clamp(rint(fl32(v * fl32(127/a_c))), -127, 127), s_c = fl32(a_c/127),
 *             a_c = max_j |v_jc| over the tokens of one (batch, head), a_c = 0 -> 0;
 *   O_ic    = s_c * sum_j P^_ij V^_jc / (255 * l_i).
 * Relative-position bias: token n sits at (r, c) = (n / gw, n % gw) on a gh x gw
 * grid; b_ij = T[h, (r_i - r_j + gh - 1) * (2 gw - 1) + (c_i - c_j + gw - 1)].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NO_PQUANT 1 /* flag: use P~ itself instead of P^/255 */
#define ORACLE_NO_VQUANT 2 /* flag: use v itself instead of s * V^ */

enum { BIAS_NONE = 0, BIAS_DENSE = 1, BIAS_RELPOS = 2 };

int oracle_words(int d) { return (d + 31) / 32; }

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Key design 1: one sign bit per channel plus the per-token scale mu. */
void oracle_pack_qk(const double* x, int64_t ntok, int d, uint32_t* bits, float* mu) {
    const int W = oracle_words(d);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        const double* row = x + t * d;
        uint32_t* out = bits + t * W;
        double sum = 0.0;
        for (int w = 0; w < W; ++w) out[w] = 0u;
        for (int c = 0; c < d; ++c) {
            if (row[c] >= 0.0) out[c / 32] |= 1u << (c % 32);
            sum += fabs(row[c]);
        }
        mu[t] = (float)(sum / (double)d);
    }
}

/* Key design 3, V half: symmetric channel-wise int8 with one fp32 scale per
 * (batch, head, channel).  vq is [nheads, N, d] row-major. */
void oracle_quant_v(const double* v, int64_t nheads, int64_t N, int d, int8_t* vq, float* scale, float* amax) {
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < nheads; ++bh) {
        const double* vh = v + bh * N * d;
        int8_t* qh = vq + bh * N * d;
        for (int c = 0; c < d; ++c) {
            float a = 0.0f;
            for (int64_t j = 0; j < N; ++j) {
                float x = fabsf((float)vh[j * d + c]);
                if (x > a) a = x;
            }
            if (amax) amax[bh * d + c] = a;
            if (a == 0.0f) {
                scale[bh * d + c] = 0.0f;
                for (int64_t j = 0; j < N; ++j) qh[j * d + c] = 0;
                continue;
            }
            const float s = a / 127.0f;
            const float inv = 127.0f / a;
            scale[bh * d + c] = s;
            for (int64_t j = 0; j < N; ++j) {
                const float prod = (float)vh[j * d + c] * inv;
                float r = rintf(prod);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                qh[j * d + c] = (int8_t)r;
            }
        }
    }
}

static int popcount32(uint32_t x) {
    int n = 0;
    while (x) {
        x &= x - 1u;
        ++n;
    }
    return n;
}

/* Key design 1: D_ij = sum_c sign(q_ic) sign(k_jc) = d - 2 * popcount(q XOR k). */
static int32_t sign_dot(const uint32_t* a, const uint32_t* b, int d) {
    const int W = oracle_words(d);
    int h = 0;
    for (int w = 0; w < W; ++w) h += popcount32(a[w] ^ b[w]);
    return (int32_t)(d - 2 * h);
}

void oracle_scores_i32(const uint32_t* qbits, const uint32_t* kbits, int64_t nheads, int64_t N, int d,
                       int32_t* D) {
    const int W = oracle_words(d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nheads * N; ++r) {
        const int64_t bh = r / N;
        const uint32_t* qi = qbits + r * W;
        for (int64_t j = 0; j < N; ++j) D[r * N + j] = sign_dot(qi, kbits + (bh * N + j) * W, d);
    }
}

/* Selected rows of D: rows[] index the flattened (bh, i) space; D_rows is [nrows, N]. */
void oracle_scores_rows(const uint32_t* qbits, const uint32_t* kbits, int64_t nheads, int64_t N, int d,
                        const int64_t* rows, int64_t nrows, int32_t* D_rows) {
    const int W = oracle_words(d);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t];
        if (r < 0 || r >= nheads * N) continue;
        const int64_t bh = r / N;
        for (int64_t j = 0; j < N; ++j) D_rows[t * N + j] = sign_dot(qbits + r * W, kbits + (bh * N + j) * W, d);
    }
}

typedef struct {
    int64_t B, H, N;
    int d, W, flags;
    int bias_kind, gh, gw;
    const double* bias;
    const double* v;
    uint32_t* qb;
    uint32_t* kb;
    float* qmu;
    float* kmu;
    int8_t* vq;
    float* vs;
} fwd_ctx;

static double bias_at(const fwd_ctx* c, int64_t h, int64_t i, int64_t j) {
    if (c->bias_kind == BIAS_DENSE) return c->bias[(h * c->N + i) * c->N + j];
    if (c->bias_kind == BIAS_RELPOS) {
        const int64_t ri = i / c->gw, ci = i % c->gw, rj = j / c->gw, cj = j % c->gw;
        const int64_t row = ri - rj + c->gh - 1, col = ci - cj + c->gw - 1;
        const int64_t tsz = (int64_t)(2 * c->gh - 1) * (2 * c->gw - 1);
        return c->bias[h * tsz + row * (2 * c->gw - 1) + col];
    }
    return 0.0;
}

/* One query row (b, h, i): score, exact-max softmax, P quantiser, integer PV,
 * dequantise and normalise.  S and ph are caller scratch of length N. */
static void forward_row(const fwd_ctx* c, int64_t bh, int64_t i, double* S, double* ph, double* out,
                        double* m_out, double* l_out, uint8_t* phat_out) {
    const int64_t N = c->N, h = bh % c->H;
    const int d = c->d, W = c->W;
    const uint32_t* qi = c->qb + (bh * N + i) * W;
    const double muq = (double)c->qmu[bh * N + i];
    const double sqrt_d = sqrt((double)d);
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        const int32_t D = sign_dot(qi, c->kb + (bh * N + j) * W, d);
        S[j] = muq * (double)c->kmu[bh * N + j] * (double)D / sqrt_d + bias_at(c, h, i, j);
        if (S[j] > m) m = S[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        const double pt = exp(S[j] - m);
        l += pt;
        ph[j] = (c->flags & ORACLE_NO_PQUANT) ? pt : nearbyint(255.0 * pt);
        if (phat_out) phat_out[j] = (uint8_t)nearbyint(255.0 * pt);
    }
    const double pscale = (c->flags & ORACLE_NO_PQUANT) ? 1.0 : 255.0;
    for (int ch = 0; ch < d; ++ch) {
        double acc = 0.0;
        if (c->flags & ORACLE_NO_VQUANT) {
            const double* vh = c->v + bh * N * d;
            for (int64_t j = 0; j < N; ++j) acc += ph[j] * vh[j * d + ch];
            out[ch] = acc / (pscale * l);
        } else {
            const int8_t* qh = c->vq + bh * N * d;
            for (int64_t j = 0; j < N; ++j) acc += ph[j] * (double)qh[j * d + ch];
            out[ch] = (double)c->vs[bh * d + ch] * acc / (pscale * l);
        }
    }
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
}

static int ctx_init(fwd_ctx* c, const double* q, const double* k, const double* v, int bias_kind,
                    const double* bias, int gh, int gw, int64_t B, int64_t H, int64_t N, int d, int flags) {
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return -1;
    if (bias_kind == BIAS_RELPOS && ((int64_t)gh * gw != N || gh <= 0 || gw <= 0)) return -1;
    if (bias_kind != BIAS_NONE && !bias) return -1;
    memset(c, 0, sizeof(*c));
    c->B = B; c->H = H; c->N = N; c->d = d; c->W = oracle_words(d); c->flags = flags;
    c->bias_kind = bias_kind; c->bias = bias; c->gh = gh; c->gw = gw; c->v = v;
    const int64_t ntok = B * H * N;
    c->qb = (uint32_t*)malloc(sizeof(uint32_t) * ntok * c->W);
    c->kb = (uint32_t*)malloc(sizeof(uint32_t) * ntok * c->W);
    c->qmu = (float*)malloc(sizeof(float) * ntok);
    c->kmu = (float*)malloc(sizeof(float) * ntok);
    c->vq = (int8_t*)malloc((size_t)ntok * d);
    c->vs = (float*)malloc(sizeof(float) * B * H * d);
    if (!c->qb || !c->kb || !c->qmu || !c->kmu || !c->vq || !c->vs) return -2;
    oracle_pack_qk(q, ntok, d, c->qb, c->qmu);
    oracle_pack_qk(k, ntok, d, c->kb, c->kmu);
    oracle_quant_v(v, B * H, N, d, c->vq, c->vs, NULL);
    return 0;
}

static void ctx_free(fwd_ctx* c) {
    free(c->qb); free(c->kb); free(c->qmu); free(c->kmu); free(c->vq); free(c->vs);
}

/* Whole forward: out [B,H,N,d] fp64.  m_out / l_out [B,H,N] and phat_out
 * [B,H,N,N] are optional diagnostics (NULL to skip).  Returns 0 on success. */
int oracle_forward(const double* q, const double* k, const double* v, int bias_kind, const double* bias,
                   int gh, int gw, int64_t B, int64_t H, int64_t N, int d, int flags, double* out,
                   double* m_out, double* l_out, uint8_t* phat_out) {
    fwd_ctx c;
    int rc = ctx_init(&c, q, k, v, bias_kind, bias, gh, gw, B, H, N, d, flags);
    if (rc) { if (rc == -2) ctx_free(&c); return rc; }
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * N);
        double* ph = (double*)malloc(sizeof(double) * N);
        const int ok = S && ph;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
        /* every thread reaches the worksharing loop; one without its buffers only skips work */
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            if (ok)
                forward_row(&c, r / N, r % N, S, ph, out + r * d, m_out ? m_out + r : NULL,
                            l_out ? l_out + r : NULL, phat_out ? phat_out + r * N : NULL);
        }
        free(S);
        free(ph);
    }
    ctx_free(&c);
    return fail ? -2 : 0;
}

/* Selected rows only: rows[] index the flattened (b, h, i) space; out_rows is
 * [nrows, d].  Used to check full-size launches on a sample of outputs. */
int oracle_forward_rows(const double* q, const double* k, const double* v, int bias_kind, const double* bias,
                        int gh, int gw, int64_t B, int64_t H, int64_t N, int d, int flags, const int64_t* rows,
                        int64_t nrows, double* out_rows) {
    fwd_ctx c;
    int rc = ctx_init(&c, q, k, v, bias_kind, bias, gh, gw, B, H, N, d, flags);
    if (rc) { if (rc == -2) ctx_free(&c); return rc; }
    int fail = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * N);
        double* ph = (double*)malloc(sizeof(double) * N);
        const int ok = S && ph;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t r = rows[t];
            if (!ok || r < 0 || r >= B * H * N) continue;
            forward_row(&c, r / N, r % N, S, ph, out_rows + t * d, NULL, NULL, NULL);
        }
        free(S);
        free(ph);
    }
    ctx_free(&c);
    return fail ? -2 : 0;
}

/* ---------------------------------------------------------------------------------------------
 * Backward of the quantisation-aware forward (key design 4: QAT with a straight-through
 * estimator for sign).  The forward above is the model; its backward, given dO, is derived here
 * step by step under these readings (the pages only say that the sign is passed straight
 * through):
 *   - sign: d sign(x)/dx := ste(x) = 1, or 1 when |x| <= clip and 0 otherwise (clip > 0);
 *   - mu = mean|x| is differentiated exactly: d mu/dx_c = sgn(x_c)/d with sgn(0) = 0;
 *   - the P and V quantisers are straight-through: P^/255 passes its gradient to P~ and
 *     s_c V^ to v, while their forward values are the quantised ones;
 *   - the row max m is a constant (it only shifts the exponent: FlashAttention-2's convention);
 *   - the row sum l = sum P~ is differentiated.
 * With A = P^/255, Vt = s V^ (dequantised), O = A Vt / l:
 *   dVt_j = sum_i A_ij dO_i / l_i,   Delta_i = dO_i . O_i,   dP_ij = dO_i . Vt_j,
 *   dS_ij = (P~_ij / l_i) (dP_ij - Delta_i),   db_ij = dS_ij (summed over the batch; the
 *   relative-position table entry of (i, j) collects every dS_ij that indexes it),
 *   with s_i = mu_q sign(q_i) and t_j = mu_k sign(k_j):
 *   ds_i = sum_j dS_ij t_j / sqrt(d),   dt_j = sum_i dS_ij s_i / sqrt(d),
 *   dq_ic = mu_q ds_ic ste(q_ic) + sgn(q_ic)/d sum_e ds_ie sign(q_ie)   (likewise dk), dv = dVt.
 * Outputs: dq, dk, dv [B,H,N,d]; db dense [H,N,N] or table [H,(2gh-1)(2gw-1)] (NULL: skipped). */
static int team_size(void) {
#ifdef _OPENMP
    return omp_get_num_threads();
#else
    return 1;
#endif
}

static double ste_grad(double x, double clip) { return (clip > 0.0 && fabs(x) > clip) ? 0.0 : 1.0; }

static double sgn0(double x) { return x > 0.0 ? 1.0 : (x < 0.0 ? -1.0 : 0.0); }

static int64_t table_index(const fwd_ctx* c, int64_t i, int64_t j) {
    const int64_t ri = i / c->gw, ci = i % c->gw, rj = j / c->gw, cj = j % c->gw;
    return (ri - rj + c->gh - 1) * (2 * c->gw - 1) + (ci - cj + c->gw - 1);
}

int oracle_backward(const double* q, const double* k, const double* v, int bias_kind, const double* bias,
                    int gh, int gw, int64_t B, int64_t H, int64_t N, int d, const double* dout, double clip,
                    double* dq, double* dk, double* dv, double* db) {
    fwd_ctx c;
    int rc = ctx_init(&c, q, k, v, bias_kind, bias, gh, gw, B, H, N, d, 0);
    if (rc) { if (rc == -2) ctx_free(&c); return rc; }
    const int W = c.W;
    const double sqrt_d = sqrt((double)d);
    const int64_t tsz = (int64_t)(2 * gh - 1) * (2 * gw - 1);
    const int64_t dbn = bias_kind == BIAS_DENSE ? H * N * N : (bias_kind == BIAS_RELPOS ? H * tsz : 0);
    if (db) memset(db, 0, sizeof(double) * (size_t)dbn);
    int fail = 0;
    /* one (b, h) at a time per thread; the bias gradient is summed over the batch, so each thread
     * keeps its own copy and the copies are added at the end in thread order */
#pragma omp parallel
    {
        const int64_t nn = N * N;
        double* S = (double*)malloc(sizeof(double) * nn);      /* S, then P~ */
        double* dS = (double*)malloc(sizeof(double) * nn);
        double* l = (double*)malloc(sizeof(double) * N);
        double* O = (double*)malloc(sizeof(double) * N * d);
        double* Vt = (double*)malloc(sizeof(double) * N * d);
        double* sv = (double*)malloc(sizeof(double) * N * d);  /* s_i (queries) */
        double* tv = (double*)malloc(sizeof(double) * N * d);  /* t_j (keys) */
        double* ds = (double*)malloc(sizeof(double) * N * d);
        double* dt = (double*)malloc(sizeof(double) * N * d);
        double* dbl = db ? (double*)calloc((size_t)(dbn > 0 ? dbn : 1), sizeof(double)) : NULL;
        const int ok = S && dS && l && O && Vt && sv && tv && ds && dt && (!db || dbl);
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
        /* every thread reaches the worksharing loops; one without its buffers only skips work */
#pragma omp for schedule(static)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (ok) {
                const int64_t h = bh % H, base = bh * N;
                for (int64_t n = 0; n < N; ++n)
                    for (int ch = 0; ch < d; ++ch) {
                        const double sq = (c.qb[(base + n) * W + ch / 32] >> (ch % 32)) & 1u ? 1.0 : -1.0;
                        const double sk = (c.kb[(base + n) * W + ch / 32] >> (ch % 32)) & 1u ? 1.0 : -1.0;
                        sv[n * d + ch] = (double)c.qmu[base + n] * sq;
                        tv[n * d + ch] = (double)c.kmu[base + n] * sk;
                        Vt[n * d + ch] = (double)c.vs[bh * d + ch] * (double)c.vq[(base + n) * d + ch];
                    }
                /* forward: S, P~ (in S), l, O with A = P^/255 */
                for (int64_t i = 0; i < N; ++i) {
                    double m = -INFINITY;
                    for (int64_t j = 0; j < N; ++j) {
                        double dot = 0.0;
                        for (int ch = 0; ch < d; ++ch) dot += sv[i * d + ch] * tv[j * d + ch];
                        S[i * N + j] = dot / sqrt_d + bias_at(&c, h, i, j);
                        if (S[i * N + j] > m) m = S[i * N + j];
                    }
                    double li = 0.0;
                    for (int64_t j = 0; j < N; ++j) {
                        S[i * N + j] = exp(S[i * N + j] - m);
                        li += S[i * N + j];
                    }
                    l[i] = li;
                    for (int ch = 0; ch < d; ++ch) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < N; ++j) acc += nearbyint(255.0 * S[i * N + j]) / 255.0 * Vt[j * d + ch];
                        O[i * d + ch] = acc / li;
                    }
                }
                /* dVt, dS, db */
                const double* dO = dout + base * d;
                for (int64_t j = 0; j < N; ++j)
                    for (int ch = 0; ch < d; ++ch) {
                        double acc = 0.0;
                        for (int64_t i = 0; i < N; ++i) acc += nearbyint(255.0 * S[i * N + j]) / 255.0 / l[i] * dO[i * d + ch];
                        dv[(base + j) * d + ch] = acc;
                    }
                for (int64_t i = 0; i < N; ++i) {
                    double delta = 0.0;
                    for (int ch = 0; ch < d; ++ch) delta += dO[i * d + ch] * O[i * d + ch];
                    for (int64_t j = 0; j < N; ++j) {
                        double dp = 0.0;
                        for (int ch = 0; ch < d; ++ch) dp += dO[i * d + ch] * Vt[j * d + ch];
                        const double g = S[i * N + j] / l[i] * (dp - delta);
                        dS[i * N + j] = g;
                        if (dbl && bias_kind == BIAS_DENSE) dbl[(h * N + i) * N + j] += g;
                        if (dbl && bias_kind == BIAS_RELPOS) dbl[h * tsz + table_index(&c, i, j)] += g;
                    }
                }
                /* ds, dt, then dq, dk through mu and the straight-through sign */
                for (int64_t i = 0; i < N; ++i)
                    for (int ch = 0; ch < d; ++ch) {
                        double a = 0.0, b2 = 0.0;
                        for (int64_t j = 0; j < N; ++j) {
                            a += dS[i * N + j] * tv[j * d + ch];
                            b2 += dS[j * N + i] * sv[j * d + ch];
                        }
                        ds[i * d + ch] = a / sqrt_d;
                        dt[i * d + ch] = b2 / sqrt_d;
                    }
                for (int64_t n = 0; n < N; ++n) {
                    const double* xq = q + (base + n) * d;
                    const double* xk = k + (base + n) * d;
                    double gq = 0.0, gk = 0.0;  /* sum_e ds_e sign_e: the gradient of mu */
                    for (int ch = 0; ch < d; ++ch) {
                        gq += ds[n * d + ch] * (xq[ch] >= 0.0 ? 1.0 : -1.0);
                        gk += dt[n * d + ch] * (xk[ch] >= 0.0 ? 1.0 : -1.0);
                    }
                    for (int ch = 0; ch < d; ++ch) {
                        dq[(base + n) * d + ch] = (double)c.qmu[base + n] * ds[n * d + ch] * ste_grad(xq[ch], clip) +
                                                  sgn0(xq[ch]) / d * gq;
                        dk[(base + n) * d + ch] = (double)c.kmu[base + n] * dt[n * d + ch] * ste_grad(xk[ch], clip) +
                                                  sgn0(xk[ch]) / d * gk;
                    }
                }
            }
        }
        if (db) {  /* the per-thread bias gradients, added in thread order */
#pragma omp for ordered schedule(static, 1)
            for (int t = 0; t < team_size(); ++t) {
#pragma omp ordered
                if (dbl)
                    for (int64_t e = 0; e < dbn; ++e) db[e] += dbl[e];
            }
        }
        free(S); free(dS); free(l); free(O); free(Vt); free(sv); free(tv); free(ds); free(dt); free(dbl);
    }
    ctx_free(&c);
    return fail ? -2 : 0;
}

/* The producer of Q, K and V: the attention block's linear QKV projection, whose output is what
 * key design 1 binarises (the sign and mean |x| of each token's Q and K) and key design 3
 * quantises (V).  y[m][o] = sum_i x[m][i] w[o][i] + bias[o] in fp64, in index order, for
 * x [M, C], w [O, C] (row o: output feature o), bias [O] or NULL.  mag[m][o] = sum_i
 * |x[m][i] w[o][i]| + |bias[o]| bounds the rounding error of any other summation order (NULL:
 * not written).  The split of the O = 3C outputs into Q, K, V and heads is the caller's. */
void oracle_qkv_project(const double* x, const double* w, const double* bias, int64_t M, int C, int64_t O,
                        double* y, double* mag) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const double* xr = x + m * C;
        for (int64_t o = 0; o < O; ++o) {
            const double* wr = w + o * C;
            double s = bias ? bias[o] : 0.0, a = bias ? fabs(bias[o]) : 0.0;
            for (int i = 0; i < C; ++i) {
                s += xr[i] * wr[i];
                a += fabs(xr[i] * wr[i]);
            }
            y[m * O + o] = s;
            if (mag) mag[m * O + o] = a;
        }
    }
}
