/*
 * binattn.h -- C ABI of the BinaryAttention forward library (AMD MI355X, gfx950).
 *
 * The method: "BinaryAttention: One-bit QK-Attention for Vision and Diffusion
 * Transformers" (CVPR 2026, arXiv 2603.09582), paper-notes page, section
 * "Method details":
 *   key design 1 (Scaled Binary Representations)  -> binattn_pack_qk, binattn_scores_i32
 *   key design 2 (Bias Enhancement)               -> the bias arguments of binattn_forward
 *   key design 3 (Hybrid Quantization)            -> binattn_quant_v, binattn_forward
 *   hardware implementation bullet (a FlashAttention2-style tiled kernel with a
 *   binary QK product and an integer PV product)  -> binattn_forward
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *    caller.  The library never allocates, frees or caches device memory and
 *    keeps no state between calls.  Inputs are read only; outputs are fully
 *    overwritten.  Inputs and outputs must not overlap.
 *  - Every device pointer must be 16-byte aligned (else BINATTN_EALIGN).
 *  - Tensors are dense row-major in the order their shape is written.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; results are
 *    visible after the caller synchronises the stream.
 *  - Return value: BINATTN_OK (0) or a negative BINATTN_E* code.  All argument
 *    checks run before any HIP call; nothing is launched when a check fails.
 *    No call aborts or throws.  A fault inside a kernel (for example from a
 *    pointer that does not cover the documented extent) surfaces at the
 *    caller's next synchronisation, not here.
 *  - Supported sizes: B, H, N >= 1; N <= 65536; d a multiple of 8 with
 *    8 <= d <= 128 (BINATTN_EUNSUPPORTED otherwise); B*H*N*max(d,N) must fit
 *    in 2^62.
 *  - dtype codes: BINATTN_F32 (IEEE binary32), BINATTN_F16 (IEEE binary16).
 */
#ifndef BINATTN_H
#define BINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BINATTN_ABI_VERSION 1

#define BINATTN_F32 0
#define BINATTN_F16 1

#define BINATTN_BIAS_NONE 0
#define BINATTN_BIAS_DENSE 1
#define BINATTN_BIAS_RELPOS 2

#define BINATTN_OK 0
#define BINATTN_EINVAL (-1)       /* NULL pointer, non-positive size, inconsistent grid or leading dimension */
#define BINATTN_EUNSUPPORTED (-2) /* size, dtype or bias layout outside what the kernels implement */
#define BINATTN_EALIGN (-3)       /* a device pointer or bias row is not 16-byte aligned */
#define BINATTN_ENODEVICE (-4)    /* no HIP device is visible */
#define BINATTN_ELAUNCH (-5)      /* the HIP runtime rejected a kernel launch */

/* Version of this ABI (BINATTN_ABI_VERSION of the built library). */
int binattn_abi_version(void);

/* Static text for a return code ("unknown error" for codes it does not know). */
const char* binattn_strerror(int code);

/* Number of 32-bit sign words per token: ceil(d / 32). */
int binattn_words(int d);

/* Key stride (bytes) of a quantised V row: N rounded up to a multiple of 64. */
int64_t binattn_vq_ld(int N);

/*
 * binattn_pack_qk -- sign bits and per-token scale of Q or K.
 * Passage: key design 1 (Scaled Binary Representations): only the sign of each
 * channel is kept, and a per-token scale mu keeps the token's magnitude.
 *
 *   x     [B,H,N,d]   dtype (BINATTN_F16 or BINATTN_F32), read only
 *   bits  [B,H,N,W]   uint32, W = binattn_words(d); bit (c % 32) of word c / 32
 *                     is 1 iff x[..., c] >= 0 (so -0.0 counts as +1); bits for
 *                     c >= d are 0
 *   mu    [B,H,N]     fp32, mean |x| over the d channels of the token
 * x must hold finite values.
 */
int binattn_pack_qk(const void* x, int dtype, int B, int H, int N, int d, uint32_t* bits, float* mu,
                    void* stream);

/*
 * binattn_quant_v -- channel-wise symmetric int8 quantisation of V.
 * Passage: key design 3 (Hybrid Quantization): V is quantised channel-wise to
 * 8 bits.
 *
 *   v      [B,H,N,d]   dtype, read only, finite
 *   vq     [B,H,d,ldv] int8, ldv = binattn_vq_ld(N) (channel-major: the N
 *                      tokens of one channel are contiguous); entries for
 *                      tokens n >= N are written as 0
 *   vamax  [B,H,d]     fp32 channel absmax a; the dequantisation scale of the
 *                      channel is the fp32 quotient a / 127
 * Per (b, h, channel c), in fp32 with IEEE division and round-half-even:
 *   a = max_n |v[n,c]|;  inv = 127 / a;
 *   vq[c,n] = clamp(rint(v[n,c] * inv), -127, 127);  a == 0 -> vq = 0.
 */
int binattn_quant_v(const void* v, int dtype, int B, int H, int N, int d, int8_t* vq, float* vamax,
                    void* stream);

/*
 * binattn_vq_canonical -- the canonical token-major layout of a quantised V.
 * Passage: key design 3 (Hybrid Quantization): V is held as 8-bit integers per
 * token and channel; binattn_quant_v writes them channel-major for the PV
 * product, and this call only rearranges those bytes (no arithmetic).
 *
 *   vq   [B,H,d,ldv] int8 as binattn_quant_v writes it, ldv = binattn_vq_ld(N),
 *                    read only (the whole extent; entries for tokens n >= N are
 *                    ignored)
 *   out  [B,H,N,d]   int8: out[b,h,n,c] = vq[b,h,c,n]
 * Sizes and errors as for binattn_quant_v.
 */
int binattn_vq_canonical(const int8_t* vq, int B, int H, int N, int d, int8_t* out, void* stream);

/*
 * binattn_qkv_pack -- the QKV projection that produces the attention's inputs, with Q and K
 * binarised in its epilogue.
 * Passages: key design 1 (Scaled Binary Representations): Q and K enter the attention only as
 * channel signs and per-token mean |x|, so the producer hands over those; key design 3 (Hybrid
 * Quantization): V is quantised per channel over all N tokens of a head, which binattn_quant_v
 * does afterwards from the fp16 v written here.
 *
 *   x       [B,N,C] fp16, C = H*d: the tokens' hidden states, read only
 *   w       [3C,C]  fp16: row o is output feature o (a linear layer's weight), read only
 *   bias    [3C]    fp16, or NULL for none
 *   Output feature o = p*C + h*d + c is channel c of head h of part p (0: Q, 1: K, 2: V).
 *   y[b,n,o] = fp16(sum_i x[b,n,i] * w[o,i] + bias[o]): fp32 accumulation in an unspecified
 *   order, one round-to-nearest-even to fp16 at the end.
 *   q_bits, q_mu, k_bits, k_mu   [B,H,N,W] uint32 and [B,H,N] fp32: exactly what
 *           binattn_pack_qk writes for the fp16 Q and K of y (bit: y >= 0, -0.0 included;
 *           mu = mean |y| in fp32, pad bits 0)
 *   v       [B,H,N,d] fp16: the V part of y
 *   q, k    [B,H,N,d] fp16, or NULL: the Q and K parts of y themselves, for callers that also
 *           need them (a training step's backward); NULL skips the write
 * Sizes as for the other entry points (d a multiple of 8, 8..128; N <= 65536); B*N <= 2^40.
 * Only fp16 is implemented (the fp16 MFMA).  x, w and bias must hold finite values (the
 * kernel may multiply entries of x by zero weights past the end of a row).  x, w and the
 * outputs must not overlap.
 */
int binattn_qkv_pack(const void* x, const void* w, const void* bias, int B, int N, int H, int d,
                     uint32_t* q_bits, float* q_mu, uint32_t* k_bits, float* k_mu, void* v, void* q, void* k,
                     void* stream);

/*
 * binattn_forward -- BinaryAttention forward from packed Q/K and quantised V.
 * Passages: key design 1 (binary score with per-token scales), key design 2
 * (S_ij = mu_q mu_k s_i.t_j / sqrt(d) + b_ij), key design 3 (P quantised to u8
 * with scale 1/255, integer PV), hardware implementation bullet (one tiled
 * kernel with running max and row sum).
 *
 *   q_bits, k_bits  [B,H,N,W] uint32   from binattn_pack_qk
 *   q_mu, k_mu      [B,H,N]   fp32     from binattn_pack_qk
 *   vq              [B,H,d,ldv] int8   from binattn_quant_v
 *   vamax           [B,H,d]   fp32     from binattn_quant_v (scale s_c = vamax_c / 127)
 *   bias_kind       BINATTN_BIAS_NONE:   bias must be NULL.
 *                   BINATTN_BIAS_DENSE:  bias [H,N,bias_ld] of bias_dtype, entry
 *                       (h,i,j) = b_ij for every batch item; bias_ld >= N and
 *                       bias_ld * sizeof(dtype) a multiple of 16 bytes.
 *                   BINATTN_BIAS_RELPOS: bias is a table [H,(2gh-1)*(2gw-1)] of
 *                       bias_dtype; token n sits at (n / gw, n % gw) on a
 *                       gh x gw grid (gh*gw == N) and
 *                       b_ij = T[h, (r_i-r_j+gh-1)*(2gw-1) + (c_i-c_j+gw-1)].
 *                       Requires gw <= 171 (the rows of T that 64 queries and
 *                       64 keys touch are staged on chip; any gh).  bias_ld
 *                       ignored.
 *   out             [B,H,N,d] of out_dtype
 *
 * Computes, per (b, h, query i):
 *   D_ij = d - 2 popcount(q_bits_i XOR k_bits_j)                (exact integer)
 *   S_ij = q_mu_i * k_mu_j * D_ij / sqrt(d) + b_ij             (fp32)
 *   m = row max of S, l = sum_j exp(S_ij - m) (fp32),
 *   P^_ij = rint(255 * exp(S_ij - m)) in [0,255],
 *   O_ic = s_c * sum_j P^_ij vq_cj / (255 * l_i)                (integer PV)
 * m is the exact row max (two passes over scores held on chip) for rows of at most
 * 256 keys at any d, and for rows of at most 640 keys at d <= 64 with no bias or the
 * dense bias.  Other rows are streamed over key tiles with a running max: a tile is
 * quantised against the max known after it and earlier tiles are rescaled, so P^ may
 * differ by one rounding from the exact-max result.
 * A dense bias whose 16-row extent (16 * bias_ld * element size) reaches 2^31 bytes is
 * BINATTN_EUNSUPPORTED.
 */
int binattn_forward(const uint32_t* q_bits, const float* q_mu, const uint32_t* k_bits, const float* k_mu,
                    const int8_t* vq, const float* vamax, int bias_kind, int bias_dtype, const void* bias,
                    int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d, void* out,
                    int out_dtype, void* stream);

/*
 * binattn_scores_i32 -- the integer sign score matrix, computed by the same
 * binary QK tile code as binattn_forward (test and inspection export).
 * Passage: key design 1: s_i.t_j through XOR and popcount.
 *
 *   q_bits, k_bits [B,H,N,W] uint32;  D [B,H,N,N] int32, D_ij = d - 2 popcount(q_i XOR k_j).
 */
int binattn_scores_i32(const uint32_t* q_bits, const uint32_t* k_bits, int B, int H, int N, int d, int32_t* D,
                       void* stream);

/*
 * binattn_qk_rowstats -- probe of the binary QK tile alone (measurement and test export).
 * Passage: key design 1 computes s_i.t_j with XOR and popcount; the hardware-implementation
 * bullet runs it on binary tensor-core MMAs.  This entry computes every D_ij of a forward
 * launch's tiling with the chosen method and reduces each query row, so the two ways of
 * computing the tile on gfx950 can be timed against each other on identical work:
 *   method BINATTN_QK_MFMA     (0): fp4 MFMA on unpacked LDS operands (what binattn_forward uses);
 *   method BINATTN_QK_POPCOUNT (1): VALU XOR + v_bcnt on LDS-staged sign words.
 *
 *   q_bits, k_bits [B,H,N,W] uint32
 *   rowmax [B,H,N] fp32 = max_j D_ij;  rowsum [B,H,N] fp32 = sum_j D_ij (both exact)
 * Errors as binattn_scores_i32; an unknown method is BINATTN_EUNSUPPORTED.
 */
/*
 * binattn_prepare -- the three input-side calls in one launch where it fits: identical
 * results to binattn_pack_qk(q), binattn_pack_qk(k) and binattn_quant_v(v) (same
 * arguments, same outputs, same errors).  Passages: key designs 1 and 3.
 */
int binattn_prepare(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d,
                    uint32_t* q_bits, float* q_mu, uint32_t* k_bits, float* k_mu, int8_t* vq, float* vamax,
                    void* stream);

/*
 * binattn_attention -- the whole forward from fp16/fp32 Q, K, V, with results identical bit
 * for bit to binattn_prepare into the caller's workspace followed by binattn_forward.  The
 * pages present the method as a drop-in replacement of attention; this is that call.  For
 * fp16 inputs with rows of at most 256 keys, d of 56, 64, 72, 80, 120 or 128 (and, for the
 * relative-position bias, a table window that fits the kernel's staging) it runs as one
 * kernel that packs K, quantises V and packs its queries itself (the workspace is then not
 * written); otherwise as those two calls, except that rows the forward streams (more than
 * 640 keys at d <= 64, more than 256 keys above, and relative-position rows whose whole-row
 * window does not fit) have their queries packed inside the forward's prologue, with the
 * preparation taking only K and V -- the same results, bit for bit.
 * binattn_attention_one_kernel tells whether the one-kernel form applies.
 *
 *   q, k, v    [B,H,N,d] of dtype (contiguous)
 *   bias...    as binattn_forward
 *   out        [B,H,N,d] of out_dtype
 *   workspace  device memory of at least binattn_attention_workspace(B,H,N,d) bytes,
 *              256-byte aligned, owned by the caller; it receives the packed Q/K and
 *              the quantised V (contents unspecified after the call).  Calls that
 *              share a workspace must be ordered on one stream.
 * binattn_attention_workspace returns -1 for unsupported sizes.  Errors as the two
 * calls it makes; a workspace smaller than required is BINATTN_EINVAL, a misaligned
 * one BINATTN_EALIGN.
 */
int64_t binattn_attention_workspace(int B, int H, int N, int d);
/*
 * binattn_attention_one_kernel -- 1 when binattn_attention with these arguments runs as one
 * kernel from Q, K, V, 0 when it runs as binattn_prepare + binattn_forward; the dimension,
 * dtype and relative-position grid checks of binattn_attention give the same error codes.
 */
int binattn_attention_one_kernel(int dtype, int bias_kind, int bias_dtype, int grid_h, int grid_w, int B, int H, int N,
                                 int d);
int binattn_attention(const void* q, const void* k, const void* v, int dtype, int bias_kind, int bias_dtype,
                      const void* bias, int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d,
                      void* out, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * binattn_attention_noalloc -- binattn_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments without the workspace, the same results bit for bit, and no allocation of any
 * kind.  The packed intermediates go to a scratch array of BINATTN_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs on (allocated when its code object loads, kept until
 * the process ends).  The batch runs in chunks of as many batch items as fit the scratch
 * (binattn_attention_workspace(chunk, H, N, d) bytes), in stream order; a shape that runs as
 * one kernel (binattn_attention_one_kernel) uses no scratch.
 *   q, k, v, bias..., out, stream   as binattn_attention
 * Errors as binattn_attention; BINATTN_EUNSUPPORTED (before any launch) when the packed inputs
 * of a single batch item exceed the scratch.  Every call on one device shares that device's
 * scratch: calls that overlap on one device (other streams, other threads) race and must be
 * ordered by the caller.  The scratch needs no clearing: every byte a call reads it wrote first.
 */
#define BINATTN_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
int binattn_attention_noalloc(const void* q, const void* k, const void* v, int dtype, int bias_kind, int bias_dtype,
                              const void* bias, int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d,
                              void* out, int out_dtype, void* stream);

/*
 * binattn_backward -- gradients of the quantisation-aware forward for training (QAT).
 * Passages: key design 4 (quantisation-aware training: the forward keeps sign(Q), sign(K), and
 * a straight-through estimator (STE) makes sign differentiable) and key designs 1-3 (the forward
 * being differentiated).  The pages fix no more; the readings taken:
 *   d sign(x)/dx := 1 (ste_clip == 0) or 1{|x| <= ste_clip} (ste_clip > 0);
 *   mu = mean|x| is differentiated exactly (d mu/dx_c = sgn(x_c)/d, sgn(0) = 0);
 *   the P (u8, scale 1/255) and V (int8 per channel) quantisers are straight-through;
 *   the row max is a constant, the row sum l = sum_j exp(S_ij - m_i) is differentiated.
 * With P = exp(S - m)/l, A = P^/(255 l), Vt = s V^, O the forward output:
 *   dv_j = sum_i A_ij dO_i;  dS_ij = P_ij (dO_i . Vt_j - dO_i . O_i);  dbias = dS (dense: summed
 *   over the batch; relative position: each table entry sums the dS_ij that index it);
 *   ds_i = sum_j dS_ij mu_k_j sign(k_j)/sqrt(d);  dq_ic = mu_q_i ds_ic ste(q_ic) +
 *   sgn(q_ic)/d sum_e ds_ie sign(q_ie);  dk likewise with dt_j = sum_i dS_ij mu_q_i sign(q_i)/sqrt(d).
 * The row statistics and P^ are recomputed with the exact row max.
 *
 *   q, k, v        [B,H,N,d] of dtype (the forward's inputs)
 *   o, dout        [B,H,N,d] of grad_dtype: the forward's output and the gradient of the loss in it
 *   bias...        as binattn_forward
 *   ste_clip       >= 0 (0: no clip)
 *   dq, dk, dv     [B,H,N,d] fp32, fully overwritten
 *   dbias          fp32 dense [H,N,N] (row stride N) or table [H,(2gh-1)(2gw-1)]; fully overwritten;
 *                  may be NULL to skip the bias gradient; must be NULL for BINATTN_BIAS_NONE
 *   workspace      at least binattn_backward_workspace(B,H,N,d,bias_kind) bytes, 256-byte aligned,
 *                  caller-owned (with the dense bias it holds every batch item's dS, B*H*N*ceil64(N)
 *                  floats, summed over the batch in order; with the table, each 64-query block's
 *                  share of a table of at most 4096 entries, summed in order)
 * Errors as binattn_attention; a NaN or infinite ste_clip, a dbias with no bias or a small
 * workspace is BINATTN_EINVAL.  A table of more than 4096 entries collects its gradient with
 * fp32 atomics, so its rounding can vary from call to call; every other output is deterministic.
 * binattn_backward_workspace returns -1 for unsupported sizes or an unknown bias kind.
 */
int64_t binattn_backward_workspace(int B, int H, int N, int d, int bias_kind);
int binattn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout, int dtype,
                     int grad_dtype, int bias_kind, int bias_dtype, const void* bias, int64_t bias_ld, int grid_h,
                     int grid_w, int B, int H, int N, int d, float ste_clip, float* dq, float* dk, float* dv,
                     float* dbias, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * binattn_keep_plan -- inspection export (host only, no device call): how the head-resident
 * forward splits the query blocks of every (b, h) over workgroups.  nheads = B*H heads of
 * nqb = ceil(N / 64) query blocks (1 <= nqb <= 10, the rows that kernel takes), `slots` resident
 * workgroups on the device (the library itself uses the occupancy the runtime reports times the
 * compute units), fused != 0 for the whole-attention variant of binattn_attention.
 *   plan[4] (caller-owned) receives {a, f, b, r}: each head is covered by a segments of f query
 *   blocks (blocks [k f, k f + f), k < a, cut at nqb) followed by b segments of r blocks
 *   (from block a f on); a launch is 8 * ceil(nheads / 8) * (a + b) workgroups, workgroup w on
 *   XCD w % 8, each XCD taking a contiguous eighth of the heads.
 * The plan minimises a list-scheduling model of one XCD's makespan (a head's staging counts as
 * half a query block's work, three for the whole-attention variant).  BINATTN_EINVAL for a NULL
 * plan or non-positive sizes, BINATTN_EUNSUPPORTED for nqb > 10 or nheads > 2^24.
 */
int binattn_keep_plan(int64_t nheads, int nqb, int slots, int fused, int* plan);

#define BINATTN_QK_MFMA 0
#define BINATTN_QK_POPCOUNT 1
int binattn_qk_rowstats(const uint32_t* q_bits, const uint32_t* k_bits, int B, int H, int N, int d, int method,
                        float* rowmax, float* rowsum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BINATTN_H */
