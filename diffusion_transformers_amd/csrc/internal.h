// internal.h -- launchers behind the C ABI (host side; arguments are already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace binattn {

struct FwdArgs {
    const uint32_t* qbits;
    const float* qmu;
    const uint32_t* kbits;
    const float* kmu;
    const int8_t* vq;
    const float* vamax;    // channel absmax of V; the dequantisation scale is vamax / 127
    const void* bias;
    int64_t bias_ld;      // dense: row stride in elements
    int bias_f32;         // bias / table stored as fp32 (else fp16)
    int gh, gw;           // relative-position grid
    int B, H, N, d, W;
    int64_t ldv;          // key stride of vq rows
    void* out;
    int out_f32;
    float qk_scale;       // 1 / sqrt(d)
    int32_t* scores;      // scores export only
    const _Float16* q_raw;  // whole-attention path: fp16 Q, K, V [B,H,N,d] (packed inputs above unused)
    const _Float16* k_raw;
    const _Float16* v_raw;
    int wrs;              // head-resident kernel: LDS row stride of its relative-position window
    const void* qx;       // streamed rows: fp16 / fp32 Q packed in the kernel's prologue (qbits, qmu unused)
    int qx_f32;
};

hipError_t launch_pack_qk(const void* x, int f32, int64_t ntok, int d, uint32_t* bits, float* mu,
                          hipStream_t s);
hipError_t launch_quant_v(const void* v, int f32, int BH, int N, int d, int64_t ldv, int8_t* vq, float* vamax,
                          hipStream_t s);
hipError_t launch_vq_canonical(const int8_t* vq, int64_t BH, int N, int d, int64_t ldv, int8_t* out, hipStream_t s);
// q may be null: then only K and V are prepared.
hipError_t launch_prepare(const void* q, const void* k, const void* v, int f32, int BH, int N, int d, int64_t ldv,
                          uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq, float* vamax,
                          hipStream_t s);
hipError_t launch_forward(const FwdArgs& a, int bias_kind, hipStream_t s);
// Whether launch_forward runs the streaming kernel for this shape (which can pack Q itself).
bool forward_streams(const FwdArgs& a, int bias_kind);
// The forward with the relative-position bias on a grid whose width is not a multiple of 16.
hipError_t launch_forward_gather(const FwdArgs& a, hipStream_t s);
// Whole attention from fp16 Q, K, V in one kernel where the shape allows it (short rows);
// returns hipErrorNotSupported, launching nothing, where it does not.
hipError_t launch_attention_fused(const FwdArgs& a, int bias_kind, hipStream_t s);
bool attention_fused_applies(const FwdArgs& a, int bias_kind);
hipError_t launch_scores(const FwdArgs& a, hipStream_t s);

// Backward of the quantisation-aware forward (backward.hip): packed inputs from launch_prepare,
// scratch of backward_arrays_bytes(B, H, N, d, bias kind) bytes (256-byte aligned).
struct BwLaunch {
    const void* q;
    const void* k;
    const void* o;
    const void* dout;
    int in_f32, g_f32;
    const uint32_t* qbits;
    const float* qmu;
    const uint32_t* kbits;
    const float* kmu;
    const int8_t* vq;
    const float* vamax;
    const void* bias;
    int64_t bias_ld;
    int bias_f32, bias_kind, gh, gw;
    int B, H, N, d;
    float clip;
    float* scratch;
    float* dq;
    float* dk;
    float* dv;
    float* db;
    int64_t db_count;
};
int64_t backward_arrays_bytes(int B, int H, int N, int d, int bias_kind);
hipError_t launch_backward(const BwLaunch& L, hipStream_t s);
hipError_t launch_qk_stats(const FwdArgs& a, int method, float* rowmax, float* rowsum, hipStream_t s);
bool relpos_window_fits(int gw);
// The head-resident kernel's workgroup plan {a, f, b, r} for nheads heads of nqb query blocks
// (nqb <= keep_plan_max_blocks()) on `slots` resident workgroups: per head, a segments of f
// blocks then b segments of r blocks; fused: the whole-attention variant (costlier staging).
int keep_plan_max_blocks();
void keep_plan_host(int64_t nheads, int nqb, int slots, bool fused, int plan[4]);

// The QKV projection with Q/K binarised in its epilogue (project.hip).  The caller fills the
// pointers and x/w shapes (M tokens of C = H d features, N tokens per batch item); the launcher
// fills the tile plan.
struct ProjArgs {
    const _Float16* x;
    const _Float16* w;
    const _Float16* bias;  // may be null
    int64_t M;
    int N, H, d, C, W;
    int hpt, nsec, nmt, nnt;  // head sections per tile, 3H, token tiles, feature tiles
    uint32_t* qbits;
    float* qmu;
    uint32_t* kbits;
    float* kmu;
    _Float16* v;
    _Float16* q;  // may be null
    _Float16* k;  // may be null
};
void qkv_pack_plan(int H, int d, int64_t M, int* hpt, int* nb, int* nmt, int* nnt);
hipError_t launch_qkv_pack(const ProjArgs& a, hipStream_t s);

}  // namespace binattn
