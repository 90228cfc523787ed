// abi.hip -- extern "C" entry points declared in include/binattn.h: argument
// validation (before any HIP call), error codes, kernel launches.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "binattn.h"
#include "internal.h"

using namespace binattn;

namespace {

constexpr int kMaxN = 65536;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(int B, int H, int N, int d) {
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return BINATTN_EINVAL;
    if (N > kMaxN || d % 8 != 0 || d < 8 || d > 128) return BINATTN_EUNSUPPORTED;
    const double big = (double)B * H * N * (double)(N > d ? N : d);
    if (big > 4.6e18) return BINATTN_EUNSUPPORTED;
    if ((int64_t)B * H > (int64_t)1 << 24) return BINATTN_EUNSUPPORTED;
    return BINATTN_OK;
}

bool dtype_ok(int dt) { return dt == BINATTN_F32 || dt == BINATTN_F16; }

int device_ready() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return BINATTN_ENODEVICE;
    return BINATTN_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? BINATTN_OK : BINATTN_ELAUNCH; }

int check_bias(int bias_kind, int bias_dtype, const void* bias, int64_t bias_ld, int grid_h, int grid_w, int N) {
    switch (bias_kind) {
        case BINATTN_BIAS_NONE:
            if (bias) return BINATTN_EINVAL;
            break;
        case BINATTN_BIAS_DENSE: {
            if (!bias) return BINATTN_EINVAL;
            if (!dtype_ok(bias_dtype)) return BINATTN_EUNSUPPORTED;
            if (bias_ld < N) return BINATTN_EINVAL;
            if (bias_ld > ((int64_t)1 << 40)) return BINATTN_EUNSUPPORTED;
            const int64_t row_bytes = bias_ld * (bias_dtype == BINATTN_F32 ? 4 : 2);
            // the kernels address the 16 bias rows of a wave through one 32-bit buffer extent
            if (16 * row_bytes >= ((int64_t)1 << 31)) return BINATTN_EUNSUPPORTED;
            if (row_bytes % 16 != 0 || !aligned16(bias)) return BINATTN_EALIGN;
            break;
        }
        case BINATTN_BIAS_RELPOS:
            if (!bias) return BINATTN_EINVAL;
            if (!dtype_ok(bias_dtype)) return BINATTN_EUNSUPPORTED;
            if (grid_h <= 0 || grid_w <= 0 || (int64_t)grid_h * grid_w != N) return BINATTN_EINVAL;
            if (!relpos_window_fits(grid_w)) return BINATTN_EUNSUPPORTED;
            if (!aligned16(bias)) return BINATTN_EALIGN;
            break;
        default:
            return BINATTN_EUNSUPPORTED;
    }
    return BINATTN_OK;
}


FwdArgs forward_args(const uint32_t* q_bits, const float* q_mu, const uint32_t* k_bits, const float* k_mu,
                     const int8_t* vq, const float* vamax, int bias_dtype, const void* bias, int64_t bias_ld,
                     int grid_h, int grid_w, int B, int H, int N, int d, void* out, int out_dtype) {
    FwdArgs a = {};
    a.qbits = q_bits; a.qmu = q_mu; a.kbits = k_bits; a.kmu = k_mu; a.vq = vq; a.vamax = vamax;
    a.bias = bias; a.bias_ld = bias_ld; a.bias_f32 = bias_dtype == BINATTN_F32;
    a.gh = grid_h; a.gw = grid_w;
    a.B = B; a.H = H; a.N = N; a.d = d; a.W = (d + 31) / 32; a.ldv = ((int64_t)N + 63) / 64 * 64;
    a.out = out; a.out_f32 = out_dtype == BINATTN_F32;
    a.qk_scale = (float)(1.0 / sqrt((double)d));
    return a;
}

// Byte offsets of the packed inputs inside a workspace (each region 256-byte aligned).
struct WorkspaceLayout {
    int64_t qbits, kbits, qmu, kmu, vq, vamax, total;
};

WorkspaceLayout workspace_layout(int B, int H, int N, int d) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t tok = (int64_t)B * H * N, W = (d + 31) / 32, ldv = ((int64_t)N + 63) / 64 * 64;
    WorkspaceLayout l;
    l.qbits = 0;
    l.kbits = l.qbits + up(tok * W * 4);
    l.qmu = l.kbits + up(tok * W * 4);
    l.kmu = l.qmu + up(tok * 4);
    l.vq = l.kmu + up(tok * 4);
    l.vamax = l.vq + up((int64_t)B * H * d * ldv);
    l.total = l.vamax + up((int64_t)B * H * d * 4);
    return l;
}

// The whole forward into caller memory: one kernel from fp16 Q, K, V where the shape allows it,
// else the preparation launch into the workspace `ws` (laid out by workspace_layout(B,H,N,d))
// followed by the forward from the packed inputs.  Arguments are already validated.
int run_attention(const void* q, const void* k, const void* v, int dtype, int bias_kind, int bias_dtype,
                  const void* bias, int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d, void* out,
                  int out_dtype, char* ws, hipStream_t stream) {
    if (dtype == BINATTN_F16) {  // short rows: one kernel straight from Q, K, V
        FwdArgs f = forward_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, bias_dtype, bias, bias_ld,
                                 grid_h, grid_w, B, H, N, d, out, out_dtype);
        f.q_raw = static_cast<const _Float16*>(q);
        f.k_raw = static_cast<const _Float16*>(k);
        f.v_raw = static_cast<const _Float16*>(v);
        const hipError_t e = launch_attention_fused(f, bias_kind, stream);
        if (e != hipErrorNotSupported) return launched(e);
    }
    const WorkspaceLayout l = workspace_layout(B, H, N, d);
    uint32_t* qb = reinterpret_cast<uint32_t*>(ws + l.qbits);
    uint32_t* kb = reinterpret_cast<uint32_t*>(ws + l.kbits);
    float* qm = reinterpret_cast<float*>(ws + l.qmu);
    float* km = reinterpret_cast<float*>(ws + l.kmu);
    int8_t* vq = reinterpret_cast<int8_t*>(ws + l.vq);
    float* va = reinterpret_cast<float*>(ws + l.vamax);
    FwdArgs a = forward_args(qb, qm, kb, km, vq, va, bias_dtype, bias, bias_ld, grid_h, grid_w, B, H, N, d, out,
                             out_dtype);
    // streamed rows: the forward packs Q in its own prologue, the preparation takes K and V only
    const bool qx = forward_streams(a, bias_kind);
    if (qx) {
        a.qbits = nullptr;
        a.qmu = nullptr;
        a.qx = q;
        a.qx_f32 = dtype == BINATTN_F32;
    }
    hipError_t e = launch_prepare(qx ? nullptr : q, k, v, dtype == BINATTN_F32, B * H, N, d, binattn_vq_ld(N), qb, qm,
                                  kb, km, vq, va, stream);
    if (e != hipSuccess) return BINATTN_ELAUNCH;
    return launched(launch_forward(a, bias_kind, stream));
}

// ---- Scratch of the no-allocation entry point (binattn_attention_noalloc).  Each device the
// library runs on holds its own copy of this array from the code object's load until the process
// ends.  `scratch` names a host-side stand-in in host code: its device address on the current
// device comes from hipGetSymbolAddress (scratch_on_current_device), and only that address is
// handed to kernels.
constexpr int64_t kScratchBytes = BINATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept; nullptr when the lookup fails.
char* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    return g_scratch_ptr[dev];
}

// Batch items whose packed inputs fit the scratch together (0: not even one).
int noalloc_chunk(int B, int H, int N, int d) {
    if (workspace_layout(1, H, N, d).total > kScratchBytes) return 0;
    int lo = 1, hi = B;  // the workspace grows with the batch: largest nb that fits
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (workspace_layout(mid, H, N, d).total <= kScratchBytes) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace

extern "C" {

int binattn_abi_version(void) { return BINATTN_ABI_VERSION; }

const char* binattn_strerror(int code) {
    switch (code) {
        case BINATTN_OK: return "ok";
        case BINATTN_EINVAL: return "invalid argument (null pointer, non-positive size, inconsistent grid or stride)";
        case BINATTN_EUNSUPPORTED: return "unsupported size, dtype or bias layout";
        case BINATTN_EALIGN: return "device pointer or bias row not 16-byte aligned";
        case BINATTN_ENODEVICE: return "no HIP device visible";
        case BINATTN_ELAUNCH: return "kernel launch failed";
        default: return "unknown error";
    }
}

int binattn_words(int d) { return d > 0 ? (d + 31) / 32 : 0; }

int64_t binattn_vq_ld(int N) { return N > 0 ? ((int64_t)N + 63) / 64 * 64 : 0; }

int binattn_pack_qk(const void* x, int dtype, int B, int H, int N, int d, uint32_t* bits, float* mu,
                    void* stream) {
    if (!x || !bits || !mu) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype)) return BINATTN_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(bits) || !aligned16(mu)) return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    return launched(launch_pack_qk(x, dtype == BINATTN_F32, (int64_t)B * H * N, d, bits, mu, (hipStream_t)stream));
}

int binattn_quant_v(const void* v, int dtype, int B, int H, int N, int d, int8_t* vq, float* vamax,
                    void* stream) {
    if (!v || !vq || !vamax) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype)) return BINATTN_EUNSUPPORTED;
    if (!aligned16(v) || !aligned16(vq) || !aligned16(vamax)) return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    return launched(launch_quant_v(v, dtype == BINATTN_F32, B * H, N, d, binattn_vq_ld(N), vq, vamax,
                                   (hipStream_t)stream));
}

int binattn_vq_canonical(const int8_t* vq, int B, int H, int N, int d, int8_t* out, void* stream) {
    if (!vq || !out) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!aligned16(vq) || !aligned16(out)) return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    return launched(launch_vq_canonical(vq, (int64_t)B * H, N, d, binattn_vq_ld(N), out, (hipStream_t)stream));
}

int binattn_forward(const uint32_t* q_bits, const float* q_mu, const uint32_t* k_bits, const float* k_mu,
                    const int8_t* vq, const float* vamax, int bias_kind, int bias_dtype, const void* bias,
                    int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d, void* out,
                    int out_dtype, void* stream) {
    if (!q_bits || !q_mu || !k_bits || !k_mu || !vq || !vamax || !out) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(out_dtype)) return BINATTN_EUNSUPPORTED;
    if (!aligned16(q_bits) || !aligned16(q_mu) || !aligned16(k_bits) || !aligned16(k_mu) || !aligned16(vq) ||
        !aligned16(vamax) || !aligned16(out))
        return BINATTN_EALIGN;
    if ((rc = check_bias(bias_kind, bias_dtype, bias, bias_ld, grid_h, grid_w, N))) return rc;
    if ((rc = device_ready())) return rc;
    const FwdArgs a = forward_args(q_bits, q_mu, k_bits, k_mu, vq, vamax, bias_dtype, bias, bias_ld, grid_h, grid_w,
                                   B, H, N, d, out, out_dtype);
    return launched(launch_forward(a, bias_kind, (hipStream_t)stream));
}

int binattn_scores_i32(const uint32_t* q_bits, const uint32_t* k_bits, int B, int H, int N, int d, int32_t* D,
                       void* stream) {
    if (!q_bits || !k_bits || !D) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!aligned16(q_bits) || !aligned16(k_bits) || !aligned16(D)) return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    FwdArgs a = {};
    a.qbits = q_bits; a.kbits = k_bits;
    a.B = B; a.H = H; a.N = N; a.d = d; a.W = binattn_words(d);
    a.scores = D;
    return launched(launch_scores(a, (hipStream_t)stream));
}

int binattn_qk_rowstats(const uint32_t* q_bits, const uint32_t* k_bits, int B, int H, int N, int d, int method,
                       float* rowmax, float* rowsum, void* stream) {
    if (!q_bits || !k_bits || !rowmax || !rowsum) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (method != BINATTN_QK_MFMA && method != BINATTN_QK_POPCOUNT) return BINATTN_EUNSUPPORTED;
    if (!aligned16(q_bits) || !aligned16(k_bits) || !aligned16(rowmax) || !aligned16(rowsum)) return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    FwdArgs a = {};
    a.qbits = q_bits; a.kbits = k_bits;
    a.B = B; a.H = H; a.N = N; a.d = d; a.W = binattn_words(d);
    return launched(launch_qk_stats(a, method, rowmax, rowsum, (hipStream_t)stream));
}

int binattn_prepare(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d,
                    uint32_t* q_bits, float* q_mu, uint32_t* k_bits, float* k_mu, int8_t* vq, float* vamax,
                    void* stream) {
    if (!q || !k || !v || !q_bits || !q_mu || !k_bits || !k_mu || !vq || !vamax) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype)) return BINATTN_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_bits) || !aligned16(q_mu) ||
        !aligned16(k_bits) || !aligned16(k_mu) || !aligned16(vq) || !aligned16(vamax))
        return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    return launched(launch_prepare(q, k, v, dtype == BINATTN_F32, B * H, N, d, binattn_vq_ld(N), q_bits, q_mu,
                                   k_bits, k_mu, vq, vamax, (hipStream_t)stream));
}

int64_t binattn_attention_workspace(int B, int H, int N, int d) {
    if (check_dims(B, H, N, d)) return -1;
    return workspace_layout(B, H, N, d).total;
}

int binattn_attention_one_kernel(int dtype, int bias_kind, int bias_dtype, int grid_h, int grid_w, int B, int H, int N,
                                 int d) {
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype)) return BINATTN_EUNSUPPORTED;
    if (bias_kind < BINATTN_BIAS_NONE || bias_kind > BINATTN_BIAS_RELPOS) return BINATTN_EUNSUPPORTED;
    if (bias_kind != BINATTN_BIAS_NONE && !dtype_ok(bias_dtype)) return BINATTN_EUNSUPPORTED;
    if (bias_kind == BINATTN_BIAS_RELPOS) {  // as check_bias
        if (grid_h <= 0 || grid_w <= 0 || (int64_t)grid_h * grid_w != N) return BINATTN_EINVAL;
        if (!relpos_window_fits(grid_w)) return BINATTN_EUNSUPPORTED;
    }
    if (dtype != BINATTN_F16) return 0;
    FwdArgs f = {};
    f.B = B; f.H = H; f.N = N; f.d = d; f.gh = grid_h; f.gw = grid_w;
    f.bias_f32 = bias_dtype == BINATTN_F32;
    return attention_fused_applies(f, bias_kind) ? 1 : 0;
}

int binattn_keep_plan(int64_t nheads, int nqb, int slots, int fused, int* plan) {
    if (!plan || nheads <= 0 || nqb <= 0 || slots <= 0) return BINATTN_EINVAL;
    if (nheads > (int64_t)1 << 24 || nqb > keep_plan_max_blocks()) return BINATTN_EUNSUPPORTED;
    keep_plan_host(nheads, nqb, slots, fused != 0, plan);
    return BINATTN_OK;
}

int binattn_attention(const void* q, const void* k, const void* v, int dtype, int bias_kind, int bias_dtype,
                      const void* bias, int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d,
                      void* out, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out || !workspace) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return BINATTN_EUNSUPPORTED;
    if (workspace_bytes < workspace_layout(B, H, N, d).total) return BINATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return BINATTN_EALIGN;
    if ((rc = check_bias(bias_kind, bias_dtype, bias, bias_ld, grid_h, grid_w, N))) return rc;
    if ((rc = device_ready())) return rc;
    return run_attention(q, k, v, dtype, bias_kind, bias_dtype, bias, bias_ld, grid_h, grid_w, B, H, N, d, out,
                         out_dtype, static_cast<char*>(workspace), (hipStream_t)stream);
}

int64_t binattn_backward_workspace(int B, int H, int N, int d, int bias_kind) {
    if (check_dims(B, H, N, d) || bias_kind < BINATTN_BIAS_NONE || bias_kind > BINATTN_BIAS_RELPOS) return -1;
    return workspace_layout(B, H, N, d).total + backward_arrays_bytes(B, H, N, d, bias_kind);
}

int binattn_qkv_pack(const void* x, const void* w, const void* bias, int B, int N, int H, int d,
                     uint32_t* q_bits, float* q_mu, uint32_t* k_bits, float* k_mu, void* v, void* q, void* k,
                     void* stream) {
    if (!x || !w || !q_bits || !q_mu || !k_bits || !k_mu || !v) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    const int64_t M = (int64_t)B * N;
    int hpt = 0, nb = 0, nmt = 0, nnt = 0;
    if ((int64_t)H * d > (1 << 20) || M > ((int64_t)1 << 40)) return BINATTN_EUNSUPPORTED;
    qkv_pack_plan(H, d, M, &hpt, &nb, &nmt, &nnt);
    if ((int64_t)nmt * nnt > 0x7FFFFFFF) return BINATTN_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || (bias && !aligned16(bias)) || !aligned16(q_bits) || !aligned16(q_mu) ||
        !aligned16(k_bits) || !aligned16(k_mu) || !aligned16(v) || (q && !aligned16(q)) || (k && !aligned16(k)))
        return BINATTN_EALIGN;
    if ((rc = device_ready())) return rc;
    ProjArgs a = {};
    a.x = static_cast<const _Float16*>(x);
    a.w = static_cast<const _Float16*>(w);
    a.bias = static_cast<const _Float16*>(bias);
    a.M = M; a.N = N; a.H = H; a.d = d;
    a.qbits = q_bits; a.qmu = q_mu; a.kbits = k_bits; a.kmu = k_mu;
    a.v = static_cast<_Float16*>(v);
    a.q = static_cast<_Float16*>(q);
    a.k = static_cast<_Float16*>(k);
    return launched(launch_qkv_pack(a, (hipStream_t)stream));
}

int binattn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout, int dtype,
                     int grad_dtype, int bias_kind, int bias_dtype, const void* bias, int64_t bias_ld, int grid_h,
                     int grid_w, int B, int H, int N, int d, float ste_clip, float* dq, float* dk, float* dv,
                     float* dbias, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !o || !dout || !dq || !dk || !dv || !workspace) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype) || !dtype_ok(grad_dtype)) return BINATTN_EUNSUPPORTED;
    if (!(ste_clip >= 0.0f) || ste_clip > 3.0e38f) return BINATTN_EINVAL;  // NaN or infinite clip
    const WorkspaceLayout l = workspace_layout(B, H, N, d);
    if (workspace_bytes < l.total + backward_arrays_bytes(B, H, N, d, bias_kind))
        return BINATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || (dbias && !aligned16(dbias)) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return BINATTN_EALIGN;
    if ((rc = check_bias(bias_kind, bias_dtype, bias, bias_ld, grid_h, grid_w, N))) return rc;
    if (bias_kind == BINATTN_BIAS_NONE && dbias) return BINATTN_EINVAL;
    if ((rc = device_ready())) return rc;
    char* ws = static_cast<char*>(workspace);
    BwLaunch L = {};
    L.qbits = reinterpret_cast<uint32_t*>(ws + l.qbits);
    L.kbits = reinterpret_cast<uint32_t*>(ws + l.kbits);
    L.qmu = reinterpret_cast<float*>(ws + l.qmu);
    L.kmu = reinterpret_cast<float*>(ws + l.kmu);
    L.vq = reinterpret_cast<int8_t*>(ws + l.vq);
    L.vamax = reinterpret_cast<float*>(ws + l.vamax);
    hipError_t e = launch_prepare(q, k, v, dtype == BINATTN_F32, B * H, N, d, binattn_vq_ld(N),
                                  const_cast<uint32_t*>(L.qbits), const_cast<float*>(L.qmu),
                                  const_cast<uint32_t*>(L.kbits), const_cast<float*>(L.kmu),
                                  const_cast<int8_t*>(L.vq), const_cast<float*>(L.vamax), (hipStream_t)stream);
    if (e != hipSuccess) return BINATTN_ELAUNCH;
    L.q = q; L.k = k; L.o = o; L.dout = dout;
    L.in_f32 = dtype == BINATTN_F32; L.g_f32 = grad_dtype == BINATTN_F32;
    L.bias = bias; L.bias_ld = bias_ld; L.bias_f32 = bias_dtype == BINATTN_F32; L.bias_kind = bias_kind;
    L.gh = grid_h; L.gw = grid_w;
    L.B = B; L.H = H; L.N = N; L.d = d; L.clip = ste_clip;
    L.scratch = reinterpret_cast<float*>(ws + l.total);
    L.dq = dq; L.dk = dk; L.dv = dv; L.db = dbias;
    if (bias_kind == BINATTN_BIAS_DENSE) L.db_count = (int64_t)H * N * N;
    if (bias_kind == BINATTN_BIAS_RELPOS) L.db_count = (int64_t)H * (2 * grid_h - 1) * (2 * grid_w - 1);
    return launched(launch_backward(L, (hipStream_t)stream));
}

int binattn_attention_noalloc(const void* q, const void* k, const void* v, int dtype, int bias_kind, int bias_dtype,
                              const void* bias, int64_t bias_ld, int grid_h, int grid_w, int B, int H, int N, int d,
                              void* out, int out_dtype, void* stream) {
    if (!q || !k || !v || !out) return BINATTN_EINVAL;
    int rc = check_dims(B, H, N, d);
    if (rc) return rc;
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return BINATTN_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return BINATTN_EALIGN;
    if ((rc = check_bias(bias_kind, bias_dtype, bias, bias_ld, grid_h, grid_w, N))) return rc;
    const int one = binattn_attention_one_kernel(dtype, bias_kind, bias_dtype, grid_h, grid_w, B, H, N, d);
    if (one < 0) return one;
    const int nb = one ? B : noalloc_chunk(B, H, N, d);  // the one-kernel path uses no scratch
    if (nb == 0) return BINATTN_EUNSUPPORTED;            // one batch item's packed inputs exceed the scratch
    if ((rc = device_ready())) return rc;
    char* ws = one ? nullptr : scratch_on_current_device();
    if (!one && !ws) return BINATTN_ELAUNCH;
    // Batch items are independent (the bias is shared over the batch), so the batch runs in
    // chunks of nb items through the same scratch, in stream order.
    const int64_t in_item = (int64_t)H * N * d * (dtype == BINATTN_F32 ? 4 : 2);
    const int64_t out_item = (int64_t)H * N * d * (out_dtype == BINATTN_F32 ? 4 : 2);
    for (int b0 = 0; b0 < B; b0 += nb) {
        const int n = B - b0 < nb ? B - b0 : nb;
        const int64_t io = b0 * in_item;
        rc = run_attention(static_cast<const char*>(q) + io, static_cast<const char*>(k) + io,
                           static_cast<const char*>(v) + io, dtype, bias_kind, bias_dtype, bias, bias_ld, grid_h,
                           grid_w, n, H, N, d, static_cast<char*>(out) + b0 * out_item, out_dtype, ws,
                           (hipStream_t)stream);
        if (rc) return rc;
    }
    return BINATTN_OK;
}

}  // extern "C"
