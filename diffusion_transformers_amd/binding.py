"""Thin ctypes binding over libbinattn.so (include/binattn.h).

Argument marshalling only: every step of the BinaryAttention forward runs in
the library's HIP kernels.  PyTorch provides device memory (output tensors are
allocated here with ``torch.empty``) and the stream (``torch.cuda.current_stream()``).
The library must be built (``python -m diffusion_transformers_amd.build`` or
``__graft_entry__.build()``); importing this module without it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbinattn.so")

F32, F16 = 0, 1
BIAS_NONE, BIAS_DENSE, BIAS_RELPOS = 0, 1, 2
ERRORS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EALIGN", -4: "ENODEVICE", -5: "ELAUNCH"}


class BinAttnError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)} ({_lib.binattn_strerror(code).decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.binattn_abi_version.restype = i32
    lib.binattn_strerror.argtypes = [i32]
    lib.binattn_strerror.restype = ctypes.c_char_p
    lib.binattn_words.argtypes = [i32]
    lib.binattn_words.restype = i32
    lib.binattn_vq_ld.argtypes = [i32]
    lib.binattn_vq_ld.restype = i64
    lib.binattn_pack_qk.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.binattn_pack_qk.restype = i32
    lib.binattn_quant_v.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.binattn_quant_v.restype = i32
    lib.binattn_vq_canonical.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.binattn_vq_canonical.restype = i32
    lib.binattn_forward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, vp, i32, vp]
    lib.binattn_forward.restype = i32
    lib.binattn_scores_i32.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    lib.binattn_scores_i32.restype = i32
    lib.binattn_qk_rowstats.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.binattn_qk_rowstats.restype = i32
    lib.binattn_prepare.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.binattn_prepare.restype = i32
    lib.binattn_attention_workspace.argtypes = [i32, i32, i32, i32]
    lib.binattn_attention_workspace.restype = i64
    lib.binattn_attention.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, vp, i32, vp,
                                      i64, vp]
    lib.binattn_attention.restype = i32
    lib.binattn_attention_one_kernel.argtypes = [i32] * 9
    lib.binattn_attention_one_kernel.restype = i32
    lib.binattn_attention_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, vp,
                                              i32, vp]
    lib.binattn_attention_noalloc.restype = i32
    lib.binattn_backward_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.binattn_backward_workspace.restype = i64
    lib.binattn_backward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_float, vp, vp, vp, vp, vp, i64, vp]
    lib.binattn_backward.restype = i32
    lib.binattn_keep_plan.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_int)]
    lib.binattn_keep_plan.restype = i32
    lib.binattn_qkv_pack.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.binattn_qkv_pack.restype = i32
    return lib


_lib = _load()
EXPORTS = ["binattn_abi_version", "binattn_strerror", "binattn_words", "binattn_vq_ld", "binattn_pack_qk",
           "binattn_quant_v", "binattn_vq_canonical", "binattn_forward", "binattn_scores_i32", "binattn_qk_rowstats",
           "binattn_prepare", "binattn_attention_workspace", "binattn_attention", "binattn_attention_one_kernel",
           "binattn_keep_plan", "binattn_attention_noalloc", "binattn_backward_workspace", "binattn_backward",
           "binattn_qkv_pack"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # BINATTN_NOALLOC_SCRATCH_BYTES
QK_MFMA, QK_POPCOUNT = 0, 1


def lib():
    return _lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtypes, device=None):
    """Marshalling check: t is a dense (contiguous) device tensor of the given shape and dtype.
    The library reads raw pointers as dense row-major storage, so a strided view (for example a
    permuted qkv projection) would be read as the wrong elements: it is refused here instead."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on {device or 'a cuda device'} (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {[str(x) for x in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (call .contiguous() on strided views)")


_FLOATS = (torch.float16, torch.float32)


def _need_qkv(*xs, names=("q", "k", "v")):
    """q, k, v: 4-D [B,H,N,d], contiguous, one dtype (fp16 or fp32), one device."""
    x0 = xs[0]
    if not isinstance(x0, torch.Tensor) or x0.dim() != 4:
        raise ValueError(f"{names[0]} must be a 4-D tensor [B,H,N,d]")
    for x, n in zip(xs, names):
        _need(x, n, x0.shape, (x0.dtype,) if x0.dtype in _FLOATS else _FLOATS, x0.device)
    return x0.shape


def _need_bias(bias, bias_kind, grid, H, N, device):
    """Bias marshalling: None for BIAS_NONE; dense [H,N,ld] with ld >= N; table [H,(2gh-1)(2gw-1)]."""
    if bias_kind == BIAS_NONE:
        if bias is not None:
            raise ValueError("bias given with bias_kind BIAS_NONE")
        return
    if bias is None:
        raise ValueError("bias_kind needs a bias tensor")
    if bias_kind == BIAS_DENSE:
        if bias.dim() != 3 or bias.shape[0] != H or bias.shape[1] != N or bias.shape[2] < N:
            raise ValueError(f"dense bias must be [H={H}, N={N}, ld>=N], got {tuple(bias.shape)}")
        _need(bias, "bias", bias.shape, _FLOATS, device)
    elif bias_kind == BIAS_RELPOS:
        if grid is None or len(grid) != 2:
            raise ValueError("relative-position bias needs grid=(gh, gw)")
        gh, gw = grid
        _need(bias, "bias", (H, (2 * gh - 1) * (2 * gw - 1)), _FLOATS, device)
    else:
        raise ValueError(f"unknown bias_kind {bias_kind}")


def _need_packed(q_bits, q_mu, k_bits, k_mu, vq, vamax, d):
    """Packed forward inputs: bits [B,H,N,W] int32, mu [B,H,N] fp32, vq [B,H,d,ldv] int8, vamax [B,H,d]."""
    if not isinstance(q_bits, torch.Tensor) or q_bits.dim() != 4:
        raise ValueError("q_bits must be a 4-D tensor [B,H,N,W]")
    B, H, N, _ = q_bits.shape
    dev = q_bits.device
    _need(q_bits, "q_bits", (B, H, N, words(d)), (torch.int32,), dev)
    _need(k_bits, "k_bits", (B, H, N, words(d)), (torch.int32,), dev)
    _need(q_mu, "q_mu", (B, H, N), (torch.float32,), dev)
    _need(k_mu, "k_mu", (B, H, N), (torch.float32,), dev)
    _need(vq, "vq", (B, H, d, vq_ld(N)), (torch.int8,), dev)
    _need(vamax, "vamax", (B, H, d), (torch.float32,), dev)
    return B, H, N, dev


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise BinAttnError(fn, rc)


def words(d: int) -> int:
    return _lib.binattn_words(d)


def vq_ld(N: int) -> int:
    return _lib.binattn_vq_ld(N)


def vq_token_major(vq: torch.Tensor, N: int) -> torch.Tensor:
    """The canonical [B,H,N,d] view of a quantised V in the library's channel-major layout
    [B,H,d,ldv] (keys past N dropped): a strided view, no copy and no arithmetic."""
    return vq[..., :N].transpose(2, 3)


def pack_qk(x: torch.Tensor, bits=None, mu=None):
    """x [B,H,N,d] (fp16/fp32, cuda, contiguous) -> (bits uint32-as-int32 [B,H,N,W], mu fp32 [B,H,N])."""
    B, H, N, d = _need_qkv(x, names=("x",))
    if bits is None:
        bits = torch.empty((B, H, N, words(d)), dtype=torch.int32, device=x.device)
    if mu is None:
        mu = torch.empty((B, H, N), dtype=torch.float32, device=x.device)
    _need(bits, "bits", (B, H, N, words(d)), (torch.int32,), x.device)
    _need(mu, "mu", (B, H, N), (torch.float32,), x.device)
    _check("binattn_pack_qk", _lib.binattn_pack_qk(_p(x), _dt(x), B, H, N, d, _p(bits), _p(mu), _stream()))
    return bits, mu


def qkv_pack(x: torch.Tensor, w: torch.Tensor, bias, H: int, d: int, with_qk: bool = False):
    """The QKV projection with Q and K binarised in its epilogue.

    x [B,N,H d] fp16, w [3 H d, H d] fp16 (a linear layer's weight), bias [3 H d] fp16 or None
    -> (q_bits, q_mu, k_bits, k_mu, v [B,H,N,d] fp16), plus (q, k) fp16 [B,H,N,d] with_qk."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a 3-D tensor [B,N,C]")
    B, N, C = x.shape
    if C != H * d:
        raise ValueError(f"x has {C} features, expected H*d = {H * d}")
    _need(x, "x", (B, N, C), (torch.float16,))
    _need(w, "w", (3 * C, C), (torch.float16,), x.device)
    if bias is not None:
        _need(bias, "bias", (3 * C,), (torch.float16,), x.device)
    dev, W = x.device, words(d)
    qb = torch.empty((B, H, N, W), dtype=torch.int32, device=dev)
    kb = torch.empty((B, H, N, W), dtype=torch.int32, device=dev)
    qm = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    km = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    v = torch.empty((B, H, N, d), dtype=torch.float16, device=dev)
    q = torch.empty((B, H, N, d), dtype=torch.float16, device=dev) if with_qk else None
    k = torch.empty((B, H, N, d), dtype=torch.float16, device=dev) if with_qk else None
    _check("binattn_qkv_pack", _lib.binattn_qkv_pack(_p(x), _p(w), _p(bias), B, N, H, d, _p(qb), _p(qm), _p(kb),
                                                     _p(km), _p(v), _p(q), _p(k), _stream()))
    return (qb, qm, kb, km, v, q, k) if with_qk else (qb, qm, kb, km, v)


def quant_v(v: torch.Tensor, vq=None, vamax=None):
    """v [B,H,N,d] -> (vq int8 [B,H,d,ldv] channel-major, vamax fp32 [B,H,d] channel absmax).

    The dequantisation scale of channel c is vamax[..., c] / 127 (fp32 division)."""
    B, H, N, d = _need_qkv(v, names=("v",))
    if vq is None:
        vq = torch.empty((B, H, d, vq_ld(N)), dtype=torch.int8, device=v.device)
    if vamax is None:
        vamax = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    _need(vq, "vq", (B, H, d, vq_ld(N)), (torch.int8,), v.device)
    _need(vamax, "vamax", (B, H, d), (torch.float32,), v.device)
    _check("binattn_quant_v", _lib.binattn_quant_v(_p(v), _dt(v), B, H, N, d, _p(vq), _p(vamax), _stream()))
    return vq, vamax


def vq_canonical(vq: torch.Tensor, N: int, out=None) -> torch.Tensor:
    """vq int8 [B,H,d,ldv] (channel-major, as quant_v writes it) -> int8 [B,H,N,d] token-major,
    rearranged by the library's kernel (binattn_vq_canonical)."""
    if vq.dim() != 4:
        raise ValueError(f"vq must be 4-D [B,H,d,ldv], got {tuple(vq.shape)}")
    B, H, d, _ = vq.shape
    _need(vq, "vq", (B, H, d, vq_ld(N)), (torch.int8,), vq.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.int8, device=vq.device)
    _need(out, "out", (B, H, N, d), (torch.int8,), vq.device)
    _check("binattn_vq_canonical", _lib.binattn_vq_canonical(_p(vq), B, H, N, d, _p(out), _stream()))
    return out


def aligned_dense_bias(bias: torch.Tensor) -> torch.Tensor:
    """Copy a dense bias [H,N,N] into a [H,N,ld] buffer whose rows are 16-byte aligned (layout marshalling)."""
    H, N, N2 = bias.shape
    per16 = 16 // bias.element_size()
    ld = (N + per16 - 1) // per16 * per16
    if ld == N and bias.is_contiguous():
        return bias
    out = torch.zeros((H, N, ld), dtype=bias.dtype, device=bias.device)
    out[:, :, :N] = bias
    return out


def forward(q_bits, q_mu, k_bits, k_mu, vq, vamax, d, bias=None, bias_kind=BIAS_NONE, grid=None,
            out_dtype=torch.float16, out=None):
    """BinaryAttention forward -> O [B,H,N,d].

    bias: None; dense [H,N,ld] (ld >= N, 16-byte rows; see aligned_dense_bias); or a
    relative-position table [H,(2gh-1)(2gw-1)] with grid=(gh, gw).
    """
    B, H, N, dev = _need_packed(q_bits, q_mu, k_bits, k_mu, vq, vamax, d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    _need(out, "out", (B, H, N, d), _FLOATS, dev)
    _need_bias(bias, bias_kind, grid, H, N, dev)
    bdt, ld, gh, gw = F16, 0, 0, 0
    if bias is not None:
        bdt = _dt(bias)
        if bias_kind == BIAS_DENSE:
            ld = bias.shape[-1]
        elif bias_kind == BIAS_RELPOS:
            gh, gw = grid
    rc = _lib.binattn_forward(_p(q_bits), _p(q_mu), _p(k_bits), _p(k_mu), _p(vq), _p(vamax), bias_kind, bdt,
                              _p(bias), ld, gh, gw, B, H, N, d, _p(out), _dt(out), _stream())
    _check("binattn_forward", rc)
    return out


def scores_i32(q_bits, k_bits, d, D=None):
    """Integer sign scores D [B,H,N,N] int32 through the forward kernel's QK tile code."""
    B, H, N, _ = q_bits.shape
    _need(q_bits, "q_bits", (B, H, N, words(d)), (torch.int32,))
    _need(k_bits, "k_bits", (B, H, N, words(d)), (torch.int32,), q_bits.device)
    if D is None:
        D = torch.empty((B, H, N, N), dtype=torch.int32, device=q_bits.device)
    _need(D, "D", (B, H, N, N), (torch.int32,), q_bits.device)
    _check("binattn_scores_i32", _lib.binattn_scores_i32(_p(q_bits), _p(k_bits), B, H, N, d, _p(D), _stream()))
    return D


def qk_rowstats(q_bits, k_bits, d, method=QK_MFMA, rowmax=None, rowsum=None):
    """Binary QK tile probe: (max_j D_ij, sum_j D_ij) per query row, fp32 [B,H,N] each."""
    B, H, N, _ = q_bits.shape
    _need(q_bits, "q_bits", (B, H, N, words(d)), (torch.int32,))
    _need(k_bits, "k_bits", (B, H, N, words(d)), (torch.int32,), q_bits.device)
    if rowmax is None:
        rowmax = torch.empty((B, H, N), dtype=torch.float32, device=q_bits.device)
    if rowsum is None:
        rowsum = torch.empty((B, H, N), dtype=torch.float32, device=q_bits.device)
    _check("binattn_qk_rowstats", _lib.binattn_qk_rowstats(_p(q_bits), _p(k_bits), B, H, N, d, method, _p(rowmax),
                                                           _p(rowsum), _stream()))
    return rowmax, rowsum


def prepare(q, k, v, qbits=None, qmu=None, kbits=None, kmu=None, vq=None, vamax=None):
    """The three input-side steps in one call: (q_bits, q_mu, k_bits, k_mu, vq, vamax)."""
    B, H, N, d = _need_qkv(q, k, v)
    dev = q.device
    if qbits is None:
        qbits = torch.empty((B, H, N, words(d)), dtype=torch.int32, device=dev)
        kbits = torch.empty_like(qbits)
        qmu = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        kmu = torch.empty_like(qmu)
        vq = torch.empty((B, H, d, vq_ld(N)), dtype=torch.int8, device=dev)
        vamax = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _need_packed(qbits, qmu, kbits, kmu, vq, vamax, d)
    _check("binattn_prepare", _lib.binattn_prepare(_p(q), _p(k), _p(v), _dt(q), B, H, N, d, _p(qbits), _p(qmu), _p(kbits), _p(kmu),
                                                   _p(vq), _p(vamax), _stream()))
    return qbits, qmu, kbits, kmu, vq, vamax


def attention_workspace(B, H, N, d, device):
    """Caller-owned workspace for attention() (uint8 tensor; torch allocations are 256-byte aligned)."""
    n = _lib.binattn_attention_workspace(B, H, N, d)
    if n < 0:
        raise BinAttnError("binattn_attention_workspace", -2)
    return torch.empty((n,), dtype=torch.uint8, device=device)


def keep_plan(nheads, nqb, slots, fused=False):
    """The head-resident forward's workgroup plan (a, f, b, r) (binattn_keep_plan; host only)."""
    out = (ctypes.c_int * 4)()
    _check("binattn_keep_plan", _lib.binattn_keep_plan(int(nheads), int(nqb), int(slots), int(bool(fused)), out))
    return tuple(out)


def attention_one_kernel(B, H, N, d, dtype, bias_kind=BIAS_NONE, bias_dtype=None, grid=None):
    """Whether attention() on these shapes runs as one kernel (True) or as prepare + forward."""
    gh, gw = grid if grid else (0, 0)
    bdt = F16 if bias_dtype is None else (F32 if bias_dtype == torch.float32 else F16)
    dt = F32 if dtype == torch.float32 else F16
    rc = _lib.binattn_attention_one_kernel(dt, bias_kind, bdt, gh, gw, B, H, N, d)
    if rc < 0:
        raise BinAttnError("binattn_attention_one_kernel", rc)
    return rc == 1


def attention(q, k, v, bias=None, bias_kind=BIAS_NONE, grid=None, out_dtype=None, out=None, workspace=None):
    """Whole BinaryAttention forward from q, k, v [B,H,N,d] (fp16/fp32) -> O [B,H,N,d]."""
    B, H, N, d = _need_qkv(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", (B, H, N, d), _FLOATS, q.device)
    if workspace is None:
        workspace = attention_workspace(B, H, N, d, q.device)
    _need(workspace, "workspace", (workspace.numel(),), (torch.uint8,), q.device)
    _need_bias(bias, bias_kind, grid, H, N, q.device)
    bdt, ld, gh, gw = F16, 0, 0, 0
    if bias is not None:
        bdt = _dt(bias)
        if bias_kind == BIAS_DENSE:
            ld = bias.shape[-1]
        elif bias_kind == BIAS_RELPOS:
            gh, gw = grid
    rc = _lib.binattn_attention(_p(q), _p(k), _p(v), _dt(q), bias_kind, bdt, _p(bias), ld, gh, gw, B, H, N, d, _p(out),
                                _dt(out), _p(workspace), workspace.numel(), _stream())
    _check("binattn_attention", rc)
    return out


def attention_noalloc(q, k, v, bias=None, bias_kind=BIAS_NONE, grid=None, out_dtype=None, out=None):
    """attention() without a workspace: the library's own per-device scratch holds the packed
    intermediates (binattn_attention_noalloc), so the call allocates nothing when `out` is given.
    Calls that overlap on one device share that scratch and must be ordered by the caller."""
    B, H, N, d = _need_qkv(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", (B, H, N, d), _FLOATS, q.device)
    _need_bias(bias, bias_kind, grid, H, N, q.device)
    bdt, ld, gh, gw = F16, 0, 0, 0
    if bias is not None:
        bdt = _dt(bias)
        if bias_kind == BIAS_DENSE:
            ld = bias.shape[-1]
        elif bias_kind == BIAS_RELPOS:
            gh, gw = grid
    rc = _lib.binattn_attention_noalloc(_p(q), _p(k), _p(v), _dt(q), bias_kind, bdt, _p(bias), ld, gh, gw, B, H, N, d,
                                        _p(out), _dt(out), _stream())
    _check("binattn_attention_noalloc", rc)
    return out


def backward(q, k, v, o, dout, bias=None, bias_kind=BIAS_NONE, grid=None, ste_clip=0.0, bias_grad=True,
             workspace=None):
    """Gradients of the quantisation-aware forward (binattn_backward): q, k, v [B,H,N,d] the forward's
    inputs, o its output and dout the loss gradient in it (both of one dtype) -> (dq, dk, dv fp32
    [B,H,N,d], dbias fp32 dense [H,N,N] or table [H,(2gh-1)(2gw-1)], or None)."""
    B, H, N, d = _need_qkv(q, k, v)
    _need_qkv(o, dout, names=("o", "dout"))
    if tuple(o.shape) != (B, H, N, d):
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {(B, H, N, d)}")
    _need_bias(bias, bias_kind, grid, H, N, q.device)
    dev = q.device
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    db = None
    bdt, ld, gh, gw = F16, 0, 0, 0
    if bias is not None:
        bdt = _dt(bias)
        if bias_kind == BIAS_DENSE:
            ld = bias.shape[-1]
            if bias_grad:
                db = torch.empty((H, N, N), dtype=torch.float32, device=dev)
        elif bias_kind == BIAS_RELPOS:
            gh, gw = grid
            if bias_grad:
                db = torch.empty((H, (2 * gh - 1) * (2 * gw - 1)), dtype=torch.float32, device=dev)
    n = _lib.binattn_backward_workspace(B, H, N, d, bias_kind)
    if n < 0:
        raise BinAttnError("binattn_backward_workspace", -2)
    if workspace is None:
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (workspace.numel(),), (torch.uint8,), dev)
    rc = _lib.binattn_backward(_p(q), _p(k), _p(v), _p(o), _p(dout), _dt(q), _dt(o), bias_kind, bdt, _p(bias), ld, gh,
                               gw, B, H, N, d, float(ste_clip), _p(dq), _p(dk), _p(dv), _p(db), _p(workspace),
                               workspace.numel(), _stream())
    _check("binattn_backward", rc)
    return dq, dk, dv, db
