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
    lib.binattn_keep_plan.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_int)]
    lib.binattn_keep_plan.restype = i32
    return lib


_lib = _load()
EXPORTS = ["binattn_abi_version", "binattn_strerror", "binattn_words", "binattn_vq_ld", "binattn_pack_qk",
           "binattn_quant_v", "binattn_forward", "binattn_scores_i32", "binattn_qk_rowstats",
           "binattn_prepare", "binattn_attention_workspace", "binattn_attention", "binattn_attention_one_kernel",
           "binattn_keep_plan"]
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
    B, H, N, d = x.shape
    if bits is None:
        bits = torch.empty((B, H, N, words(d)), dtype=torch.int32, device=x.device)
    if mu is None:
        mu = torch.empty((B, H, N), dtype=torch.float32, device=x.device)
    _check("binattn_pack_qk", _lib.binattn_pack_qk(_p(x), _dt(x), B, H, N, d, _p(bits), _p(mu), _stream()))
    return bits, mu


def quant_v(v: torch.Tensor, vq=None, vamax=None):
    """v [B,H,N,d] -> (vq int8 [B,H,d,ldv] channel-major, vamax fp32 [B,H,d] channel absmax).

    The dequantisation scale of channel c is vamax[..., c] / 127 (fp32 division)."""
    B, H, N, d = v.shape
    if vq is None:
        vq = torch.empty((B, H, d, vq_ld(N)), dtype=torch.int8, device=v.device)
    if vamax is None:
        vamax = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    _check("binattn_quant_v", _lib.binattn_quant_v(_p(v), _dt(v), B, H, N, d, _p(vq), _p(vamax), _stream()))
    return vq, vamax


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
    B, H, N, _ = q_bits.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_bits.device)
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
    if D is None:
        D = torch.empty((B, H, N, N), dtype=torch.int32, device=q_bits.device)
    _check("binattn_scores_i32", _lib.binattn_scores_i32(_p(q_bits), _p(k_bits), B, H, N, d, _p(D), _stream()))
    return D


def qk_rowstats(q_bits, k_bits, d, method=QK_MFMA, rowmax=None, rowsum=None):
    """Binary QK tile probe: (max_j D_ij, sum_j D_ij) per query row, fp32 [B,H,N] each."""
    B, H, N, _ = q_bits.shape
    if rowmax is None:
        rowmax = torch.empty((B, H, N), dtype=torch.float32, device=q_bits.device)
    if rowsum is None:
        rowsum = torch.empty((B, H, N), dtype=torch.float32, device=q_bits.device)
    _check("binattn_qk_rowstats", _lib.binattn_qk_rowstats(_p(q_bits), _p(k_bits), B, H, N, d, method, _p(rowmax),
                                                           _p(rowsum), _stream()))
    return rowmax, rowsum


def prepare(q, k, v, qbits=None, qmu=None, kbits=None, kmu=None, vq=None, vamax=None):
    """The three input-side steps in one call: (q_bits, q_mu, k_bits, k_mu, vq, vamax)."""
    B, H, N, d = q.shape
    dev = q.device
    if qbits is None:
        qbits = torch.empty((B, H, N, words(d)), dtype=torch.int32, device=dev)
        kbits = torch.empty_like(qbits)
        qmu = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        kmu = torch.empty_like(qmu)
        vq = torch.empty((B, H, d, vq_ld(N)), dtype=torch.int8, device=dev)
        vamax = torch.empty((B, H, d), dtype=torch.float32, device=dev)
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
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = attention_workspace(B, H, N, d, q.device)
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
