"""CPU oracle for the BinaryAttention forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and this package imports nothing from the
product path: the two share no code.

The arithmetic lives in ``binattn_oracle.c`` (plain C, fp64, OpenMP), built with
gcc into ``liboracle.so`` beside this file.  This module only marshals numpy
arrays into it.  The method follows "BinaryAttention: One-bit QK-Attention for
Vision and Diffusion Transformers" (CVPR 2026), paper-notes page, section
"Method details", key designs 1-3; see the header of ``binattn_oracle.c``.

Parity pins: every function here is checked against something other than
itself in ``tests/test_oracle.py`` (brute force on tiny inputs, closed forms,
invariants, reduction to a library softmax attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "binattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

NO_PQUANT = 1  # use P~ itself instead of P^/255
NO_VQUANT = 2  # use v itself instead of s * V^
BIAS_NONE, BIAS_DENSE, BIAS_RELPOS = 0, 1, 2

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_words.argtypes = [i32]
    lib.oracle_words.restype = i32
    lib.oracle_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_pack_qk.argtypes = [vp, i64, i32, vp, vp]
    lib.oracle_quant_v.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.oracle_scores_i32.argtypes = [vp, vp, i64, i64, i32, vp]
    lib.oracle_scores_rows.argtypes = [vp, vp, i64, i64, i32, vp, i64, vp]
    lib.oracle_forward.argtypes = [vp, vp, vp, i32, vp, i32, i32, i64, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.oracle_forward.restype = i32
    lib.oracle_forward_rows.argtypes = [vp, vp, vp, i32, vp, i32, i32, i64, i64, i64, i32, i32, vp, i64, vp]
    lib.oracle_forward_rows.restype = i32
    lib.oracle_backward.argtypes = [vp, vp, vp, i32, vp, i32, i32, i64, i64, i64, i32, vp, ctypes.c_double, vp, vp, vp,
                                    vp]
    lib.oracle_backward.restype = i32
    lib.oracle_qkv_project.argtypes = [vp, vp, vp, i64, i32, i64, vp, vp]
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def words(d: int) -> int:
    return int(_load().oracle_words(d))


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def pack_qk(x):
    """Sign bits and per-token scale of x [..., d] -> (bits uint32 [..., W], mu fp32 [...])."""
    x = _f64(x)
    d = x.shape[-1]
    lead = x.shape[:-1]
    ntok = int(np.prod(lead)) if lead else 1
    bits = np.zeros(lead + (words(d),), dtype=np.uint32)
    mu = np.zeros(lead, dtype=np.float32)
    _load().oracle_pack_qk(_ptr(x), ntok, d, _ptr(bits), _ptr(mu))
    return bits, mu


def quant_v(v, with_amax: bool = False):
    """Channel-wise int8 V of v [B,H,N,d] -> (vq int8 [B,H,N,d], scale fp32 [B,H,d]).

    with_amax=True also returns the fp32 channel absmax a [B,H,d] (scale = a / 127)."""
    v = _f64(v)
    B, H, N, d = v.shape
    vq = np.zeros((B, H, N, d), dtype=np.int8)
    s = np.zeros((B, H, d), dtype=np.float32)
    a = np.zeros((B, H, d), dtype=np.float32)
    _load().oracle_quant_v(_ptr(v), B * H, N, d, _ptr(vq), _ptr(s), _ptr(a))
    return (vq, s, a) if with_amax else (vq, s)


def scores_i32(qbits, kbits, d: int):
    """Integer sign dot products D [B,H,N,N] from packed bits [B,H,N,W]."""
    qbits = np.ascontiguousarray(qbits, dtype=np.uint32)
    kbits = np.ascontiguousarray(kbits, dtype=np.uint32)
    B, H, N, _ = qbits.shape
    D = np.zeros((B, H, N, N), dtype=np.int32)
    _load().oracle_scores_i32(_ptr(qbits), _ptr(kbits), B * H, N, d, _ptr(D))
    return D


def scores_rows(qbits, kbits, d: int, rows):
    """Rows of D for selected flattened (b, h, i) indices -> [len(rows), N] int32."""
    qbits = np.ascontiguousarray(qbits, dtype=np.uint32)
    kbits = np.ascontiguousarray(kbits, dtype=np.uint32)
    B, H, N, _ = qbits.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    D = np.zeros((rows.size, N), dtype=np.int32)
    _load().oracle_scores_rows(_ptr(qbits), _ptr(kbits), B * H, N, d, _ptr(rows), rows.size, _ptr(D))
    return D


def _bias_args(bias, bias_kind, grid):
    if bias_kind == BIAS_NONE or bias is None:
        return BIAS_NONE, None, 0, 0
    b = _f64(bias)
    gh, gw = grid if grid is not None else (0, 0)
    return bias_kind, b, int(gh), int(gw)


def forward(q, k, v, bias=None, bias_kind=BIAS_NONE, grid=None, flags=0, diagnostics=False):
    """Full forward O [B,H,N,d] (fp64).

    bias: dense [H,N,N] (bias_kind=BIAS_DENSE) or relative-position table
    [H,(2gh-1)*(2gw-1)] (bias_kind=BIAS_RELPOS, grid=(gh, gw)).
    With diagnostics=True also returns (m, l, phat) with m, l [B,H,N] and
    phat uint8 [B,H,N,N].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    kind, b, gh, gw = _bias_args(bias, bias_kind, grid)
    out = np.zeros((B, H, N, d), dtype=np.float64)
    m = l = ph = None
    if diagnostics:
        m = np.zeros((B, H, N), dtype=np.float64)
        l = np.zeros((B, H, N), dtype=np.float64)
        ph = np.zeros((B, H, N, N), dtype=np.uint8)
    rc = _load().oracle_forward(_ptr(q), _ptr(k), _ptr(v), kind, _ptr(b), gh, gw, B, H, N, d, int(flags),
                                _ptr(out), _ptr(m), _ptr(l), _ptr(ph))
    if rc != 0:
        raise ValueError(f"oracle_forward failed with code {rc}")
    if diagnostics:
        return out, m, l, ph
    return out


def forward_rows(q, k, v, rows, bias=None, bias_kind=BIAS_NONE, grid=None, flags=0):
    """O for selected flattened (b, h, i) rows -> [len(rows), d] (fp64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    kind, b, gh, gw = _bias_args(bias, bias_kind, grid)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, d), dtype=np.float64)
    rc = _load().oracle_forward_rows(_ptr(q), _ptr(k), _ptr(v), kind, _ptr(b), gh, gw, B, H, N, d, int(flags),
                                     _ptr(rows), rows.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_forward_rows failed with code {rc}")
    return out


def backward(q, k, v, dout, bias=None, bias_kind=BIAS_NONE, grid=None, ste_clip=0.0, with_bias_grad=True):
    """Gradients of the quantisation-aware forward (straight-through sign; see binattn_oracle.c)
    for an output gradient dout [B,H,N,d] -> (dq, dk, dv [B,H,N,d], db) in fp64, with db the
    dense [H,N,N] or table [H,(2gh-1)(2gw-1)] bias gradient (None without a bias).
    ste_clip > 0 passes the sign's gradient only where |x| <= ste_clip."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    kind, b, gh, gw = _bias_args(bias, bias_kind, grid)
    dq, dk, dv = (np.zeros((B, H, N, d), dtype=np.float64) for _ in range(3))
    db = None
    if kind == BIAS_DENSE and with_bias_grad:
        db = np.zeros((H, N, N), dtype=np.float64)
    elif kind == BIAS_RELPOS and with_bias_grad:
        db = np.zeros((H, (2 * gh - 1) * (2 * gw - 1)), dtype=np.float64)
    rc = _load().oracle_backward(_ptr(q), _ptr(k), _ptr(v), kind, _ptr(b), gh, gw, B, H, N, d, _ptr(dout),
                                 float(ste_clip), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db))
    if rc != 0:
        raise ValueError(f"oracle_backward failed with code {rc}")
    return dq, dk, dv, db


def qkv_project(x, w, bias, H: int, d: int):
    """The QKV projection that produces the attention's inputs, in fp64.

    x [B,N,C] (C = H d), w [3C,C] (row o is output feature o), bias [3C] or None.  Output
    feature o = p C + h d + c is channel c of head h of part p (0: Q, 1: K, 2: V), the usual
    [3, H, d] order of a fused projection.  Returns q, k, v [B,H,N,d] and, in the same layout,
    mq, mk, mv: sum_i |x_i w_oi| + |bias_o|, the magnitude that bounds any summation order's
    rounding error."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    B, N, C = x.shape
    if C != H * d or w.shape != (3 * C, C) or (b is not None and b.shape != (3 * C,)):
        raise ValueError("shapes of x, w, bias do not match H, d")
    y = np.zeros((B * N, 3 * C), dtype=np.float64)
    mag = np.zeros((B * N, 3 * C), dtype=np.float64)
    _load().oracle_qkv_project(_ptr(x), _ptr(w), _ptr(b), B * N, C, 3 * C, _ptr(y), _ptr(mag))
    split = lambda a: np.ascontiguousarray(a.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4))
    ys, ms = split(y), split(mag)
    return ys[0], ys[1], ys[2], ms[0], ms[1], ms[2]
