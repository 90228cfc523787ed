"""Pins of the oracle's backward (the quantisation-aware training step of the pages' key design
4: QAT with a straight-through estimator for sign) against things other than itself.

The main pin is torch.autograd in float64 applied to an independently written forward in which
every quantiser is straight-through in the usual way -- the value is the quantised one, the
gradient that of the identity (x + (quant(x) - x).detach()) -- with mu = mean|x| differentiated
by autograd itself and the row max detached.  The oracle derives the same gradients by hand in
plain C; the two share no code.  Closed forms check the value-side formulas independently of
autograd (identical keys, a one-hot bias).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from diffusion_transformers_amd import workloads as W


def _binarize(x, clip):
    """mu * sign(x) whose sign passes the gradient straight through (times 1{|x| <= clip} when
    clip > 0); mu = mean |x| is left to autograd, its value stored as fp32 as the forward defines."""
    sign = torch.where(x >= 0, 1.0, -1.0).to(x.dtype)
    ste = torch.ones_like(x) if clip <= 0 else (x.abs() <= clip).to(x.dtype)
    sign_st = sign + (x * ste - (x * ste).detach())
    mu = x.abs().mean(-1, keepdim=True)
    mu = mu + (mu.to(torch.float32).to(mu.dtype) - mu).detach()
    return mu * sign_st


def _quant_v_values(v):
    """s_c * V^ per channel in fp32 exactly as the forward defines it (a = max|v| over tokens,
    s = fl32(a / 127), inv = fl32(127 / a), V^ = clamp(rint(fl32(v * inv)), +-127))."""
    v32 = v.detach().to(torch.float32)
    a = v32.abs().amax(-2, keepdim=True)
    inv = torch.where(a > 0, torch.tensor(127.0, dtype=torch.float32) / a, torch.zeros_like(a))
    vh = torch.clamp(torch.round(v32 * inv), -127, 127)
    s = torch.where(a > 0, a / torch.tensor(127.0, dtype=torch.float32), torch.zeros_like(a))
    return (s.to(torch.float64) * vh.to(torch.float64))


def _torch_forward(q, k, v, bias, kind, grid, clip):
    d = q.shape[-1]
    N = q.shape[-2]
    s, t = _binarize(q, clip), _binarize(k, clip)
    S = s @ t.transpose(-1, -2) / math.sqrt(d)
    if kind == oracle.BIAS_DENSE:
        S = S + bias
    elif kind == oracle.BIAS_RELPOS:
        gh, gw = grid
        n = torch.arange(N)
        r, c = n // gw, n % gw
        idx = (r[:, None] - r[None, :] + gh - 1) * (2 * gw - 1) + (c[:, None] - c[None, :] + gw - 1)
        S = S + bias[:, idx]
    m = S.max(-1, keepdim=True).values.detach()
    pt = torch.exp(S - m)
    l = pt.sum(-1, keepdim=True)
    a = pt + (torch.round(255.0 * pt) / 255.0 - pt).detach()  # P^/255, straight through
    vt = v + (_quant_v_values(v) - v).detach()                # s V^, straight through
    return (a @ vt) / l


def _autograd(inp, kind, grid, dout, clip):
    q, k, v = (torch.tensor(inp[n].astype(np.float64), requires_grad=True) for n in ("q", "k", "v"))
    bias = None
    if inp["bias"] is not None:
        bias = torch.tensor(inp["bias"].astype(np.float64), requires_grad=True)
    o = _torch_forward(q, k, v, bias, kind, grid, clip)
    (o * torch.tensor(dout)).sum().backward()
    return (q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), None if bias is None else bias.grad.numpy(),
            o.detach().numpy())


CASES = [
    # B, H, N, d, bias, grid, clip
    (2, 2, 17, 8, "dense", (), 0.0),
    (1, 2, 33, 33, "none", (), 0.0),
    (2, 1, 24, 64, "relpos", (4, 6), 0.0),
    (1, 3, 20, 72, "dense", (), 1.0),
    (2, 2, 30, 40, "relpos", (5, 6), 0.5),
    (1, 1, 1, 16, "dense", (), 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4]}-clip{c[6]}")
def test_backward_equals_autograd_of_the_straight_through_forward(case):
    B, H, N, d, bias, grid, clip = case
    inp = W.custom(B, H, N, d, "f32", bias, grid, seed=N * d + B)
    x = inp["q"].reshape(-1)
    x[::13] = 0.0  # exact zeros: sign +1 in the forward, sgn 0 in the gradient of |x|
    dout = np.random.default_rng(N + d).standard_normal((B, H, N, d))
    kind = {"none": oracle.BIAS_NONE, "dense": oracle.BIAS_DENSE, "relpos": oracle.BIAS_RELPOS}[bias]
    dq, dk, dv, db = oracle.backward(inp["q"], inp["k"], inp["v"], dout, inp["bias"], kind, grid or None, clip)
    gq, gk, gv, gb, o = _autograd(inp, kind, grid, dout, clip)
    # the autograd model's forward value is the oracle's forward
    np.testing.assert_allclose(o, oracle.forward(inp["q"], inp["k"], inp["v"], inp["bias"], kind, grid or None),
                               rtol=1e-12, atol=1e-13)
    for name, a, b in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12 * max(1.0, np.abs(b).max()), err_msg=name)
    if gb is None:
        assert db is None
    else:
        np.testing.assert_allclose(db, gb, rtol=1e-9, atol=1e-12 * max(1.0, np.abs(gb).max()), err_msg="db")


def test_backward_clip_zeroes_the_sign_path():
    """With a clip below every |q|, dq keeps only the mu path: sgn(q)/d times sum_e ds_e sign(q_e),
    the same value for every channel up to its sign."""
    inp = W.custom(1, 1, 9, 16, "f32", "none", seed=3)
    q = inp["q"]
    q[np.abs(q) < 0.05] = 0.05
    dout = np.random.default_rng(1).standard_normal(q.shape)
    dq, _, _, _ = oracle.backward(q, inp["k"], inp["v"], dout, ste_clip=1e-3)
    ratio = dq / np.sign(q)
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), rtol=1e-12, atol=1e-15)


def test_backward_identical_keys_closed_form():
    """All keys identical, no bias: every P~ = 1, P^ = 255, l = N, so dv_j = mean_i dO_i for every
    key j, and dS_ij = (dO_i . Vt_j - dO_i . O_i) / N with O_i = mean_j Vt_j: every dS_ij of a
    row is the same number, so dq (through the keys' t) is the row's dS times sum_j t_j."""
    B, H, N, d = 1, 2, 12, 16
    rng = np.random.default_rng(4)
    q = rng.standard_normal((B, H, N, d))
    k = np.repeat(rng.standard_normal((B, H, 1, d)), N, axis=2)
    v = rng.standard_normal((B, H, N, d))
    dout = rng.standard_normal((B, H, N, d))
    dq, dk, dv, _ = oracle.backward(q, k, v, dout)
    np.testing.assert_allclose(dv, np.broadcast_to(dout.mean(axis=2, keepdims=True), dv.shape), rtol=1e-12,
                               atol=1e-14)


def test_backward_one_hot_bias_routes_dv_to_the_chosen_key():
    """A +40 dense bias on key j*(i) makes P~ one-hot per row (P^ = 255 there, 0 elsewhere), so dv
    of key j collects exactly the dO of the rows that chose it, and the bias gradient is (to
    e^-40) zero: a one-hot softmax does not move."""
    B, H, N, d = 1, 1, 10, 8
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    jstar = (np.arange(N) * 3 + 1) % N
    bias = np.zeros((H, N, N))
    bias[:, np.arange(N), jstar] = 40.0
    dout = rng.standard_normal((B, H, N, d))
    _, _, dv, db = oracle.backward(q, k, v, dout, bias, oracle.BIAS_DENSE)
    exp = np.zeros_like(dv)
    for i, j in enumerate(jstar):
        exp[0, 0, j] += dout[0, 0, i]
    np.testing.assert_allclose(dv, exp, rtol=1e-12, atol=1e-12)
    assert np.abs(db).max() < 1e-12
