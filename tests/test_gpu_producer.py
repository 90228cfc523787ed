"""GPU parity of the QKV projection with Q/K binarised in its epilogue (binattn_qkv_pack
through the C ABI) against the oracle's projection followed by the oracle's packing
(key design 1 of the "BinaryAttention" paper notes, "Method details").

Tolerance, derived from the arithmetic: the GPU sums the C products in fp32 in its own order,
so its sum s differs from the oracle's fp64 y by at most eps = C * 2^-24 * mag (mag = sum of
|x_i w_i| + |bias|, from the oracle), and both are then rounded to fp16 once.  Hence
  fp16 values:   |gpu - fp16(y)| <= eps + one fp16 spacing at max(|y|, |y| + eps);
  sign bits:     equal wherever |y| > eps + 2^-24 (neither side can cross zero or round to a
                 signed zero there); elsewhere either bit is right;
  mu:            |gpu - ref| <= mean over channels of the fp16 bound above, plus d 2^-24 mu
                 for the fp32 sum of the d magnitudes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from diffusion_transformers_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _fp16_bound(y, mag, C):
    eps = C * 2.0 ** -24 * mag
    hi = np.abs(y) + eps
    sp = np.spacing(np.minimum(hi, 65504.0).astype(np.float16)).astype(np.float64)
    return eps, eps + sp


def _unpack(bits, d):
    b = np.ascontiguousarray(bits).view(np.uint32)
    as_bytes = b.view(np.uint8).reshape(b.shape[:-1] + (-1,))
    return np.unpackbits(as_bytes, axis=-1, bitorder="little")


def check_part(name, y, mag, C, d, bits=None, mu=None, vals=None, min_decided=0.99):
    """y, mag: oracle [..., d] fp64; bits [..., W] / mu [...] / vals [..., d] from the GPU."""
    eps, tol = _fp16_bound(y, mag, C)
    ref16 = y.astype(np.float16).astype(np.float64)
    if vals is not None:
        err = np.abs(vals.astype(np.float64) - ref16)
        assert np.all(err <= tol), (name, "values", float((err - tol).max()))
    if bits is not None:
        got = _unpack(bits, d)
        refb, _ = oracle.pack_qk(ref16)
        want = _unpack(refb, d)
        decided = np.abs(y) > eps + 2.0 ** -24
        assert np.all(got[..., d:] == 0), (name, "pad bits")
        assert np.array_equal(got[..., :d][decided], want[..., :d][decided]), (name, "sign bits")
        assert decided.mean() >= min_decided, (name, "too few decided signs", decided.mean())
        _, refmu = oracle.pack_qk(ref16)
        mub = tol.mean(axis=-1) + d * 2.0 ** -24 * refmu.astype(np.float64) + 1e-30
        err = np.abs(mu.astype(np.float64) - refmu.astype(np.float64))
        assert np.all(err <= mub), (name, "mu", float((err - mub).max()))


def run_case(B, N, H, d, bias, seed, with_qk=True):
    from diffusion_transformers_amd import binding as b
    inp = W.projection_inputs(B, N, H, d, bias=bias, seed=seed)
    x, w = _t(inp["x"]), _t(inp["w"])
    bt = None if inp["bias"] is None else _t(inp["bias"])
    out = b.qkv_pack(x, w, bt, H, d, with_qk=with_qk)
    torch.cuda.synchronize()
    qb, qm, kb, km, v = (t.cpu().numpy() for t in out[:5])
    rq, rk, rv, mq, mk, mv = oracle.qkv_project(inp["x"], inp["w"], inp["bias"], H, d)
    C = H * d
    check_part("v", rv, mv, C, d, vals=v)
    check_part("q", rq, mq, C, d, bits=qb, mu=qm, vals=out[5].cpu().numpy() if with_qk else None)
    check_part("k", rk, mk, C, d, bits=kb, mu=km, vals=out[6].cpu().numpy() if with_qk else None)
    return out


CASES = [
    # B, N, H, d, bias: one token; DeiT-S-like (two token tiles, ragged); a DiT-XL/2 slice;
    # d = 40 (three heads per tile, padded tile, k tail); d = 128 (one head per tile); d = 96;
    # d = 56; d = 24 (six heads per tile); H = 1, d = 8 (fewer sections than a tile holds)
    (1, 1, 1, 8, True),
    (2, 197, 6, 64, True),
    (1, 256, 16, 72, True),
    (1, 300, 3, 40, True),
    (2, 70, 2, 128, False),
    (1, 130, 5, 96, True),
    (3, 50, 4, 56, True),
    (1, 64, 12, 24, False),
    (1, 40, 1, 8, True),
    (1, 600, 8, 88, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])) + ("-bias" if c[4] else ""))
def test_qkv_pack_parity(case):
    B, N, H, d, bias = case
    _say(f"qkv_pack {case}")
    run_case(B, N, H, d, bias, seed=N + d)


def test_qkv_pack_matches_the_packing_entry_and_pipeline():
    """The epilogue's bits and mu are binattn_pack_qk's for the same fp16 Q and K (bit for bit),
    and the forward from the producer's outputs equals the forward from packing its fp16 Q and K
    separately (the same inputs give the same result)."""
    from diffusion_transformers_amd import binding as b
    B, N, H, d = 2, 256, 4, 72
    _say("qkv_pack vs pack_qk")
    qb, qm, kb, km, v, q, k = run_case(B, N, H, d, True, seed=3)
    qb2, qm2 = b.pack_qk(q)
    kb2, km2 = b.pack_qk(k)
    for x, y in ((qb, qb2), (qm, qm2), (kb, kb2), (km, km2)):
        assert torch.equal(x, y)
    vq, va = b.quant_v(v)
    o1 = b.forward(qb, qm, kb, km, vq, va, d)
    o2 = b.forward(qb2, qm2, kb2, km2, vq, va, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_qkv_pack_zero_weight_rows():
    """Weight rows of zeros with zero bias give y = +0: sign bit 1 (zero counts as +1), mu 0."""
    from diffusion_transformers_amd import binding as b
    B, N, H, d = 1, 70, 2, 32
    inp = W.projection_inputs(B, N, H, d, bias=True, seed=4)
    C = H * d
    w, bias = inp["w"].copy(), inp["bias"].copy()
    w[C:C + d] = 0  # every channel of K head 0
    bias[C:C + d] = 0
    w[5] = 0        # channel 5 of Q head 0
    bias[5] = 0
    qb, qm, kb, km, v = b.qkv_pack(_t(inp["x"]), _t(w), _t(bias), H, d)
    torch.cuda.synchronize()
    kbits = _unpack(kb.cpu().numpy(), d)
    assert np.all(kbits[:, 0, :, :d] == 1) and np.all(km.cpu().numpy()[:, 0] == 0)
    assert np.all(_unpack(qb.cpu().numpy(), d)[:, 0, :, 5] == 1)
    rq, rk, rv, mq, mk, mv = oracle.qkv_project(inp["x"], w, bias, H, d)
    # (the planted zeros are the undecided signs here; they are checked above)
    check_part("q", rq, mq, C, d, bits=qb.cpu().numpy(), mu=qm.cpu().numpy(), min_decided=0.0)
    check_part("k", rk, mk, C, d, bits=kb.cpu().numpy(), mu=km.cpu().numpy(), min_decided=0.0)


@pytest.mark.parametrize("name", ["deit_b_384", "dit_xl2_256", "highres_16k"])
def test_qkv_pack_full_size_sampled_tokens(name):
    """The projection at a workload's full size (all B N tokens in one launch); the oracle
    recomputes 384 sampled tokens (first and last included) and every head of each."""
    from diffusion_transformers_amd import binding as b
    wl = W.BY_NAME[name]
    B, N, H, d = wl.B, wl.N, wl.H, wl.d
    _say(f"qkv_pack full size {name}")
    inp = W.projection_inputs(B, N, H, d, bias=True, seed=7)
    out = b.qkv_pack(_t(inp["x"]), _t(inp["w"]), _t(inp["bias"]), H, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([[0, B * N - 1], rng.integers(0, B * N, 382)]))
    bi, ni = toks // N, toks % N
    xs = inp["x"].reshape(B * N, -1)[toks][None]
    rq, rk, rv, mq, mk, mv = oracle.qkv_project(xs, inp["w"], inp["bias"], H, d)  # [1,H,T,d]
    sel = lambda t: t.cpu().numpy()[bi, :, ni]                                      # [T,H,...]
    qb, qm, kb, km, v = (sel(t) for t in out)
    tr = lambda a: np.ascontiguousarray(np.swapaxes(a[0], 0, 1))                    # [T,H,d]
    C = H * d
    check_part("v", tr(rv), tr(mv), C, d, vals=v)
    check_part("q", tr(rq), tr(mq), C, d, bits=qb, mu=qm)
    check_part("k", tr(rk), tr(mk), C, d, bits=kb, mu=km)


@pytest.mark.parametrize("case", [(2, 256, 4, 72, "relpos", (16, 16)), (1, 197, 3, 64, "dense", ())],
                         ids=["dit-like-relpos", "deit-like-dense"])
def test_producer_pipeline_against_the_oracle_attention(case):
    """End to end: the producer's outputs through binattn_quant_v and binattn_forward give the
    oracle's attention of the oracle's projection (its fp16-rounded Q, K, V), to the forward's
    own bar: max |O - O_ref| <= 1e-2 max|V|, mean <= 1e-3 max|V|, relative Frobenius <= 5e-2."""
    from diffusion_transformers_amd import binding as b
    B, N, H, d, bias_kind, grid = case
    _say(f"producer pipeline {case}")
    inp = W.projection_inputs(B, N, H, d, bias=True, seed=11)
    rng = np.random.default_rng(12)
    if bias_kind == "relpos":
        gh, gw = grid
        table = (rng.standard_normal((H, (2 * gh - 1) * (2 * gw - 1))) * 0.02).astype(np.float16)
        bt, kind, okind = _t(table), b.BIAS_RELPOS, oracle.BIAS_RELPOS
        obias = table
    else:
        dense = (rng.standard_normal((H, N, N)) * 0.02).astype(np.float16)
        bt, kind, okind = b.aligned_dense_bias(_t(dense)), b.BIAS_DENSE, oracle.BIAS_DENSE
        obias = dense
    qb, qm, kb, km, v = b.qkv_pack(_t(inp["x"]), _t(inp["w"]), _t(inp["bias"]), H, d)
    vq, va = b.quant_v(v)
    o = b.forward(qb, qm, kb, km, vq, va, d, bt, kind, grid or None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, *_ = oracle.qkv_project(inp["x"], inp["w"], inp["bias"], H, d)
    f16 = lambda a: a.astype(np.float16).astype(np.float64)
    ref = oracle.forward(f16(rq), f16(rk), f16(rv), obias, okind, grid or None)
    vmax = float(np.abs(f16(rv)).max())
    err = np.abs(o.cpu().numpy().astype(np.float64) - ref)
    mx, mn = err.max() / vmax, err.mean() / vmax
    fro = np.linalg.norm(err) / np.linalg.norm(ref)
    _say(f"  O err: max {mx:.3e} mean {mn:.3e} relfro {fro:.3e} (x max|V|)")
    assert mx <= 1e-2 and mn <= 1e-3 and fro <= 5e-2, (mx, mn, fro)
