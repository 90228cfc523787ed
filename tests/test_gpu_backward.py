"""GPU parity of the backward (binattn_backward through the C ABI) against the oracle's backward
(key design 4: QAT with a straight-through sign; the readings are in both sources' headers).

Tolerance, derived from the arithmetic: the GPU works in fp32 (fp32 MFMA, fp32 exp) against the
oracle's fp64, takes Delta = dO . O from the forward's output O as given (an fp16 O carries a
relative rounding of 2^-11), and its P^ can sit one step from the oracle's where 255 exp(S - m) is
within fp32 rounding of a half-integer (one step is 1/255 of a weight).  Per tensor:
relative Frobenius error <= 1e-2 and max |error| <= 2e-2 max |reference|.
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


def _kind(bias):
    return {"none": oracle.BIAS_NONE, "dense": oracle.BIAS_DENSE, "relpos": oracle.BIAS_RELPOS}[bias]


def _cmp(name, got, ref, tag):
    err = np.abs(got.astype(np.float64) - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    _say(f"  {tag} {name}: max {err.max() / scale:.2e} relfro {fro:.2e}")
    assert np.all(np.isfinite(got)), name
    assert fro <= 1e-2 and err.max() <= 2e-2 * scale, (name, fro, err.max() / scale)


def run_case(B, H, N, d, dt, bias, grid, clip, gdt="f32", seed=0, tag=""):
    from diffusion_transformers_amd import binding as b
    inp = W.custom(B, H, N, d, dt, bias, grid, seed=seed)
    rng = np.random.default_rng(seed + 1)
    dout = rng.standard_normal((B, H, N, d)).astype(np.float32)
    q, k, v = _t(inp["q"]), _t(inp["k"]), _t(inp["v"])
    bt, kind = None, b.BIAS_NONE
    if bias == "dense":
        bt, kind = b.aligned_dense_bias(_t(inp["bias"])), b.BIAS_DENSE
    elif bias == "relpos":
        bt, kind = _t(inp["bias"]), b.BIAS_RELPOS
    gt = torch.float32 if gdt == "f32" else torch.float16
    o = b.attention(q, k, v, bt, kind, grid or None, out_dtype=gt)
    do = _t(dout).to(gt)
    dq, dk, dv, db = b.backward(q, k, v, o, do, bt, kind, grid or None, ste_clip=clip)
    torch.cuda.synchronize()
    rq, rk, rv, rb = oracle.backward(inp["q"], inp["k"], inp["v"], do.float().cpu().numpy(), inp["bias"], _kind(bias),
                                     grid or None, clip)
    _cmp("dq", dq.cpu().numpy(), rq, tag)
    _cmp("dk", dk.cpu().numpy(), rk, tag)
    _cmp("dv", dv.cpu().numpy(), rv, tag)
    if rb is not None:
        g = db.cpu().numpy()
        if bias == "dense":
            g = g[:, :, :N]
        _cmp("db", g, rb, tag)


CASES = [
    # B, H, N, d, dtype, bias, grid, clip
    (2, 2, 17, 64, "f16", "none", (), 0.0),
    (1, 2, 2, 32, "f16", "dense", (), 0.0),
    (1, 2, 64, 64, "f32", "dense", (), 0.0),
    (2, 1, 65, 72, "f16", "relpos", (5, 13), 0.0),
    (1, 2, 130, 8, "f16", "dense", (), 1.0),
    (2, 2, 197, 64, "f16", "dense", (), 0.0),
    (1, 2, 256, 72, "f16", "relpos", (16, 16), 0.0),
    (1, 1, 196, 64, "f32", "relpos", (14, 14), 0.5),
    (1, 1, 300, 128, "f16", "none", (), 0.0),
    (1, 2, 100, 40, "f32", "dense", (), 0.0),
    (1, 1, 577, 64, "f16", "dense", (), 0.0),
    # many key tiles for the row statistics (their next tile loaded during the current one) and
    # Delta from whole 16-byte chunks of dO and O, fp32 over d = 128
    (1, 2, 1100, 64, "f16", "dense", (), 0.0),
    (1, 1, 1500, 128, "f32", "none", (), 0.0),
    (1, 1, 1024, 64, "f16", "relpos", (8, 128), 0.0),
    # grid widths that are multiples of 16 take the diagonal sums of the table gradient: a table
    # larger than the kernel's LDS copy (31 x 255 entries: per-tile windows) and d = 32 (no room
    # for the diagonal scratch: per-key atomics)
    (1, 1, 2048, 64, "f16", "relpos", (16, 128), 0.0),
    (2, 1, 256, 32, "f16", "relpos", (16, 16), 0.0),
    (1, 2, 512, 96, "f32", "relpos", (16, 32), 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4]}-{c[5]}-clip{c[7]}")
def test_backward_parity(case):
    B, H, N, d, dt, bias, grid, clip = case
    _say(f"backward {case}")
    run_case(B, H, N, d, dt, bias, grid, clip, seed=N + d, tag=str(case[:4]))


def test_backward_fp16_output_and_gradient():
    """O and dO in fp16 (the forward's usual output): Delta takes the fp16 O as given."""
    _say("backward fp16 o/dout")
    run_case(2, 2, 197, 64, "f16", "dense", (), 0.0, gdt="f16", seed=9, tag="fp16 o")


def test_backward_model_shape_dit():
    """A DiT-XL/2-shaped slice (H=16, N=256 on the 16 x 16 latent grid, d=72, relative-position
    table) with B=4, every element against the oracle."""
    _say("backward dit slice")
    run_case(4, 16, 256, 72, "f16", "relpos", (16, 16), 0.0, seed=256, tag="dit")


def test_backward_without_bias_gradient_and_workspace_reuse():
    """dbias may be skipped (NULL); a second call through the same workspace gives the same
    dq, dk, dv bit for bit (no state is carried between calls)."""
    from diffusion_transformers_amd import binding as b
    inp = W.custom(1, 2, 150, 64, "f16", "dense", seed=3)
    q, k, v = _t(inp["q"]), _t(inp["k"]), _t(inp["v"])
    bt = b.aligned_dense_bias(_t(inp["bias"]))
    o = b.attention(q, k, v, bt, b.BIAS_DENSE, out_dtype=torch.float32)
    do = torch.randn(q.shape, dtype=torch.float32, device=DEV)
    ws = torch.empty((b.lib().binattn_backward_workspace(1, 2, 150, 64, b.BIAS_DENSE),), dtype=torch.uint8, device=DEV)
    r1 = b.backward(q, k, v, o, do, bt, b.BIAS_DENSE, bias_grad=False, workspace=ws)
    r2 = b.backward(q, k, v, o, do, bt, b.BIAS_DENSE, bias_grad=True, workspace=ws)
    torch.cuda.synchronize()
    assert r1[3] is None and r2[3] is not None
    for x, y in zip(r1[:3], r2[:3]):
        assert torch.equal(x, y)


def test_backward_single_key_closed_form():
    """N = 1: P = 1 and O = Vt_0, so dS = dO . Vt_0 - dO . O = 0 up to the rounding of the two dot
    products.  dP runs on the MFMA with dO s as two bf16 terms (2^-16 relative each) and Delta in
    fp32, so per row |dS| <= 2^-15 sum_c |dO_c| |Vt_c| <= 2^-15 d max|dO| max|V| =: e.  dq and dk
    are dS times mu_q mu_k / sqrt(d) (1 + at most one more such term) and stay below e for these
    inputs; the dense bias gradient sums dS over the B batch items: <= B e.  dv = dO (P^ = 255,
    l = 1): the dV operand dO / (255 l) enters the MFMA as two bf16 terms, exact to a relative
    2^-16 at worst, so dv matches dO to 2^-15."""
    from diffusion_transformers_amd import binding as b
    _say("backward N=1")
    B, H, N, d = 2, 3, 1, 64
    inp = W.custom(B, H, N, d, "f16", "dense", seed=1)
    q, k, v = _t(inp["q"]), _t(inp["k"]), _t(inp["v"])
    bt = b.aligned_dense_bias(_t(inp["bias"]))
    o = b.attention(q, k, v, bt, b.BIAS_DENSE, out_dtype=torch.float32)
    do = _t(np.random.default_rng(2).standard_normal(q.shape).astype(np.float32))
    dq, dk, dv, db = b.backward(q, k, v, o, do, bt, b.BIAS_DENSE)
    torch.cuda.synchronize()
    e = 2.0 ** -15 * d * float(do.abs().max()) * float(np.abs(inp["v"].astype(np.float64)).max())
    for name, x, bound in (("dq", dq, e), ("dk", dk, e), ("db", db[:, :, :1], B * e)):
        assert float(x.abs().max()) <= bound, (name, float(x.abs().max()), bound)
    torch.testing.assert_close(dv, do, rtol=2.0**-15, atol=1e-30)
