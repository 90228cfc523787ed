"""binattn_attention_noalloc -- the entry point that allocates nothing -- against the workspace
entry point binattn_attention it is a variant of: equal outputs bit for bit, on two calls in a
row whose second input is smaller (the scratch keeps the first call's contents), across the
one-kernel path (no scratch), the two-launch path in one chunk, the two-launch path over several
chunks of batch items, and fp32 inputs.  Equality with binattn_attention carries its oracle parity;
one case is also checked against the oracle directly."""
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


def _inputs(B, H, N, d, dt, bias, grid, seed):
    from diffusion_transformers_amd import binding as b
    inp = W.custom(B, H, N, d, dt, bias, grid, seed=seed)
    q, k, v = (torch.from_numpy(inp[n]).to(DEV) for n in ("q", "k", "v"))
    bt, kind = None, b.BIAS_NONE
    if bias == "dense":
        bt, kind = b.aligned_dense_bias(torch.from_numpy(inp["bias"]).to(DEV)), b.BIAS_DENSE
    elif bias == "relpos":
        bt, kind = torch.from_numpy(inp["bias"]).to(DEV), b.BIAS_RELPOS
    return inp, q, k, v, bt, kind


def _both(case, seed):
    """(noalloc output, workspace-entry output, inputs) for one case; the noalloc output buffer is
    pre-filled with NaN so that an unwritten element shows."""
    from diffusion_transformers_amd import binding as b
    B, H, N, d, dt, bias, grid = case
    inp, q, k, v, bt, kind = _inputs(B, H, N, d, dt, bias, grid, seed)
    o = torch.full((B, H, N, d), float("nan"), dtype=q.dtype, device=DEV)
    b.attention_noalloc(q, k, v, bt, kind, grid or None, out=o)
    ref = b.attention(q, k, v, bt, kind, grid or None)
    torch.cuda.synchronize()
    return o, ref, inp


# pairs of cases run back to back: (first, second smaller)
PAIRS = [
    # two-launch path, several chunks (about 5.5 MB of packed inputs per batch item: 11 items a chunk),
    # then one chunk of a smaller shape
    ((16, 16, 4096, 64, "f16", "relpos", (64, 64)), (2, 4, 1000, 64, "f16", "dense", ())),
    # one kernel (no scratch), then a smaller one-kernel shape
    ((8, 16, 256, 72, "f16", "relpos", (16, 16)), (2, 6, 197, 64, "f16", "dense", ())),
    # two-launch path from fp32 inputs, then a smaller head-resident long row
    ((4, 8, 2048, 32, "f32", "none", ()), (1, 3, 577, 64, "f16", "dense", ())),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][:4]}-then-{p[1][:4]}")
def test_noalloc_equals_workspace_entry_point(pair):
    from diffusion_transformers_amd import binding as b
    for i, case in enumerate(pair):
        _say(f"noalloc call {i + 1}: {case}")
        o, ref, _ = _both(case, seed=17 + i)
        assert int((~torch.isfinite(o)).sum()) == 0, "unwritten output elements"
        assert torch.equal(o, ref), f"noalloc output differs from binattn_attention on {case}"
    B, H, N, d = pair[0][:4]
    nbytes = b.lib().binattn_attention_workspace(B, H, N, d)
    _say(f"  first case packed inputs {nbytes / 2**20:.1f} MiB against {b.NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB scratch")


def test_noalloc_against_the_oracle():
    """A two-launch shape with a ragged last tile, directly against the oracle."""
    case = (2, 3, 700, 64, "f16", "dense", ())
    _say(f"noalloc vs oracle {case}")
    o, ref, inp = _both(case, seed=5)
    assert torch.equal(o, ref)
    exp = oracle.forward(inp["q"], inp["k"], inp["v"], inp["bias"], oracle.BIAS_DENSE)
    vmax = float(np.abs(inp["v"].astype(np.float64)).max())
    err = np.abs(o.cpu().numpy().astype(np.float64) - exp)
    assert err.max() <= 1e-2 * vmax and err.mean() <= 1e-3 * vmax
    assert np.linalg.norm(err) <= 5e-2 * np.linalg.norm(exp)


def test_noalloc_rejects_a_batch_item_beyond_the_scratch():
    """One batch item whose packed inputs exceed the scratch is refused before any launch."""
    from diffusion_transformers_amd import binding as b
    H, N, d = 64, 8192, 128  # one item: 64 heads x 8192 tokens x 128 channels of V^ alone is 64 MiB
    assert b.lib().binattn_attention_workspace(1, H, N, d) > b.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, H, N, d), dtype=torch.float16, device=DEV)
    with pytest.raises(b.BinAttnError, match="EUNSUPPORTED"):
        b.attention_noalloc(q, q, q)
