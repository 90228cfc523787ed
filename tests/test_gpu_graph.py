"""The hot path captured in a HIP graph (as bench.py replays it) gives the eager result on
every replay, with eager work and synchronisation between replays."""
import numpy as np
import pytest
import torch

from diffusion_transformers_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    from diffusion_transformers_amd import binding as b
    dev = "cuda:0"
    inp = W.custom(8, 6, 197, 64, "f16", "dense", seed=31)
    q, k, v = (torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v"))
    bias = b.aligned_dense_bias(torch.from_numpy(inp["bias"]).to(dev))
    qb, qm = b.pack_qk(q)
    kb, km = b.pack_qk(k)
    vq, vs = b.quant_v(v)
    out = torch.empty((8, 6, 197, 64), dtype=torch.float16, device=dev)

    def step():
        b.pack_qk(q, qb, qm)
        b.pack_qk(k, kb, km)
        b.quant_v(v, vq, vs)
        b.forward(qb, qm, kb, km, vq, vs, 64, bias, b.BIAS_DENSE, out=out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    refs = [t.clone() for t in (qb, qm, kb, km, vq, vs)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        for t in (qb, qm, kb, km, vq, vs):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from eager"
        for t, r in zip((qb, qm, kb, km, vq, vs), refs):
            assert torch.equal(t, r), f"replay {rep}: intermediate differs"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays


def test_graph_replays_split_quant_path():
    # long N takes the four-kernel V schedule; its zero-fill is a kernel, not a memset node
    from diffusion_transformers_amd import binding as b
    dev = "cuda:0"
    inp = W.custom(1, 2, 4096, 64, "f16", "none", seed=32)
    v = torch.from_numpy(inp["v"]).to(dev)
    vq, vs = b.quant_v(v)
    torch.cuda.synchronize()
    ref_q, ref_s = vq.clone(), vs.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.quant_v(v, vq, vs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        b.quant_v(v, vq, vs)
    for rep in range(4):
        vq.fill_(7)
        vs.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(vq, ref_q) and torch.equal(vs, ref_s), f"replay {rep}"


@pytest.mark.parametrize("name", ["deit_s_224", "dit_xl2_256"])
def test_graph_replays_attention(name):
    """binattn_attention (one preparation launch + forward) captured in a graph, as bench.py
    replays it: every replay equals the eager result."""
    from diffusion_transformers_amd import binding as b
    dev = "cuda:0"
    w = W.BY_NAME[name]
    inp = W.custom(4, w.H, w.N, w.d, w.dtype, w.bias, w.grid, seed=33)
    q, k, v = (torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v"))
    bias, kind, grid = None, b.BIAS_NONE, None
    if w.bias == "dense":
        bias, kind = b.aligned_dense_bias(torch.from_numpy(inp["bias"]).to(dev)), b.BIAS_DENSE
    elif w.bias == "relpos":
        bias, kind, grid = torch.from_numpy(inp["bias"]).to(dev), b.BIAS_RELPOS, w.grid
    ws = b.attention_workspace(4, w.H, w.N, w.d, dev)
    out = torch.empty((4, w.H, w.N, w.d), dtype=torch.float16, device=dev)

    def step():
        b.attention(q, k, v, bias, kind, grid, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from eager"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays
