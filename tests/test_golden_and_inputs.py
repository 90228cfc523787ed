"""Regression anchor for the oracle (tests/golden) and determinism of the seeded input recipe."""
import json
import os

import numpy as np
import pytest

import oracle
from diffusion_transformers_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_forward.json")


def test_oracle_matches_golden_fixture():
    g = json.load(open(GOLDEN))
    q, k, v, bias = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "bias"))
    d = q.shape[-1]
    qb, qmu = oracle.pack_qk(q)
    kb, kmu = oracle.pack_qk(k)
    np.testing.assert_array_equal(qb, np.array(g["q_bits"], dtype=np.uint32))
    np.testing.assert_array_equal(kb, np.array(g["k_bits"], dtype=np.uint32))
    np.testing.assert_array_equal(qmu, np.array(g["q_mu"], dtype=np.float32))
    np.testing.assert_array_equal(oracle.scores_i32(qb, kb, d), np.array(g["D"], dtype=np.int32))
    vq, s = oracle.quant_v(v)
    np.testing.assert_array_equal(vq, np.array(g["vq"], dtype=np.int8))
    np.testing.assert_array_equal(s, np.array(g["v_scale"], dtype=np.float32))
    out, m, l, ph = oracle.forward(q, k, v, bias, oracle.BIAS_DENSE, diagnostics=True)
    np.testing.assert_array_equal(ph, np.array(g["phat"], dtype=np.uint8))
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l, np.array(g["l"]), rtol=1e-13)


def test_workload_table_matches_named_shapes():
    names = [w.name for w in W.WORKLOADS]
    assert names == ["deit_t_toy", "deit_s_224", "deit_b_384", "dit_xl2_256", "highres_16k"]
    shapes = [(w.B, w.H, w.N, w.d) for w in W.WORKLOADS]
    assert shapes == [(1, 3, 197, 64), (64, 6, 197, 64), (32, 12, 577, 64), (64, 16, 256, 72), (2, 16, 16384, 64)]
    for w in W.WORKLOADS:
        if w.bias == "relpos":
            assert w.grid[0] * w.grid[1] == w.N


def test_inputs_are_deterministic_and_shaped():
    a = W.custom(2, 3, 37, 72, "f16", "relpos", grid=(1, 37), seed=4)
    b = W.custom(2, 3, 37, 72, "f16", "relpos", grid=(1, 37), seed=4)
    for key in ("q", "k", "v", "bias"):
        assert a[key].tobytes() == b[key].tobytes()
    assert a["q"].dtype == np.float16 and a["q"].shape == (2, 3, 37, 72)
    assert a["bias"].shape == (3, (2 * 1 - 1) * (2 * 37 - 1))
    c = W.custom(2, 3, 37, 72, "f16", "relpos", grid=(1, 37), seed=5)
    assert a["q"].tobytes() != c["q"].tobytes()


def test_toy_workload_is_fp32_with_dense_bias():
    x = W.make(W.WORKLOADS[0])
    assert x["q"].dtype == np.float32 and x["bias"].shape == (3, 197, 197)
    assert abs(float(np.std(x["bias"])) - 0.02) < 0.002


def test_outlier_channels_count():
    w = W.Workload("o", 2, 12, 9, 64, "f32", "none", outlier_frac=0.01)
    x = W.make(w, seed=3)
    rng = np.random.default_rng(3)
    base = rng.standard_normal((2, 12, 9, 64), dtype=np.float32)
    ratio = np.abs(x["q"]) / np.maximum(np.abs(base), 1e-30)
    scaled = np.isclose(ratio, 8.0).all(axis=(0, 2))
    assert int(scaled.sum()) == round(0.01 * 12 * 64) == 8


def test_bench_roofline_helpers():
    """bench.py's roofline bookkeeping (host arithmetic only): the forward kernel named per
    shape, the MFMA time of the effective ops at the fp4 and int8 peaks, and the algorithmic
    bytes of the DeiT-B/384 forward from packed inputs."""
    import bench
    names = {w.name: bench.forward_kernel(w) for w in W.WORKLOADS}
    assert names["deit_s_224"] == names["deit_b_384"] == names["dit_xl2_256"] == "binattn_fwd_keep_kernel"
    assert names["highres_16k"] == "binattn_fwd_stream_kernel"
    # 4 B H N^2 d effective ops: half at 10.1, half at 5.0 dense POPS -> 6.69 POPS overall
    ops = 4.0e15
    assert abs(bench.mfma_seconds(ops) - (2.0e15 / 10.1e15 + 2.0e15 / 5.0e15)) < 1e-15
    assert abs(ops / bench.mfma_seconds(ops) / 1e12 - 6688.7) < 0.1
    w = next(x for x in W.WORKLOADS if x.name == "deit_b_384")
    # sign words + mu of Q and K, V^ bytes, channel absmax, dense fp16 bias once, fp16 O
    B, H, N, d = w.B, w.H, w.N, w.d
    expect = 2 * B * H * N * 2 * 4 + 2 * B * H * N * 4 + B * H * N * d + 4 * B * H * d + H * N * N * 2 + B * H * N * d * 2
    assert abs(bench.fwd_bytes(w) - expect) <= 0.02 * expect
