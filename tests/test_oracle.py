"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with an independent fact: a library
routine (numpy bit packing, a float matmul, torch's scaled-dot-product
attention), a closed form, an invariant, or brute force on tiny inputs.  Each
is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, a missing scale) makes one of them fail.

Method: "BinaryAttention: One-bit QK-Attention for Vision and Diffusion
Transformers" (CVPR 2026) paper notes, "Method details", key designs 1-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle

D_LIST = [1, 5, 31, 32, 33, 64, 72]


def _rand(shape, seed, zeros=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    if zeros:  # sprinkle +0.0 and -0.0: both have sign +1 (design reading of sign(0))
        mask = rng.random(shape) < 0.05
        x[mask] = 0.0
        neg = rng.random(shape) < 0.5
        x[mask & neg] = -0.0
    return x


def _signs_from_bits(bits, d):
    """+1/-1 matrix from packed words using numpy's own bit unpacking (little bit order)."""
    as_bytes = bits.view(np.uint8).reshape(bits.shape[:-1] + (-1,))
    b = np.unpackbits(as_bytes, axis=-1, bitorder="little")[..., :d]
    return 2.0 * b.astype(np.float64) - 1.0


# ---------------------------------------------------------------- key design 1: sign bits and mu

@pytest.mark.parametrize("d", D_LIST)
def test_pack_bits_match_numpy_packbits(d):
    x = _rand((3, 7, d), seed=d)
    bits, _ = oracle.pack_qk(x)
    W = (d + 31) // 32
    expect = np.packbits(~np.signbit(x) | (x == 0), axis=-1, bitorder="little")
    pad = np.zeros(x.shape[:-1] + (4 * W - expect.shape[-1],), dtype=np.uint8)
    expect_words = np.concatenate([expect, pad], axis=-1).view(np.uint32)
    assert bits.shape == x.shape[:-1] + (W,)
    np.testing.assert_array_equal(bits, expect_words)


def test_pack_special_cases():
    d = 72
    pos = np.ones((1, d))
    neg = -np.ones((1, d))
    bp, _ = oracle.pack_qk(pos)
    bn, _ = oracle.pack_qk(neg)
    assert list(bp[0]) == [0xFFFFFFFF, 0xFFFFFFFF, 0x000000FF]  # pad bits stay 0
    assert list(bn[0]) == [0, 0, 0]
    # -0.0 and +0.0 both count as the positive state
    z = np.array([[0.0, -0.0, -1e-300, 1e-300]])
    bz, _ = oracle.pack_qk(z)
    assert bz[0, 0] == 0b1011
    # LSB-first layout: a single negative channel c clears exactly bit c % 32 of word c // 32
    for c in [0, 1, 31, 32, 63, 64, 71]:
        x = np.ones((1, d))
        x[0, c] = -2.0
        b, _ = oracle.pack_qk(x)
        full = np.array([0xFFFFFFFF, 0xFFFFFFFF, 0xFF], dtype=np.uint64)
        full[c // 32] &= ~np.uint64(1 << (c % 32))
        np.testing.assert_array_equal(b[0].astype(np.uint64), full)


def test_mu_closed_forms():
    rng = np.random.default_rng(1)
    d = 64
    # constant magnitude c with random signs -> mu = c exactly
    for c in [0.0, 0.5, 3.0, 1024.0]:
        x = c * np.where(rng.random((5, d)) < 0.5, -1.0, 1.0)
        _, mu = oracle.pack_qk(x)
        np.testing.assert_array_equal(mu, np.float32(c))
    # scaling x by 2^k scales mu by 2^k exactly
    x = rng.standard_normal((9, d)).astype(np.float16).astype(np.float64)
    _, mu = oracle.pack_qk(x)
    for k in [-6, 3, 9]:
        _, mu2 = oracle.pack_qk(x * 2.0**k)
        np.testing.assert_array_equal(mu2, (mu.astype(np.float64) * 2.0**k).astype(np.float32))
    # against the library mean of |x|
    np.testing.assert_allclose(mu, np.mean(np.abs(x), axis=-1), rtol=2e-7)


# ---------------------------------------------------------------- key design 1: the integer score

@pytest.mark.parametrize("d", D_LIST)
def test_scores_equal_pm1_float_matmul(d):
    q = _rand((2, 3, 11, d), seed=100 + d)
    k = _rand((2, 3, 11, d), seed=200 + d)
    qb, _ = oracle.pack_qk(q)
    kb, _ = oracle.pack_qk(k)
    D = oracle.scores_i32(qb, kb, d)
    sq, sk = _signs_from_bits(qb, d), _signs_from_bits(kb, d)
    brute = np.einsum("bhic,bhjc->bhij", sq, sk)
    np.testing.assert_array_equal(D, brute.astype(np.int32))
    assert np.all(np.abs(D) <= d) and np.all((D - d) % 2 == 0)


@pytest.mark.parametrize("d,N", [(72, 37), (64, 65), (33, 16)])
def test_scores_rows_equal_pm1_float_matmul(d, N):
    """scores_rows (the selected-rows export used to check long launches) gives, for every
    requested flattened (b, h, i) row -- first and last head, first and last query, a ragged N --
    the row of the +-1 float product sigma(Q) sigma(K)^T, in the order requested, and the rows of
    scores_i32.  A row index outside [0, B*H*N) leaves its output row untouched."""
    B, H = 2, 3
    q = _rand((B, H, N, d), seed=300 + d)
    k = _rand((B, H, N, d), seed=400 + d)
    qb, _ = oracle.pack_qk(q)
    kb, _ = oracle.pack_qk(k)
    sq, sk = _signs_from_bits(qb, d), _signs_from_bits(kb, d)
    brute = np.einsum("bhic,bhjc->bhij", sq, sk).astype(np.int32).reshape(B * H * N, N)
    last = B * H * N - 1
    rows = np.array([last, 0, N - 1, N, (B * H - 1) * N, 5 * N + N // 2, last - 1], dtype=np.int64)
    got = oracle.scores_rows(qb, kb, d, rows)
    np.testing.assert_array_equal(got, brute[rows])
    np.testing.assert_array_equal(got, oracle.scores_i32(qb, kb, d).reshape(B * H * N, N)[rows])
    out = oracle.scores_rows(qb, kb, d, np.array([-1, last + 1, 3], dtype=np.int64))
    assert not out[:2].any()
    np.testing.assert_array_equal(out[2], brute[3])


def test_scores_special_cases():
    d = 72
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 1, 6, d))
    x[x == 0] = 1.0
    b, _ = oracle.pack_qk(x)
    bneg, _ = oracle.pack_qk(-x)
    D_self = oracle.scores_i32(b, b, d)
    assert np.all(np.diag(D_self[0, 0]) == d)
    D_anti = oracle.scores_i32(b, bneg, d)
    assert np.all(np.diag(D_anti[0, 0]) == -d)
    # one flipped channel changes D by exactly 2
    y = x.copy()
    y[0, 0, 0, 5] = -y[0, 0, 0, 5]
    by, _ = oracle.pack_qk(y)
    D = oracle.scores_i32(b, by, d)
    assert D[0, 0, 0, 0] == d - 2


# ---------------------------------------------------------------- key design 3: channel-wise int8 V

def test_quant_v_invariants():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((2, 3, 50, 72)).astype(np.float16).astype(np.float64)
    v[0, 1, :, 7] = 0.0  # an all-zero channel
    v[1, 2, :, 3] *= 8.0  # an outlier channel
    vq, s, a = oracle.quant_v(v, with_amax=True)
    assert vq.dtype == np.int8 and s.dtype == np.float32 and a.dtype == np.float32
    assert np.all(np.abs(vq.astype(int)) <= 127)
    amax = np.max(np.abs(v), axis=2)
    # the absmax output is the channel max of |v| (exact in fp32 for fp16 inputs)
    np.testing.assert_array_equal(a, amax.astype(np.float32))
    nz = amax > 0
    assert np.all(np.max(np.abs(vq.astype(int)), axis=2)[nz] == 127)
    assert np.all(s[~nz] == 0) and np.all(vq[0, 1, :, 7] == 0)
    # s = a / 127 to fp32 rounding
    np.testing.assert_allclose(s[nz], amax[nz] / 127.0, rtol=1e-7)
    # reconstruction error at most half a step, plus |V^| * |s - 1/inv| from the two fp32 roundings
    err = np.abs(vq * s[:, :, None, :].astype(np.float64) - v)
    assert np.all(err <= s[:, :, None, :] * (0.5 + 127 * 2.0**-22))


def test_quant_v_lossless_and_ties():
    rng = np.random.default_rng(6)
    V = rng.integers(-127, 128, size=(1, 2, 40, 16)).astype(np.float64)
    V[:, :, 0, :] = 127.0  # every channel reaches 127 -> scale exactly 1
    vq, s = oracle.quant_v(V)
    np.testing.assert_array_equal(s, 1.0)
    np.testing.assert_array_equal(vq, V.astype(np.int8))
    # round half to even on exact ties (scale 1 because max is 127)
    t = np.zeros((1, 1, 7, 1))
    t[0, 0, :, 0] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    vq, _ = oracle.quant_v(t)
    assert list(vq[0, 0, :, 0]) == [127, 2, 4, -2, -4, 0, 0]


# ---------------------------------------------------------------- key design 2 + softmax: reduction to library attention

def _dense_from_oracle_inputs(q, k):
    qb, qmu = oracle.pack_qk(q)
    kb, kmu = oracle.pack_qk(k)
    d = q.shape[-1]
    qs = _signs_from_bits(qb, d) * qmu[..., None].astype(np.float64)
    ks = _signs_from_bits(kb, d) * kmu[..., None].astype(np.float64)
    return qs, ks


@pytest.mark.parametrize("N,d", [(1, 8), (7, 64), (33, 72), (50, 5)])
def test_unquantised_forward_equals_sdpa(N, d):
    B, H = 2, 3
    rng = np.random.default_rng(N * 100 + d)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    bias = 0.3 * rng.standard_normal((H, N, N))
    out = oracle.forward(q, k, v, bias, oracle.BIAS_DENSE, flags=oracle.NO_PQUANT | oracle.NO_VQUANT)
    qs, ks = _dense_from_oracle_inputs(q, k)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qs), torch.from_numpy(ks), torch.from_numpy(v),
        attn_mask=torch.from_numpy(bias)[None].expand(B, H, N, N)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def _bias_probe(bias_kind, bias, N, grid=None):
    """Recover S - rowmax from the oracle when Q = K = 0 (mu = 0, so S = b) and V = I."""
    d = N
    z = np.zeros((1, 1, N, d))
    v = np.eye(N)[None, None]
    out = oracle.forward(z, z, v, bias, bias_kind, grid=grid, flags=oracle.NO_PQUANT | oracle.NO_VQUANT)
    logp = np.log(out[0, 0])
    return logp - logp.max(axis=1, keepdims=True)


def test_dense_bias_indexing():
    N, H = 6, 2
    bias = np.zeros((H, N, N))
    bias[0, 1, 4] = 2.0  # head 0 is what a (b=0, h=0) probe sees
    bias[1, 4, 1] = 5.0
    S = _bias_probe(oracle.BIAS_DENSE, bias, N)
    expect = np.zeros((N, N))
    expect[1, :] = -2.0
    expect[1, 4] = 0.0
    np.testing.assert_allclose(S, expect, atol=1e-12)


@pytest.mark.parametrize("dr,dc", [(0, 0), (1, 0), (0, 1), (-1, 2), (2, -3)])
def test_relpos_bias_indexing(dr, dc):
    gh, gw = 3, 4
    N = gh * gw
    table = np.zeros((1, (2 * gh - 1) * (2 * gw - 1)))
    table[0, (dr + gh - 1) * (2 * gw - 1) + (dc + gw - 1)] = 3.0
    S = _bias_probe(oracle.BIAS_RELPOS, table, N, grid=(gh, gw))
    # b_ij = 3 exactly when token i sits dr rows below and dc columns right of token j
    for i in range(N):
        for j in range(N):
            hit = (i // gw - j // gw == dr) and (i % gw - j % gw == dc)
            row_has_hit = any((i // gw - jj // gw == dr) and (i % gw - jj % gw == dc) for jj in range(N))
            want = 0.0 if (hit or not row_has_hit) else -3.0
            assert abs(S[i, j] - want) < 1e-12, (i, j, S[i, j], want)


# ---------------------------------------------------------------- closed forms of the quantised output

def _int_v(rng, B, H, N, d):
    V = rng.integers(-127, 128, size=(B, H, N, d)).astype(np.float64)
    V[:, :, 0, :] = 127.0  # lossless: scale 1, V^ = V
    return V


def test_identical_keys_give_column_mean():
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 2, 37, 16
    q = rng.standard_normal((B, H, N, d))
    k = np.repeat(rng.standard_normal((B, H, 1, d)), N, axis=2)
    V = _int_v(rng, B, H, N, d)
    out = oracle.forward(q, k, V)
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=2, keepdims=True), out.shape), rtol=1e-12)


def test_one_hot_bias_selects_a_value_row():
    rng = np.random.default_rng(9)
    B, H, N, d = 1, 1, 20, 8
    q, k = rng.standard_normal((2, B, H, N, d))
    V = _int_v(rng, B, H, N, d)
    bias = np.zeros((H, N, N))
    jstar = (np.arange(N) * 7 + 3) % N
    bias[0, np.arange(N), jstar] = 30.0
    out = oracle.forward(q, k, V, bias, oracle.BIAS_DENSE)
    np.testing.assert_allclose(out[0, 0], V[0, 0, jstar], rtol=1e-9, atol=1e-9)


def test_single_token():
    rng = np.random.default_rng(10)
    q, k, v = rng.standard_normal((3, 2, 3, 1, 24))
    out = oracle.forward(q, k, v)
    vq, s = oracle.quant_v(v)
    np.testing.assert_allclose(out, vq * s[:, :, None, :].astype(np.float64), rtol=1e-12)


def test_row_sum_is_unquantised():
    # P~ = e^-7 for the 99 non-selected keys rounds to P^ = 0, but still counts in l
    B, H, N, d = 1, 1, 100, 8
    rng = np.random.default_rng(11)
    V = _int_v(rng, B, H, N, d)
    z = np.zeros((B, H, N, d))
    bias = np.zeros((H, N, N))
    bias[0, :, 5] = 7.0
    out = oracle.forward(z, z, V, bias, oracle.BIAS_DENSE)
    l = 1.0 + (N - 1) * math.exp(-7.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(V[0, 0, 5] / l, (N, d)), rtol=1e-12)


def test_quantised_output_within_bound_of_float_attention():
    rng = np.random.default_rng(12)
    B, H, N, d = 2, 2, 97, 64
    q, k, v = rng.standard_normal((3, B, H, N, d))
    bias = 0.5 * rng.standard_normal((H, N, N))
    out, m, l, ph = oracle.forward(q, k, v, bias, oracle.BIAS_DENSE, diagnostics=True)
    flo = oracle.forward(q, k, v, bias, oracle.BIAS_DENSE, flags=oracle.NO_PQUANT | oracle.NO_VQUANT)
    vq, s = oracle.quant_v(v)
    vd = vq * s[:, :, None, :].astype(np.float64)
    # |P^/255 - P~| <= 0.5/255 and |V^ s - v| <= s/2
    bound = (0.5 / 255 * np.abs(vd).sum(axis=2, keepdims=True) + 0.5 * s[:, :, None, :] * l[..., None]) / l[..., None]
    assert np.all(np.abs(out - flo) <= bound * (1 + 1e-9))
    # the quantisers do move the result (the check can fail)
    assert np.max(np.abs(out - flo)) > 1e-4


def test_softmax_invariants():
    rng = np.random.default_rng(13)
    B, H, N, d = 2, 3, 61, 64
    q, k, v = rng.standard_normal((3, B, H, N, d))
    out, m, l, ph = oracle.forward(q, k, v, diagnostics=True)
    assert np.all(ph.max(axis=-1) == 255)          # the row max has P~ = 1
    assert np.all(l >= 1.0) and np.all(l <= N)     # P~ in (0, 1], max attained
    # row sums of the normalised weights P~/l are 1: P^/255 approximates P~ within half a step
    assert np.all(np.abs(ph.sum(axis=-1) / 255.0 - l) <= 0.5 / 255 * N + 1e-12)


def test_rows_match_full_forward():
    rng = np.random.default_rng(14)
    B, H, N, d = 2, 2, 40, 72
    q, k, v = rng.standard_normal((3, B, H, N, d))
    table = rng.standard_normal((H, (2 * 5 - 1) * (2 * 8 - 1)))
    full = oracle.forward(q, k, v, table, oracle.BIAS_RELPOS, grid=(5, 8))
    rows = np.array([0, 7, 39, 40, 111, B * H * N - 1])
    part = oracle.forward_rows(q, k, v, rows, table, oracle.BIAS_RELPOS, grid=(5, 8))
    np.testing.assert_array_equal(part, full.reshape(-1, d)[rows])


# ---- the QKV projection (the producer whose output key designs 1 and 3 take) ----

def test_qkv_project_equals_float_matmul_by_index():
    """Every q/k/v entry equals numpy's fp64 x @ w.T + bias at the feature o = p C + h d + c,
    looked up entry by entry (the [3, H, d] split and the [B,H,N,d] layout)."""
    B, N, H, d = 2, 5, 3, 8
    C = H * d
    rng = np.random.default_rng(11)
    x, w, bias = rng.standard_normal((B, N, C)), rng.standard_normal((3 * C, C)), rng.standard_normal(3 * C)
    q, k, v, mq, mk, mv = oracle.qkv_project(x, w, bias, H, d)
    y = x.reshape(B * N, C) @ w.T + bias
    a = np.abs(x.reshape(B * N, C))[:, None, :] * np.abs(w)[None, :, :]
    mag = a.sum(-1) + np.abs(bias)
    for p, (t, m) in enumerate(((q, mq), (k, mk), (v, mv))):
        assert t.shape == (B, H, N, d)
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    for c in range(d):
                        o = p * C + h * d + c
                        assert abs(t[b, h, n, c] - y[b * N + n, o]) <= 1e-12 * mag[b * N + n, o]
                        assert abs(m[b, h, n, c] - mag[b * N + n, o]) <= 1e-12 * mag[b * N + n, o]
                        assert abs(t[b, h, n, c]) <= m[b, h, n, c]


def test_qkv_project_selection_weights():
    """One-hot weight rows copy one input feature: output o of token (b, n) is x[b, n, pi(o)]
    exactly, plus the bias; with no bias it is the copy itself."""
    B, N, H, d = 2, 3, 2, 16
    C = H * d
    rng = np.random.default_rng(5)
    pi = rng.integers(0, C, 3 * C)
    w = np.zeros((3 * C, C))
    w[np.arange(3 * C), pi] = 1.0
    x = np.arange(B * N * C, dtype=np.float64).reshape(B, N, C) - 40.0
    q, k, v, *_ = oracle.qkv_project(x, w, None, H, d)
    bias = np.arange(3 * C, dtype=np.float64) * 0.5
    qb, kb, vb, *_ = oracle.qkv_project(x, w, bias, H, d)
    for p, (t, tb) in enumerate(((q, qb), (k, kb), (v, vb))):
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    for c in range(d):
                        o = p * C + h * d + c
                        assert t[b, h, n, c] == x[b, n, pi[o]]
                        assert tb[b, h, n, c] == x[b, n, pi[o]] + bias[o]


def test_qkv_project_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        oracle.qkv_project(np.zeros((1, 2, 12)), np.zeros((36, 12)), None, 2, 8)
    with pytest.raises(ValueError):
        oracle.qkv_project(np.zeros((1, 2, 16)), np.zeros((48, 16)), np.zeros(47), 2, 8)
