"""Writes tests/golden/tiny_forward.json from the CPU oracle only.

The pages print no worked numeric example ("BinaryAttention" paper notes,
CVPR 2026, key designs 1-3 give the equations but no numbers), so this fixture
is a regression anchor for the oracle: a tiny seeded case with every
intermediate the method defines (sign words, mu, D, V^, s, O).  It is
regenerated only when the oracle's arithmetic changes for a reason the pages
give; its correctness is pinned separately by tests/test_oracle.py.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(2026)
    B, H, N, d = 1, 2, 5, 40
    q = rng.standard_normal((B, H, N, d)).astype(np.float16).astype(np.float64)
    k = rng.standard_normal((B, H, N, d)).astype(np.float16).astype(np.float64)
    v = rng.standard_normal((B, H, N, d)).astype(np.float16).astype(np.float64)
    bias = (0.02 * rng.standard_normal((H, N, N))).astype(np.float16).astype(np.float64)
    qb, qmu = oracle.pack_qk(q)
    kb, kmu = oracle.pack_qk(k)
    D = oracle.scores_i32(qb, kb, d)
    vq, s = oracle.quant_v(v)
    out, m, l, ph = oracle.forward(q, k, v, bias, oracle.BIAS_DENSE, diagnostics=True)
    doc = {
        "source": "BinaryAttention paper notes (CVPR 2026), Method details, key designs 1-3; values from the CPU oracle",
        "shape": [B, H, N, d],
        "q": q.tolist(), "k": k.tolist(), "v": v.tolist(), "bias": bias.tolist(),
        "q_bits": qb.astype(int).tolist(), "q_mu": qmu.astype(float).tolist(),
        "k_bits": kb.astype(int).tolist(), "k_mu": kmu.astype(float).tolist(),
        "D": D.astype(int).tolist(), "vq": vq.astype(int).tolist(), "v_scale": s.astype(float).tolist(),
        "phat": ph.astype(int).tolist(), "l": l.tolist(), "m": m.tolist(), "out": out.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_forward.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
