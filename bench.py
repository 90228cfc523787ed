"""Benchmark of the BinaryAttention forward hot path on one MI355X.

A step is one pass of the whole hot path over one batch: sign-pack Q and K, quantise V,
the forward -- binattn_attention through the C ABI, which runs either as one kernel
straight from fp16 Q, K, V (rows of at most 256 keys) or as the preparation launch
followed by the forward from packed inputs.  The default workload is DeiT-S 224^2
(B=64, H=6, N=197, d=64, fp16, dense per-head bias); ``--workload`` selects another named
shape.  Inputs are seeded synthetic activations (diffusion_transformers_amd/workloads.py)
already resident in HBM; ``--rotate`` input sets are cycled so the 256 MB last-level cache
does not hold the step's working set.

Prints ONE JSON line.  value = effective TOPS of the step, counting 2*B*H*N^2*d for QK^T
plus the same for PV.  The roofline object is for the step's dominant kernel (the one
kernel, or the forward from packed inputs): algorithmic bytes per launch over its average
launch time measured with HIP events on the launch stream, against the binding roofline of
the two the method names: HBM 8 TB/s, or the MFMA time of the ops at each half's own peak
(QK^T on fp4 operands, dense 10.1 PFLOP/s; PV on int8, dense 5.0 POPS; together 6.69 POPS).  fwd_ms_per_call times the
forward from packed inputs alone.  cpu_baseline times the CPU oracle (whole hot path) on
the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "binary-attention fwd ms/call & effective TOPS; % of int8 MFMA peak (1 GPU)"
HBM_PEAK_GBS = 8000.0
I8_PEAK_TOPS = 5000.0    # dense int8 MFMA (the PV product)
FP4_PEAK_TOPS = 10100.0  # dense fp4 MFMA (the QK^T tile's operands)
CSRC = os.path.join(ROOT, "diffusion_transformers_amd", "csrc")


def mfma_seconds(ops: float) -> float:
    """MFMA time of the effective ops at the dense peaks: half QK^T on fp4, half PV on int8."""
    return ops / 2 / (FP4_PEAK_TOPS * 1e12) + ops / 2 / (I8_PEAK_TOPS * 1e12)


def forward_kernel(w) -> str:
    """The forward kernel binattn_forward launches for this shape: head-resident for rows of
    <= 4 tiles, and of <= 10 tiles at d <= 64 without relative-position bias; else streaming."""
    ntiles, nt = -(-w.N // 64), -(-w.d // 16)
    keep = ntiles <= 4 or (ntiles <= 10 and nt <= 4 and w.bias != "relpos")
    return "binattn_fwd_keep_kernel" if keep else "binattn_fwd_stream_kernel"


def bias_bytes(w) -> float:
    """Bias bytes read once per launch: the dense [H,N,N] bias (shared over the batch) or the tables."""
    esz = 2 if w.dtype == "f16" else 4
    if w.bias == "dense":
        return float(w.H * w.N * w.N * esz)
    if w.bias == "relpos":
        gh, gw = w.grid
        return float(w.H * (2 * gh - 1) * (2 * gw - 1) * esz)
    return 0.0


def fwd_bytes(w) -> float:
    """Algorithmic HBM bytes of one forward launch: each input read once, O written once."""
    B, H, N, d = w.B, w.H, w.N, w.d
    W = (d + 31) // 32
    bits = 2 * B * H * N * W * 4            # Q and K sign words
    mu = 2 * B * H * N * 4                  # mu_q, mu_k
    vq = B * H * N * d                      # int8 V^
    vs = B * H * d * 4                      # V scales
    esz = 2 if w.dtype == "f16" else 4
    out = B * H * N * d * esz
    return float(bits + mu + vq + vs + out) + bias_bytes(w)


def one_kernel_bytes(w) -> float:
    """Algorithmic HBM bytes of the one-kernel step: Q, K, V read once, the bias once, O written once."""
    esz = 2 if w.dtype == "f16" else 4
    return float(4 * w.B * w.H * w.N * w.d * esz) + bias_bytes(w)


def step_bytes(w) -> float:
    """Algorithmic HBM bytes of a whole step (pack Q, pack K, quantise V, forward)."""
    B, H, N, d = w.B, w.H, w.N, w.d
    esz = 2 if w.dtype == "f16" else 4
    W = (d + 31) // 32
    pack = 2 * (B * H * N * d * esz + B * H * N * (4 * W + 4))
    quant = B * H * N * d * esz + B * H * N * d + B * H * d * 4  # V read once, V^ and the absmax written
    return float(pack + quant + fwd_bytes(w))


def sources_sha() -> str:
    """sha256 (first 16 hex digits) over the kernel sources, in name order."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel_tag: str):
    """HBM traffic per launch of the dominant kernel from the committed rocprofv3 PMC summary,
    or None when that summary was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("sources_sha256_16") != sources_sha() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(inp, w, seconds: float):
    import numpy as np

    import oracle
    q, k, v = (np.ascontiguousarray(inp[n], dtype=np.float64) for n in ("q", "k", "v"))
    bias = None if inp["bias"] is None else np.ascontiguousarray(inp["bias"], dtype=np.float64)
    kind = {"none": oracle.BIAS_NONE, "dense": oracle.BIAS_DENSE, "relpos": oracle.BIAS_RELPOS}[w.bias]
    grid = w.grid or None
    # bound the sample: whole batch when one oracle step is cheap, else a prefix of the batch
    per_item = w.H * w.N * w.N * (w.d + 8)
    nb = max(1, min(w.B, int(2e9 // max(per_item, 1))))
    qs, ks, vs = q[:nb], k[:nb], v[:nb]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(qs, ks, vs, bias, kind, grid=grid)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or el >= 30.0:
            break
    ops = 4.0 * nb * w.H * w.N * w.N * w.d * reps
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{reps} oracle pass(es) of the whole hot path (pack, quantise, forward) over "
                      f"{nb} of {w.B} batch items of {w.name}, {el:.1f} s wall"}


def qk_ab(w, W, b, dev, steps):
    """Time the QK-tile probe with each method on the workload's packed Q/K (same launch grid,
    same LDS staging of K, same per-row reduction; only the way D is computed differs)."""
    import torch
    inp = W.make(w, seed=W.WORKLOADS.index(w))
    qb, _ = b.pack_qk(torch.from_numpy(inp["q"]).to(dev))
    kb, _ = b.pack_qk(torch.from_numpy(inp["k"]).to(dev))
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "steps": steps}
    outs = {}
    for name, method in (("mfma", b.QK_MFMA), ("popcount", b.QK_POPCOUNT)):
        m, s = b.qk_rowstats(qb, kb, w.d, method)
        for _ in range(3):
            b.qk_rowstats(qb, kb, w.d, method, m, s)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            b.qk_rowstats(qb, kb, w.d, method, m, s)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / steps
        outs[name] = (m.clone(), s.clone())
        res[name + "_us"] = us
        res[name + "_tops_qk"] = 2.0 * w.B * w.H * w.N * w.N * w.d / (us * 1e-6) / 1e12
    res["identical"] = bool(torch.equal(outs["mfma"][0], outs["popcount"][0]) and
                            torch.equal(outs["mfma"][1], outs["popcount"][1]))
    res["popcount_over_mfma"] = res["popcount_us"] / res["mfma_us"]
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deit_s_224")
    ap.add_argument("--rotate", type=int, default=8, help="input sets cycled through the timed steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qk-ab", action="store_true",
                    help="only time the binary QK tile by its two methods (fp4 MFMA, VALU XOR+popcount) and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (PMC scaling reference) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: this build runs on one GPU only; --gpus above 1 is not supported "
                  "(the forward shards by (batch, head) with no communication; see the design notes).",
                  file=sys.stderr)
        sys.exit(2)

    import torch

    from diffusion_transformers_amd import binding as b
    from diffusion_transformers_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "dispatches": 5}))
        return

    w = W.BY_NAME[args.workload]
    if args.qk_ab:
        qk_ab(w, W, b, dev, max(1, args.steps))
        return
    sets = []
    for r in range(max(1, args.rotate)):
        inp = W.make(w, seed=W.WORKLOADS.index(w) + 1000 * r)
        q, k, v = (torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v"))
        bias, kind, grid = None, b.BIAS_NONE, None
        if w.bias == "dense":
            bias, kind = b.aligned_dense_bias(torch.from_numpy(inp["bias"]).to(dev)), b.BIAS_DENSE
        elif w.bias == "relpos":
            bias, kind, grid = torch.from_numpy(inp["bias"]).to(dev), b.BIAS_RELPOS, w.grid
        qb, qm, kb, km, vq, vs = b.prepare(q, k, v)
        out_dt = torch.float16 if w.dtype == "f16" else torch.float32
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=out_dt, device=dev)
        ws = b.attention_workspace(w.B, w.H, w.N, w.d, dev)
        sets.append(dict(inp=inp if r == 0 else None, q=q, k=k, v=v, bias=bias, kind=kind, grid=grid,
                         qb=qb, qm=qm, kb=kb, km=km, vq=vq, vs=vs, o=o, ws=ws))
    torch.cuda.synchronize()

    def step(s):
        # the whole hot path from fp16/fp32 Q, K, V: sign-pack Q and K, quantise V (one launch), forward
        b.attention(s["q"], s["k"], s["v"], s["bias"], s["kind"], s["grid"], out=s["o"], workspace=s["ws"])

    def capture(fn):
        """Capture fn() into a HIP graph on a side stream (default priority)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    nset = len(sets)
    # one graph holds one step per input set; K steps = K / nset replays
    reps = max(1, -(-args.steps // nset))
    steps = reps * nset
    step_graph = capture(lambda: [step(st) for st in sets])
    fwd_graph = capture(lambda: [b.forward(st["qb"], st["qm"], st["kb"], st["km"], st["vq"], st["vs"], w.d,
                                           st["bias"], st["kind"], st["grid"], out=st["o"]) for st in sets])

    for i in range(max(1, args.warmup // nset)):
        step_graph.replay()
    torch.cuda.synchronize()

    def timed(fn, n):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # timed region: exactly `steps` steps, bracketed by synchronisation
    step_ms = timed(step_graph.replay, reps) / steps
    # forward kernel alone: average launch duration over the same number of launches
    fwd_ms = timed(fwd_graph.replay, reps) / steps
    # eager launches through the ABI (host launch cost included), for reference
    eager_ms = timed(lambda: [step(st) for st in sets], reps) / steps
    # cache-warm reference: the same number of steps, all on the first input set (its inputs stay
    # in the L2 / last-level cache), against the headline's rotated sets
    warm_graph = capture(lambda: [step(sets[0]) for _ in sets])
    warm_graph.replay()
    warm_ms = timed(warm_graph.replay, reps) / steps

    ops = w.ops()
    one = b.attention_one_kernel(w.B, w.H, w.N, w.d, sets[0]["q"].dtype, sets[0]["kind"],
                                 None if sets[0]["bias"] is None else sets[0]["bias"].dtype, sets[0]["grid"])
    if one:  # the step is one launch of the whole-attention kernel
        kernel, tag, kb, ks = ("binattn_fwd_keep_kernel (whole attention from fp16 Q, K, V)", "attention",
                               one_kernel_bytes(w), step_ms * 1e-3)
    else:    # the forward from packed inputs dominates the step
        kernel, tag, kb, ks = (f"{forward_kernel(w)} (forward from packed inputs)", "forward", fwd_bytes(w),
                               fwd_ms * 1e-3)
    t_mfma = mfma_seconds(ops)
    t_hbm = kb / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_mfma:
        achieved = kb / ks / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = ops / ks / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": ops / t_mfma / 1e12, "unit": "TOPS",
                "frac": t_mfma / ks}
    roof["traffic"] = stored_traffic(w.name, tag)
    roof["kernel"] = kernel
    roof["algorithmic_bytes_per_launch"] = kb
    roof["launch_us"] = ks * 1e6
    roof["mfma_frac"] = t_mfma / ks
    roof["ops_frac_of_int8_peak"] = ops / ks / 1e12 / I8_PEAK_TOPS  # the metric's own yardstick (5 POPS for all ops)
    roof["hbm_frac"] = kb / ks / 1e9 / HBM_PEAK_GBS
    fwd_s = fwd_ms * 1e-3

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sets[0]["inp"], w, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": ops / (step_ms * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(1, args.warmup // nset) * nset,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "input_dtype": w.dtype,
                   "bias": w.bias, "rotated_input_sets": len(sets)},
        "path": "one kernel" if one else "prepare + forward",
        "fwd_ms_per_call": fwd_ms,
        "eager_ms_per_step": eager_ms,
        "warm_ms_per_step": warm_ms,
        "timing": "HIP events around graph replays; one graph = one step per rotated input set "
                  "(warm_ms_per_step: every step on the first set)",
        "fwd_effective_tops": ops / fwd_s / 1e12,
        "step_hbm_gbs": step_bytes(w) / (step_ms * 1e-3) / 1e9,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
