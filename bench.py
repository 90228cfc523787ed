"""Benchmark of the BinaryAttention forward hot path on one MI355X.

A step is one pass of the whole hot path over one batch: sign-pack Q and K, quantise V,
the forward -- binattn_attention through the C ABI, which runs either as one kernel
straight from fp16 Q, K, V (rows of at most 256 keys) or as the preparation launch
followed by the forward from packed inputs.  The default workload is the largest
single-GPU shape, the high-resolution 128x128 token grid (B=2, H=16, N=16384, d=64, fp16,
relative-position bias); ``--workload`` selects another named shape, and ``--targets``
names shapes measured the same way and reported beside it (default: DeiT-B 384^2 and
DiT-XL/2 256^2).  Inputs are seeded synthetic activations
(diffusion_transformers_amd/workloads.py) already resident in HBM; several input sets are
cycled so the 256 MB last-level cache does not hold the step's working set.

Prints ONE JSON line.  value = effective TOPS of the step, counting 2*B*H*N^2*d for QK^T
plus the same for PV.  Exactly --steps steps are timed after exactly --warmup untimed ones.
The roofline object is for the step's dominant kernel (the one kernel, or the forward from
packed inputs): algorithmic bytes (or effective ops) per launch over its average launch time
measured with HIP events on the launch stream, against the binding roofline of the two the
method names: HBM 8 TB/s, or the MFMA time of the ops at each half's own peak (QK^T on fp4
operands, dense 10.1 PFLOP/s; PV on int8, dense 5.0 POPS; together 6.69 POPS).
fwd_ms_per_call times the forward from packed inputs alone.  cpu_baseline times the CPU
oracle (whole hot path) on the host cores over a bounded sample.
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
    """sha256 (first 16 hex digits) over the sources the forward-path kernels are built from
    (every .hip and .h of csrc but the backward's and the producer's), in name order."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")) and name not in ("backward.hip", "project.hip"):
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
    """The oracle (whole hot path: pack, quantise, forward) on the host cores over a bounded
    sample of the workload: whole batch items when one fits the time budget, else a run of
    query rows (each row is one query's share of the forward, all keys), sized from a short
    trial so that the sample takes about `seconds` of wall time."""
    import numpy as np

    import oracle
    q, k, v = (np.ascontiguousarray(inp[n], dtype=np.float64) for n in ("q", "k", "v"))
    bias = None if inp["bias"] is None else np.ascontiguousarray(inp["bias"], dtype=np.float64)
    kind = {"none": oracle.BIAS_NONE, "dense": oracle.BIAS_DENSE, "relpos": oracle.BIAS_RELPOS}[w.bias]
    grid = w.grid or None
    per_item = w.H * w.N * w.N * (w.d + 8)
    if per_item <= 2e9:  # whole batch items, repeated until the budget is spent
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
        sample = (f"{reps} oracle pass(es) of the whole hot path (pack, quantise, forward) over "
                  f"{nb} of {w.B} batch items of {w.name}, {el:.1f} s wall")
    else:  # long rows: a run of query rows of the first head (every key), sized by a trial
        q1, k1, v1 = q[:1], k[:1], v[:1]

        def trial(n):
            t0 = time.perf_counter()
            oracle.forward_rows(q1, k1, v1, np.arange(n, dtype=np.int64), bias, kind, grid=grid)
            return time.perf_counter() - t0
        # two trials: the marginal cost of a row, apart from packing the batch item once per call
        n1, n2 = min(w.N, 128), min(w.N, 640)
        t1, t2 = trial(n1), trial(n2)
        per_row = max((t2 - t1) / max(n2 - n1, 1), 1e-9)
        nrows = int(max(64, min(w.H * w.N, (seconds - max(t1 - n1 * per_row, 0.0)) / per_row)))
        t0 = time.perf_counter()
        oracle.forward_rows(q1, k1, v1, np.arange(nrows, dtype=np.int64), bias, kind, grid=grid)
        el = time.perf_counter() - t0
        ops = 4.0 * nrows * w.N * w.d
        sample = (f"the whole hot path (pack and quantise batch item 0, then the forward) for {nrows} query "
                  f"rows of batch item 0 of {w.name} ({nrows / w.N:.2f} heads of {w.N} queries, every key), "
                  f"{el:.1f} s wall")
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": oracle.threads(), "kind": "oracle",
            "sample": sample}


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


def input_sets(w, W, b, dev, rotate):
    """Rotated input sets of workload w, resident in HBM: enough sets that together they hold
    about 768 MB (three times the 256 MB last-level cache), at least 2 and at most `rotate`."""
    import torch
    nset = max(1, min(rotate, max(2, -(-768_000_000 // int(step_bytes(w))))))
    sets = []
    for r in range(nset):
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
    return sets


def measure(w, W, b, dev, steps: int, warmup: int, rotate: int):
    """Times exactly `steps` steps of the whole hot path on workload w after exactly `warmup`
    untimed ones, cycling the rotated input sets (step i runs on set i mod nset), and the
    forward from packed inputs alone over as many launches.  Returns the timings, the roofline
    of the dominant kernel and the sets (the first keeps its host inputs)."""
    import torch
    sets = input_sets(w, W, b, dev, rotate)
    nset = len(sets)

    def step(s):
        # the whole hot path from fp16/fp32 Q, K, V: sign-pack Q and K, quantise V (one launch), forward
        b.attention(s["q"], s["k"], s["v"], s["bias"], s["kind"], s["grid"], out=s["o"], workspace=s["ws"])

    def fwd(s):
        b.forward(s["qb"], s["qm"], s["kb"], s["km"], s["vq"], s["vs"], w.d, s["bias"], s["kind"], s["grid"],
                  out=s["o"])

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

    class Cycle:
        """Exactly n launches of fn over the sets: whole cycles from one graph (one step per
        set), the remainder from one graph per set."""

        def __init__(self, fn, only_first=False):
            pick = (lambda i: sets[0]) if only_first else (lambda i: sets[i])
            self.whole = capture(lambda: [fn(pick(i)) for i in range(nset)])
            self.one = [capture(lambda i=i: fn(pick(i))) for i in range(nset)]

        def run(self, n):
            full, rest = divmod(n, nset)
            for _ in range(full):
                self.whole.replay()
            for i in range(rest):
                self.one[i].replay()

    def timed(fn, n):
        """HIP events on the current stream (the one the graphs replay on), bracketed by
        device synchronisation; milliseconds per launch."""
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        fn(n)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / max(n, 1)

    steps_c, fwd_c = Cycle(step), Cycle(fwd)
    steps_c.run(warmup)
    torch.cuda.synchronize()
    step_ms = timed(steps_c.run, steps)          # the timed region: exactly `steps` steps
    fwd_ms = timed(fwd_c.run, steps)             # the forward kernel alone, as many launches
    eager_ms = timed(lambda n: [step(sets[i % nset]) for i in range(n)], steps)  # host launches included
    warm_c = Cycle(step, only_first=True)        # every step on set 0: inputs warm in L2 / MALL
    warm_c.run(nset)
    warm_ms = timed(warm_c.run, steps)

    ops = w.ops()
    one = b.attention_one_kernel(w.B, w.H, w.N, w.d, sets[0]["q"].dtype, sets[0]["kind"],
                                 None if sets[0]["bias"] is None else sets[0]["bias"].dtype, sets[0]["grid"])
    if one:  # the step is one launch of the whole-attention kernel
        kernel, tag, kb, ks = ("binattn_fwd_keep_kernel (whole attention from fp16 Q, K, V)", "attention",
                               one_kernel_bytes(w), step_ms * 1e-3)
    else:    # the forward from packed inputs dominates the step
        kernel, tag, kb, ks = (f"{forward_kernel(w)} (forward from packed inputs)", "forward", fwd_bytes(w),
                               fwd_ms * 1e-3)
    roof = roofline(w, kb, ks)
    roof["traffic"] = stored_traffic(w.name, tag)
    roof["kernel"] = kernel
    return dict(sets=sets, nset=nset, one=one, step_ms=step_ms, fwd_ms=fwd_ms, eager_ms=eager_ms, warm_ms=warm_ms,
                roofline=roof)


def roofline(w, kbytes: float, ks: float):
    """Roofline of a kernel that moves `kbytes` algorithmic bytes and does w's effective ops in
    `ks` seconds: HBM-bound when the bytes take longer at 8 TB/s than the ops at the MFMA peaks."""
    ops = w.ops()
    t_mfma = mfma_seconds(ops)
    t_hbm = kbytes / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_mfma:
        achieved = kbytes / ks / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = ops / ks / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": ops / t_mfma / 1e12, "unit": "TOPS",
                "frac": t_mfma / ks}
    roof["algorithmic_bytes_per_launch"] = kbytes
    roof["launch_us"] = ks * 1e6
    roof["mfma_frac"] = t_mfma / ks
    roof["ops_frac_of_int8_peak"] = ops / ks / 1e12 / I8_PEAK_TOPS  # the metric's own yardstick (5 POPS for all ops)
    roof["hbm_frac"] = kbytes / ks / 1e9 / HBM_PEAK_GBS
    return roof


BF16_MFMA_PEAK_TFLOPS = 2500.0


def measure_backward(w, b, sets, calls: int):
    """The QAT backward (binattn_backward) on the first input set: dO of the forward's output drawn
    once, `calls` calls timed with HIP events after one warm call.  Its dense products (dP, dQ, dK,
    dV: 8 B H N^2 d useful flops) run on the bf16 MFMA (rounded operands as two bf16 terms, so up
    to twice the useful flops are issued), so they are set against its dense peak."""
    import torch
    s = sets[0]
    o = s["o"]
    dout = torch.randn(o.shape, dtype=o.dtype, device=o.device, generator=torch.Generator(o.device).manual_seed(7))
    ws = torch.empty((b.lib().binattn_backward_workspace(w.B, w.H, w.N, w.d, s["kind"]),), dtype=torch.uint8,
                     device=o.device)

    def call():
        return b.backward(s["q"], s["k"], s["v"], o, dout, s["bias"], s["kind"], s["grid"], workspace=ws)
    call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / calls
    flops = 8.0 * w.B * w.H * w.N * w.N * w.d
    return {"ms_per_call": ms, "calls": calls, "matmul_tflops": flops / (ms * 1e-3) / 1e12,
            "frac_of_bf16_mfma_peak": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "what": "dQ, dK, dV and the bias gradient from the forward's inputs, output and dO (straight-through "
                    "sign, P and V quantisers), fp32 outputs"}


FP16_MFMA_PEAK_TFLOPS = 2500.0


def measure_producer(w, W, b, dev, calls: int):
    """The producer of the attention's inputs (binattn_qkv_pack: the QKV projection with Q and K
    binarised in its epilogue) for workload w's shapes, on seeded projection inputs, against
    the unfused route a caller would otherwise take: the library GEMM (torch.addmm, hipBLASLt)
    writing Q, K, V in fp16, their permute to [B,H,N,d] and the separate packing pass."""
    import torch
    C = w.H * w.d
    inp = W.projection_inputs(w.B, w.N, w.H, w.d, bias=True, seed=7)
    x, wt, bias = (torch.from_numpy(inp[k]).to(dev) for k in ("x", "w", "bias"))
    x2 = x.reshape(w.B * w.N, C)

    def fused():
        b.qkv_pack(x, wt, bias, w.H, w.d)

    def gemm():
        torch.addmm(bias, x2, wt.t())

    def unfused():
        y = torch.addmm(bias, x2, wt.t()).reshape(w.B, w.N, 3, w.H, w.d).permute(2, 0, 3, 1, 4).contiguous()
        b.prepare(y[0], y[1], y[2])

    def timed(f):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(calls):
            f()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / calls

    ms_f, ms_g, ms_u = timed(fused), timed(gemm), timed(unfused)
    flops = 2.0 * w.B * w.N * C * 3 * C
    tf = flops / (ms_f * 1e-3) / 1e12
    return {"ms_per_call": ms_f, "calls": calls, "tflops": tf, "frac_of_fp16_mfma_peak": tf / FP16_MFMA_PEAK_TFLOPS,
            "library_gemm_ms": ms_g, "library_gemm_tflops": flops / (ms_g * 1e-3) / 1e12,
            "unfused_ms": ms_u, "speedup_vs_unfused": ms_u / ms_f,
            "what": "x [B,N,H d] fp16 times w [3 H d, H d]^T plus bias -> Q and K sign words and mu, V fp16; "
                    "unfused: library GEMM + permute + the separate packing and V quantisation"}


def target_summary(w, m):
    """Per-workload record of a target shape (DeiT-B/384, DiT-XL/2): step and forward timings, effective
    TOPS and the roofline fractions recomputed from this run's own launch times."""
    ops = w.ops()
    fwd_s = m["fwd_ms"] * 1e-3
    fwd_roof = roofline(w, fwd_bytes(w), fwd_s)
    return {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "bias": w.bias, "path": "one kernel" if m["one"] else
            "prepare + forward", "rotated_input_sets": m["nset"], "ms_per_step": m["step_ms"],
            "step_tops": ops / (m["step_ms"] * 1e-3) / 1e12, "fwd_ms_per_call": m["fwd_ms"],
            "fwd_effective_tops": ops / fwd_s / 1e12, "fwd_hbm_frac": fwd_roof["hbm_frac"],
            "fwd_bound": fwd_roof["bound"], "fwd_frac": fwd_roof["frac"],
            "fwd_target_40pct_us": 0.4 ** -1 * max(fwd_bytes(w) / (HBM_PEAK_GBS * 1e9), mfma_seconds(ops)) * 1e6,
            "warm_ms_per_step": m["warm_ms"], "eager_ms_per_step": m["eager_ms"],
            "roofline": m["roofline"]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="highres_16k")
    ap.add_argument("--targets", default="deit_b_384,dit_xl2_256",
                    help="comma-separated workloads also measured and reported under 'targets' ('' for none)")
    ap.add_argument("--rotate", type=int, default=8, help="at most this many input sets cycled through the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the QAT backward timing of the target shapes")
    ap.add_argument("--no-producer", action="store_true",
                    help="skip the timing of the QKV projection with Q/K binarised in its epilogue")
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
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
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

    m = measure(w, W, b, dev, args.steps, args.warmup, args.rotate)
    inp0 = m["sets"][0]["inp"]
    del m["sets"]
    torch.cuda.empty_cache()
    targets = {}
    for name in [t for t in args.targets.split(",") if t and t != w.name]:
        tw = W.BY_NAME[name]
        tm = measure(tw, W, b, dev, args.steps, args.warmup, args.rotate)
        bw = None if args.no_backward else measure_backward(tw, b, tm["sets"], max(1, min(args.steps, 20)))
        del tm["sets"]
        torch.cuda.empty_cache()
        targets[name] = target_summary(tw, tm)
        targets[name]["backward"] = bw

    producer = None
    if not args.no_producer:
        producer = {name: measure_producer(W.BY_NAME[name], W, b, dev, max(1, min(args.steps, 20)))
                    for name in [w.name] + [t for t in args.targets.split(",") if t and t != w.name]}
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp0, w, args.cpu_seconds)

    ops = w.ops()
    step_ms, fwd_ms = m["step_ms"], m["fwd_ms"]
    res = {
        "metric": METRIC,
        "value": ops / (step_ms * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "input_dtype": w.dtype,
                   "bias": w.bias, "rotated_input_sets": m["nset"]},
        "path": "one kernel" if m["one"] else "prepare + forward",
        "fwd_ms_per_call": fwd_ms,
        "eager_ms_per_step": m["eager_ms"],
        "warm_ms_per_step": m["warm_ms"],
        "timing": "HIP events on the replay stream around exactly `steps` graph-replayed steps (step i on "
                  "rotated input set i mod sets) after exactly `warmup` untimed ones; fwd_ms_per_call: as many "
                  "forward launches alone; warm_ms_per_step: every step on the first set",
        "fwd_effective_tops": ops / (fwd_ms * 1e-3) / 1e12,
        "step_hbm_gbs": step_bytes(w) / (step_ms * 1e-3) / 1e9,
        "roofline": m["roofline"],
        "targets": targets,
        "producer": producer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
