"""Benchmark of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload configs|all|NAME]

A step is one call of the forward (``fa_fwd``; ``fa_fwd_splitkv`` for the
decode workload; ``fa_fwd_paged_decode`` for the paged-cache decode) over one
batch of seeded synthetic inputs already resident in device memory.  By
default (``--launch graph``) W untimed warm-up steps run first, then the K
steps are captured once into a HIP graph and replayed: untimed for
``--prewarm-s`` seconds (0.3 by default; the GPU's clock ramps up over the
first tens of milliseconds of load after idle), then one replay between two
``torch.cuda.synchronize()`` calls is the timed region, and the events around
it on the kernels' stream give the per-launch kernel time used for the
roofline fraction.  Replaying a graph keeps the host's per-call cost out of
the timed region, which matters for kernels of a few microseconds.
``--launch eager`` calls the K steps one by one instead (pre-warm steps,
W warm-up steps, K timed steps, then K steps between per-step events).

By default (``--workload configs``) the five configurations are timed in
turn, one JSON line each: single-head fp32, ragged causal fp16, long
non-causal bf16, single-token decode, and last the causal bf16 prefill
B=8, H=16, N=4096, d=128, so that the final line is the headline.
``--workload all`` adds the backward, FP8, paged-decode and variable-length
workloads before the headline.  ``--workload gemm_bf16_n8192`` times a
plain bf16 GEMM by the vendor library instead, the practical matrix-core
rate at the clock the power limit allows.  FLOPs follow the convention 4*B*H*Nq*Nk*d
(the two contractions), halved under the causal mask; bytes are one read of
Q, K, V and one write of O and LSE.

The ``cpu_baseline`` leg times the fp64 oracle (test infrastructure) on a
bounded sample of the same workload on the host cores, then compares the
GPU output of the timed steps with the oracle on that sample (``check``:
max and mean |dO|, max |dLSE|).  Each line also names the device and the
ROCm version it ran on.
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

DEFAULT_WORKLOAD = "prefill_causal_bf16_b8h16_n4096_d128"
# the configurations, in the order they are timed: the headline last
CONFIG_WORKLOADS = ["single_head_f32_n256_d64", "ragged_causal_f16_b2h8_n1000_d64",
                    "long_bf16_b1h32_n16384_d128_qsigma8", "decode_bf16_b16h32_nk8192_d128_split32",
                    DEFAULT_WORKLOAD]
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
# MI355X fp32 vector FMA without packed instructions (the library is built
# with packed fp32 off): 256 CUs x 64 lanes x 2 FLOP x 2.4 GHz
PEAK_FP32_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# the sources each workload's dominant kernel is built from (a committed
# traffic record is used only while their hash is unchanged)
_COMMON = ["io_aware_amd/csrc/fa_layout.h", "io_aware_amd/csrc/fa_device.h"]
KERNEL_SOURCES = {
    "prefill": ["io_aware_amd/csrc/fa_prefill.hip"] + _COMMON,
    "f32": ["io_aware_amd/csrc/fa_f32.hip"],
    "decode": ["io_aware_amd/csrc/fa_decode.hip"] + _COMMON,
    "backward": ["io_aware_amd/csrc/fa_backward.hip"] + _COMMON,
    "fp8": ["io_aware_amd/csrc/fa_fp8.hip"] + _COMMON,
}


# Reference GEMM: a square bf16 product by the vendor library (torch.matmul,
# hipBLASLt), the practical matrix-core rate under the GPU's power limit.
GEMM_WORKLOAD = "gemm_bf16_n8192"
GEMM_N = 8192


def workload_kernel(name: str):
    """(source family, name pattern of the dominant kernel) of a workload."""
    import fa_inputs
    if name == GEMM_WORKLOAD:
        return "gemm", "Cijk"
    if name in fa_inputs.PAGED_WORKLOADS:
        return "decode", "splitkv_partial"
    if name in fa_inputs.VARLEN_WORKLOADS:
        return "prefill", "prefill_kernel"
    w = fa_inputs.WORKLOADS[name]
    if w.fp8:
        return "fp8", "fp8_fwd_kernel"
    if w.backward:
        return "backward", "bwd_dkdv_kernel"
    if w.num_splits:
        return "decode", "splitkv_partial"
    if w.dtype == "f32":
        return "f32", "prefill_f32"
    return "prefill", "prefill_kernel"


def workload_flops(w) -> float:
    # forward: Q K^T and P V (4d per visible pair); backward: Q K^T, dO V^T,
    # P^T dO, dS K and dS^T Q (10d per visible pair)
    f = (10.0 if w.backward else 4.0) * w.B * w.H * w.Nq * w.Nk * w.d
    return f / 2 if w.causal else f


def workload_bytes(w) -> float:
    if w.fp8:  # read the E4M3 q, k, v codes; write O (16-bit) and LSE
        return float(w.B * w.H * (w.Nq * w.d + 2 * w.Nk * w.d + 2 * w.Nq * w.d) + 4 * w.B * w.H * w.Nq)
    es = 4 if w.dtype == "f32" else 2
    if w.backward:  # read q, k, v, out, dout, lse; write dq, dk, dv
        return float(es * w.B * w.H * (5 * w.Nq * w.d + 4 * w.Nk * w.d) + 4 * w.B * w.H * w.Nq)
    return float(es * w.B * w.H * (2 * w.Nq * w.d + 2 * w.Nk * w.d) + 4 * w.B * w.H * w.Nq)


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary for
    this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(workload_kernel(workload)[0]):
        return None
    return rec.get("hbm_bytes_per_launch")


def paged_bytes(w, lens, table_entries):
    """K and V rows of every key read once, q read and out written once,
    lse written, the block table and the lengths read."""
    keys = sum(max(0, int(n)) for n in lens)
    return float(2 * 2 * w.H * w.d * keys + 2 * 2 * w.B * w.H * w.d + 4 * w.B * w.H + 4 * table_entries + 4 * w.B)


def varlen_bytes(w, lq, lk):
    """q, k, v read once, out and lse written once."""
    return float(2 * w.H * w.d * (2 * sum(lq) + 2 * sum(lk)) + 4 * w.H * sum(lq))


def algorithmic_bytes(workload: str):
    """Algorithmic bytes of one step of a workload (None if unknown)."""
    import fa_inputs
    if workload == GEMM_WORKLOAD:
        return 3 * GEMM_N * GEMM_N * 2
    if workload in fa_inputs.WORKLOADS:
        return workload_bytes(fa_inputs.WORKLOADS[workload])
    if workload in fa_inputs.PAGED_WORKLOADS:
        w = fa_inputs.PAGED_WORKLOADS[workload]
        return paged_bytes(w, fa_inputs.paged_lengths(w), w.B * -(-w.max_len // w.block_size))
    if workload in fa_inputs.VARLEN_WORKLOADS:
        w = fa_inputs.VARLEN_WORKLOADS[workload]
        return varlen_bytes(w, *fa_inputs.varlen_lengths(w))
    return None


def check_fields(o, l, ref_o, ref_l, what: str):
    """max and mean |dO| and max |dLSE| of GPU outputs against the oracle's
    on the rows the oracle computed (a row without keys must give O = 0 and
    LSE = -inf on both sides; it counts in |dO| and must match in LSE)."""
    import numpy as np
    o = np.asarray(o, dtype=np.float64).reshape(ref_o.shape)
    l = np.asarray(l, dtype=np.float64).reshape(ref_l.shape)
    fin = np.isfinite(ref_l)
    d_o = np.abs(o - ref_o)
    rec = {"vs": "fp64 oracle", "rows": what, "max_abs_dO": float(d_o.max()), "mean_abs_dO": float(d_o.mean()),
           "max_abs_dLSE": float(np.abs(l[fin] - ref_l[fin]).max()) if fin.any() else 0.0}
    if not fin.all():
        rec["rows_without_keys"] = int((~fin).sum())
        rec["lse_neg_inf_match"] = bool(np.array_equal(np.isneginf(l), ~fin))
    return rec


def bwd_cpu_baseline(w, q, k, v, target_s: float, grads):
    """Time the fp64 backward oracle on whole heads (all query and key rows),
    growing the number of heads until about ``target_s`` of work; then
    compare the GPU gradients of those heads with it."""
    import numpy as np
    import oracle
    import fa_inputs
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    gf = fa_inputs.make_dout(w.B, w.H, w.Nq, w.d, w.dtype, w.seed).float().numpy()
    n = 1
    while True:
        heads = np.arange(n)
        t0 = time.perf_counter()
        ref = oracle.attention_bwd(qf, kf, vf, gf, w.scale, w.causal, heads=heads, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= w.B * w.H:
            break
        n = min(w.B * w.H, max(n + 1, int(n * target_s / max(dt, 1e-3) * 1.1)))
    flops = workload_flops(w) / (w.B * w.H) * n
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "heads 0..%d of %d, all rows, %.1f s, fp64 backward oracle" % (n - 1, w.B * w.H, dt)}
    check = {"vs": "fp64 backward oracle", "rows": "heads 0..%d, every row" % (n - 1)}
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        x = g.float().cpu().numpy().astype(np.float64).reshape(w.B * w.H, -1, w.d)[:n]
        r = np.asarray(r, dtype=np.float64)   # [n, N, d]: the heads computed
        err = np.abs(x - r)
        rms = float(np.sqrt((r ** 2).mean()))
        check[name] = {"max_abs": float(err.max()), "max_rel_to_abs_plus_rms": float((err / (np.abs(r) + rms)).max()),
                       "mean_abs_over_rms": float(err.mean() / rms) if rms > 0 else 0.0}
    return base, check


def cpu_baseline(w, q, k, v, target_s: float, out, lse):
    """Time the fp64 oracle on a sample of rows; returns the baseline object
    and the check of the GPU output (``out``, ``lse``) on those rows."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))   # exact widening, outside the timing
    total_rows = w.B * w.H * w.Nq
    n = min(total_rows, 256)
    elapsed, flops, rows_done = 0.0, 0.0, 0
    reps = 1
    while True:
        rows = np.sort(np.random.default_rng(n).choice(total_rows, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        for _ in range(reps):
            ref_o, ref_l = oracle.attention(qf, kf, vf, w.scale, w.causal, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        vis = oracle.visible_keys(w.Nq, w.Nk, w.causal, rows)
        elapsed, flops, rows_done = dt, float(4.0 * w.d * vis.sum()) * reps, n
        if dt >= target_s or (n >= total_rows and dt >= min(target_s, 1.0)):
            break
        if n >= total_rows:  # a small workload: repeat the whole computation for a stable rate
            reps = max(reps + 1, int(reps * min(target_s, 1.0) / max(dt, 1e-4) * 1.2))
        n = min(total_rows, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
    what = ("all %d query rows" % total_rows if rows_done == total_rows else
            "%d of %d query rows drawn uniformly (numpy seed %d)" % (rows_done, total_rows, rows_done))
    base = {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%s%s, %.1f s, fp64 three-pass oracle"
                      % (what, ", computed %d times" % reps if reps > 1 else "", elapsed)}
    o = out.float().cpu().numpy().reshape(-1, w.d)[rows]
    l = lse.cpu().numpy().reshape(-1)[rows]
    return base, check_fields(o, l, ref_o, ref_l, what)


def fp8_check(w, q, k, v, signs, out, lse, nrows=512):
    """The FP8 output against exact attention on the dequantised inputs (the
    FP8 oracle) on a sample of rows."""
    import numpy as np
    import fa_inputs
    from oracle import fp8
    rows = fa_inputs.sample_rows(w.B, w.H, w.Nq, nrows, seed=w.seed)
    ro, rl, _ = fp8.fp8_attention(q, k, v, w.scale, w.causal, signs=signs.numpy(), rows=rows)
    o = out.float().cpu().numpy().reshape(-1, w.d)[rows]
    l = lse.cpu().numpy().reshape(-1)[rows]
    rec = check_fields(o, l, ro.reshape(-1, w.d)[rows], rl.reshape(-1)[rows], "%d sampled query rows" % rows.size)
    rec["vs"] = "fp64 attention on the dequantised E4M3 inputs"
    return rec


def environment():
    """Device and software the line was measured on."""
    import torch
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"device": "%s (%s, %d CUs)" % (props.name, getattr(props, "gcnArchName", "?"),
                                            props.multi_processor_count),
            "rocm": rocm, "torch_hip": torch.version.hip}


# How the timed steps are launched: "graph" (default) captures the K steps
# once into a HIP graph on a side stream and replays it, so that the host's
# per-call cost (argument checks, the ctypes call, the launch API) is not in
# the timed region -- it dominates workloads whose kernels take a few us;
# "eager" calls the K steps from Python.
LAUNCH = "graph"


def time_steps(step, steps, warmup, prewarm_s):
    """(ms per step over the timed region, mean per-step kernel ms from the
    events, {median, min} of those per-step times, the launch mode used).

    eager: untimed steps for prewarm_s seconds (the clock ramps up over the
    first tens of ms of load after idle), W warm-up steps, then the K timed
    steps back to back between two synchronisations; then K more steps, each
    between its own pair of events, give the per-step times.  graph: the W
    warm-up steps run eagerly on a side stream (which gives that stream its
    library workspace), the K steps are captured into one graph on it, the
    graph is replayed untimed for prewarm_s seconds (after the GPU idled
    during the capture), then one replay between two synchronisations (the
    timed region) and between two events gives ms per step and the mean;
    five more replays between events give the spread of (replay time / K)."""
    import torch
    dev = torch.device("cuda:0")
    launch = LAUNCH
    if launch == "graph":
        try:
            return _time_steps(step, steps, warmup, prewarm_s, "graph") + ("graph",)
        except RuntimeError as e:   # capture refused: time the same steps eagerly instead
            print("bench: graph capture failed (%s); timing eager calls" % e, file=sys.stderr, flush=True)
            torch.cuda.synchronize()
    return _time_steps(step, steps, warmup, prewarm_s, "eager") + ("eager",)


def _time_steps(step, steps, warmup, prewarm_s, launch):
    import torch
    dev = torch.device("cuda:0")
    if launch == "eager":
        stream = torch.cuda.current_stream(dev)
    else:
        stream = torch.cuda.Stream(device=dev)   # default priority
        stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        if launch == "eager":
            t_end = time.perf_counter() + prewarm_s
            while time.perf_counter() < t_end:   # clock ramp-up: untimed
                for _ in range(4):
                    step()
                torch.cuda.synchronize()
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for s, e in ev:
                s.record(stream)
                step()
                e.record(stream)
            torch.cuda.synchronize()
            t = sorted(s.elapsed_time(e) for s, e in ev)
            mean = sum(t) / len(t)
        else:
            for _ in range(max(warmup, 1)):
                step()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(steps):
                    step()
            torch.cuda.synchronize()
            t_end = time.perf_counter() + prewarm_s
            while True:                           # clock ramp-up: untimed replays
                g.replay()
                torch.cuda.synchronize()
                if time.perf_counter() >= t_end:
                    break
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            mean = e0.elapsed_time(e1) / steps
            t = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                t.append(a.elapsed_time(b) / steps)
            t.sort()
    n = len(t)
    spread = {"kernel_ms_median": t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), "kernel_ms_min": t[0]}
    return wall * 1e3 / steps, mean, spread


def run_workload(name, steps, warmup, with_cpu, cpu_target_s, prewarm_s=0.3):
    import torch
    import fa_inputs
    import io_aware_amd as fa

    if name in fa_inputs.PAGED_WORKLOADS:
        return run_paged_workload(name, steps, warmup, with_cpu, cpu_target_s, prewarm_s)
    if name in fa_inputs.VARLEN_WORKLOADS:
        return run_varlen_workload(name, steps, warmup, with_cpu, cpu_target_s, prewarm_s)
    w = fa_inputs.WORKLOADS[name]
    q, k, v = fa_inputs.make_workload(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    extra = {}
    if w.fp8:
        signs = fa_inputs.make_signs(w.d, w.seed).to(dev)
        pack = fa.fa_quantize_fp8(qd, kd, vd, signs=signs)
        qms, _, _, _ = time_steps(lambda: fa.fa_quantize_fp8(qd, kd, vd, signs=signs, pack=pack), 5, 1, 0.0)
        extra["quantize_ms"] = qms

        def step():
            fa.fa_fwd_fp8(pack, w.B, w.H, w.Nq, w.Nk, w.d, scale=w.scale, causal=w.causal, out=out, lse=lse)
    elif w.backward:
        fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=w.causal, out=out, lse=lse)
        dod = fa_inputs.make_dout(w.B, w.H, w.Nq, w.d, w.dtype, w.seed).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq, w.d), dtype=torch.uint8, device=dev)

        def step():
            fa.fa_bwd(qd, kd, vd, out, dod, lse, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws)
    elif w.num_splits:
        ws = torch.empty(fa.fa_splitkv_workspace_bytes(w.B, w.H, w.Nq, w.d, w.num_splits), dtype=torch.uint8,
                         device=dev)

        def step():
            fa.fa_fwd_splitkv(qd, kd, vd, w.num_splits, scale=w.scale, workspace=ws, out=out, lse=lse)
    else:
        def step():
            fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=w.causal, out=out, lse=lse)

    ms_per_step, kernel_ms, spread, launch = time_steps(step, steps, warmup, prewarm_s)
    flops = workload_flops(w)
    nbytes = workload_bytes(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    if w.num_splits:
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else (PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS)
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma" if w.dtype != "f32" else "alu", "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak}
    roof["traffic"] = measured_traffic(name)
    rec = {
        "metric": "attention fwd TFLOP/s (and % of MI355X bf16 MFMA/HBM roofline) per config",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s, "launch": launch,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3" if w.fp8 else w.dtype,
        "data": "synthetic (seeded randn, cast with RNE)",
        "config": {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "dtype": w.dtype, "q_sigma": w.q_sigma, "num_splits": w.num_splits,
                   "flop_per_step": flops, "algorithmic_bytes_per_step": nbytes},
        "roofline": roof,
    }
    rec.update(extra)
    rec.update(environment())
    if with_cpu:
        if w.backward:
            rec["cpu_baseline"], rec["check"] = bwd_cpu_baseline(w, q, k, v, cpu_target_s, (dq, dk, dv))
        else:
            rec["cpu_baseline"], rec["check"] = cpu_baseline(w, q, k, v, cpu_target_s, out, lse)
            if w.fp8:
                rec["check"] = fp8_check(w, q, k, v, signs.cpu(), out, lse)
    return rec


def paged_cpu_baseline(w, q, kc, vc, table, lens, target_s: float, out, lse):
    """Time the fp64 paged oracle (gather, then three-pass attention) on a
    prefix of the sequences; then check the GPU output of those sequences."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float() for t in (q, kc, vc))   # exact widening, outside the timing
    n = 1
    while True:
        t0 = time.perf_counter()
        ref_o, ref_l = oracle.paged_decode(qf, kf, vf, table, lens, w.scale, seqs=range(n), threads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= w.B:
            break
        n = min(w.B, max(n + 1, int(n * target_s / max(dt, 1e-3) * 1.1)))
    keys = int(lens[:n].clamp(min=0).sum())
    flops = 4.0 * w.H * w.d * keys
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "sequences 0..%d of %d (%d keys x %d heads), %.1f s, gather + fp64 three-pass oracle"
                      % (n - 1, w.B, keys, w.H, dt)}
    o = out[:n, :, 0].float().cpu().numpy()
    l = lse[:n].cpu().numpy()
    return base, check_fields(o, l, ref_o, ref_l, "sequences 0..%d, every head" % (n - 1))


def run_paged_workload(name, steps, warmup, with_cpu, cpu_target_s, prewarm_s):
    import torch
    import fa_inputs
    import io_aware_amd as fa

    w = fa_inputs.PAGED_WORKLOADS[name]
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    dev = torch.device("cuda:0")
    qd, kcd, vcd, td, ld = (t.to(dev).contiguous() for t in (q, kc, vc, table, lens))
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(w.B, w.H, 1, w.d, w.num_splits), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_fwd_paged_decode(qd, kcd, vcd, td, ld, w.num_splits, scale=w.scale, workspace=ws, out=out, lse=lse)

    ms_per_step, kernel_ms, spread, launch = time_steps(step, steps, warmup, prewarm_s)
    keys = int(lens.clamp(min=0).sum())
    flops = 4.0 * w.H * w.d * keys
    nbytes = paged_bytes(w, lens.tolist(), table.numel())
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(name)}
    rec = {
        "metric": "attention fwd TFLOP/s (and % of MI355X bf16 MFMA/HBM roofline) per config",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s, "launch": launch,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded randn, shuffled block table)",
        "config": {"workload": name, "B": w.B, "H": w.H, "d": w.d, "block_size": w.block_size,
                   "max_len": w.max_len, "keys_total": keys, "num_blocks": int(kc.shape[0]),
                   "num_splits": w.num_splits, "dtype": w.dtype, "flop_per_step": flops,
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": roof,
    }
    rec.update(environment())
    if with_cpu:
        rec["cpu_baseline"], rec["check"] = paged_cpu_baseline(w, q, kc, vc, table, lens, cpu_target_s, out, lse)
    return rec


def varlen_pairs(w, lq, lk):
    """Visible (query, key) pairs per head of a packed batch."""
    total = 0
    for nq, nk in zip(lq, lk):
        if w.causal:  # top-left: query i sees min(i + 1, nk) keys
            full = min(nq, nk)
            total += full * (full + 1) // 2 + max(0, nq - nk) * nk
        else:
            total += nq * nk
    return total


def run_varlen_workload(name, steps, warmup, with_cpu, cpu_target_s, prewarm_s):
    import numpy as np
    import torch
    import fa_inputs
    import io_aware_amd as fa

    w = fa_inputs.VARLEN_WORKLOADS[name]
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, cqd, ckd = (t.to(dev).contiguous() for t in (q, k, v, cq, ck))
    out = torch.empty_like(qd)
    lse = torch.empty((w.H, qd.shape[0]), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_varlen_workspace_bytes(w.S, qd.shape[0]), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, scale=w.scale, causal=w.causal, out=out, lse=lse, workspace=ws)

    ms_per_step, kernel_ms, spread, launch = time_steps(step, steps, warmup, prewarm_s)
    lq = (cq[1:] - cq[:-1]).tolist()
    lk = (ck[1:] - ck[:-1]).tolist()
    flops = 4.0 * w.d * w.H * varlen_pairs(w, lq, lk)
    nbytes = varlen_bytes(w, lq, lk)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s (and % of MI355X bf16 MFMA/HBM roofline) per config",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s, "launch": launch,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded randn, seeded length mix)",
        "config": {"workload": name, "S": w.S, "H": w.H, "d": w.d, "causal": w.causal, "dtype": w.dtype,
                   "seq_lens": lq, "total_q": sum(lq), "flop_per_step": flops,
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(name)},
    }
    rec.update(environment())
    if with_cpu:
        import oracle
        threads = len(os.sched_getaffinity(0))
        # the shortest sequences first until about cpu_target_s of oracle work
        order = list(np.argsort(lq))
        qf, kf, vf = (t.float() for t in (q, k, v))
        done, t_total, pairs = [], 0.0, 0
        o_gpu, l_gpu = out.float().cpu().numpy(), lse.cpu().numpy()
        got_o, got_l, want_o, want_l = [], [], [], []
        for sidx in order:
            t0 = time.perf_counter()
            ref_o, ref_l = oracle.varlen_attention(qf, kf, vf, cq, ck, w.scale, w.causal, seqs=[int(sidx)],
                                                   threads=threads)
            t_total += time.perf_counter() - t0
            done.append(int(sidx))
            pairs += varlen_pairs(w, [lq[sidx]], [lk[sidx]])
            r0, r1 = int(cq[sidx]), int(cq[sidx + 1])
            got_o.append(o_gpu[r0:r1])
            got_l.append(l_gpu[:, r0:r1].T)
            want_o.append(ref_o[r0:r1])
            want_l.append(ref_l[:, r0:r1].T)
            if t_total >= cpu_target_s:
                break
        rec["cpu_baseline"] = {"value": 4.0 * w.d * w.H * pairs / t_total / 1e12, "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": "%d of %d sequences, shortest first (lengths %s), %.1f s, fp64 oracle"
                                         % (len(done), w.S, [lq[i] for i in done], t_total)}
        rec["check"] = check_fields(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(want_o),
                                    np.concatenate(want_l), "sequences %s, every row and head" % done)
    return rec


def copy_probe(nbytes: int, steps: int) -> int:
    """Plain copies of a known size: each reads and writes ``nbytes`` once."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": src.numel() * 4, "steps": steps, "ms_per_copy": dt * 1e3,
                      "GB/s_read_plus_write": 2 * src.numel() * 4 / dt / 1e9}), flush=True)
    return 0


def gemm_ceiling(steps: int, warmup: int, prewarm_s: float) -> int:
    """The reference GEMM (GEMM_WORKLOAD): C = A B with A, B [n, n] bf16 by
    torch.matmul, timed like the attention steps (pre-warm, warmup, K steps
    between events).  Its rate is the matrix-core throughput the vendor
    library reaches on this GPU at the clock its power limit allows."""
    import torch
    n = GEMM_N
    g = torch.Generator(device="cpu").manual_seed(1)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to("cuda:0")
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to("cuda:0")
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda:0")
    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    for _ in range(warmup):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 2.0 * n ** 3 / ms / 1e9
    print(json.dumps({"metric": "gemm_tflops", "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_gemm": ms,
                      "steps": steps, "warmup": warmup, "dtype": "bf16", "config": {"workload": GEMM_WORKLOAD},
                      "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "environment": environment()}),
          flush=True)
    return 0


# The rocprofv3 passes --summarize-rocprof reads, one directory each under
# DIR, with the command that fills it (run from the repository root).
PROFILE_PASSES = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o trace -- "
             "python -u bench.py --workload {w} --steps 10 --warmup 2 --no-cpu-baseline",
    "sq": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
          "SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv -d {dir}/sq -o sq -- "
          "python -u bench.py --workload {w} --steps 2 --warmup 1 --prewarm-s 0 --no-cpu-baseline",
    "lds": "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
           "GRBM_GUI_ACTIVE --output-format csv -d {dir}/lds -o lds -- "
           "python -u bench.py --workload {w} --steps 2 --warmup 1 --prewarm-s 0 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/fetch -o fetch -- "
             "python -u bench.py --workload {w} --steps 2 --warmup 1 --prewarm-s 0 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/write -o write -- "
             "python -u bench.py --workload {w} --steps 2 --warmup 1 --prewarm-s 0 --no-cpu-baseline",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/copy_fetch -o copy_fetch -- "
                  "python -u bench.py --copy-bytes 1073741824 --steps 3",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/copy_write -o copy_write -- "
                  "python -u bench.py --copy-bytes 1073741824 --steps 3",
}
COPY_BYTES = 1073741824


def _find_csv(root: str, suffix: str):
    import glob
    hits = sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True))
    return hits[-1] if hits else None


def _counters(path: str, pattern: str, largest: bool = False):
    """{counter: mean value per dispatch} and the mean dispatch duration (us)
    of the kernels whose name contains ``pattern``, from a rocprofv3
    counter_collection.csv; with ``largest``, each counter's largest
    per-dispatch value instead of the mean (the copy probe's own dispatches,
    not the fill that creates its source)."""
    import csv
    per = {}
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if pattern not in row.get("Kernel_Name", ""):
                continue
            disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name = row["Counter_Name"]
            per.setdefault(name, {}).setdefault(disp, 0.0)
            per[name][disp] += float(row["Counter_Value"])
            try:
                durs[disp] = (float(row["End_Timestamp"]) - float(row["Start_Timestamp"])) / 1e3
            except (KeyError, ValueError):
                pass
    means = {n: (max(v.values()) if largest else sum(v.values()) / len(v)) for n, v in per.items() if v}
    dur = sum(durs.values()) / len(durs) if durs else None
    return means, dur


def summarize_rocprof(root: str, workload: str, out_dir: str, kernel: str = None) -> int:
    """Write profiles/<kernel>_<workload>.md and profiles/traffic_<workload>.json
    from the rocprofv3 passes under ``root`` (see PROFILE_PASSES).  ``kernel``
    names another kernel of the run than the workload's dominant one (its
    summary is written, the traffic record is not)."""
    import csv
    family, pattern = workload_kernel(workload)
    dominant = kernel is None or kernel == pattern
    pattern = kernel or pattern
    lines = ["# rocprofv3 summary: `%s` kernel, workload %s" % (pattern, workload), ""]
    trace = _find_csv(os.path.join(root, "trace"), "kernel_stats.csv")
    avg_us = None
    if trace:
        lines += ["Kernel trace (`--kernel-trace --stats`), every kernel of the run:", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        with open(trace) as f:
            for row in csv.DictReader(f):
                name = row["Name"]
                avg = float(row["AverageNs"]) / 1e3
                lines.append("| `%s` | %s | %.1f | %.1f | %.1f |" % (name, row["Calls"], avg, float(row["MinNs"]) / 1e3,
                                                                 float(row["MaxNs"]) / 1e3))
                if pattern in name and (avg_us is None or avg > avg_us):
                    avg_us = avg
        lines.append("")
    c = {}
    dur = None
    for pas in ("sq", "lds", "fetch", "write"):
        path = _find_csv(os.path.join(root, pas), "counter_collection.csv")
        if path:
            m, d = _counters(path, pattern)
            c.update(m)
            dur = dur or d
    if c:
        lines += ["Counters of `%s` (`--pmc`, one pass per group, averaged over its dispatches):" % pattern, ""]
        grbm = c.get("GRBM_GUI_ACTIVE")
        per_xcd = grbm / 8.0 if grbm else None
        if per_xcd and dur and dur >= 100.0:
            lines.append("- GRBM_GUI_ACTIVE per XCD: %.0f cycles over a %.0f us dispatch -> %.2f GHz effective clock"
                         % (per_xcd, dur, per_xcd / dur / 1e3))
        elif per_xcd and dur:
            lines.append("- GRBM_GUI_ACTIVE per XCD: %.0f cycles over a %.0f us dispatch (too short to read a clock "
                         "from; busy fractions below use these cycles)" % (per_xcd, dur))
        if per_xcd and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            lines.append("- MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): %.1f %%"
                         % (100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (per_xcd * 1024)))
        if "SQ_INSTS_MFMA" in c and "SQ_INSTS_VALU" in c:
            lines.append("- SQ_INSTS_MFMA %.4g, SQ_INSTS_VALU %.4g (VALU/MFMA = %.2f), SQ_INSTS_LDS %.4g"
                         % (c["SQ_INSTS_MFMA"], c["SQ_INSTS_VALU"], c["SQ_INSTS_VALU"] / max(c["SQ_INSTS_MFMA"], 1),
                            c.get("SQ_INSTS_LDS", float("nan"))))
        for a, b in (("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"), ("SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY")):
            if a in c and b in c:
                lines.append("- %s %.4g vs %s %.4g" % (a, c[a], b, c[b]))
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
            lines.append("- SQ_LDS_BANK_CONFLICT %.0f of SQ_LDS_IDX_ACTIVE %.4g cycles (%.2f %%)"
                         % (c["SQ_LDS_BANK_CONFLICT"], c["SQ_LDS_IDX_ACTIVE"],
                            100.0 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1)))
    traffic = None
    cf, _ = _counters(_find_csv(os.path.join(root, "copy_fetch"), "counter_collection.csv") or os.devnull, "", True)
    cw, _ = _counters(_find_csv(os.path.join(root, "copy_write"), "counter_collection.csv") or os.devnull, "", True)
    if "FETCH_SIZE" in c and "WRITE_SIZE" in c and cf.get("FETCH_SIZE") and cw.get("WRITE_SIZE"):
        # the copy reads and writes COPY_BYTES once: scale each counter to that
        fs = COPY_BYTES / 1024.0 / cf["FETCH_SIZE"]
        ws = COPY_BYTES / 1024.0 / cw["WRITE_SIZE"]
        traffic = (c["FETCH_SIZE"] * fs + c["WRITE_SIZE"] * ws) * 1024.0
        alg = algorithmic_bytes(workload)
        lines.append("- FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB per dispatch; copy calibration (1 GiB copy) "
                     "reads back FETCH x%.4f, WRITE x%.4f" % (c["FETCH_SIZE"], c["WRITE_SIZE"], fs, ws))
        lines.append("- HBM traffic per launch of `%s` (calibrated): %.4f GB%s" % (
            pattern, traffic / 1e9, "" if alg is None else "; algorithmic bytes of the whole step %.4f GB (ratio %.2f)"
            % (alg / 1e9, traffic / alg)))
    lines += ["", "Commands (each run from the repository root; OUT is a scratch directory), then "
              "`python bench.py --summarize-rocprof OUT --workload %s`:" % workload, ""]
    for pas in PROFILE_PASSES:
        if os.path.isdir(os.path.join(root, pas)):
            lines.append("    " + PROFILE_PASSES[pas].format(dir="OUT", w=workload))
    os.makedirs(out_dir, exist_ok=True)
    md = "%s_%s.md" % (pattern, workload)
    with open(os.path.join(out_dir, md), "w") as f:
        f.write("\n".join(lines) + "\n")
    if traffic is not None and dominant and family in KERNEL_SOURCES:
        rec = {"workload": workload, "kernel": pattern, "kernel_source_hash": kernel_source_hash(family),
               "fetch_kib_per_dispatch": c["FETCH_SIZE"], "write_kib_per_dispatch": c["WRITE_SIZE"],
               "copy_fetch_scale": fs, "copy_write_scale": ws, "hbm_bytes_per_launch": traffic,
               "kernel_avg_us_under_profiler": avg_us, "summary": md}
        with open(os.path.join(out_dir, "traffic_%s.json" % workload), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print("\n".join(lines))
    return 0



def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="configs",
                    help="configs (the five configurations, headline last), all, one workload name, or "
                         "gemm_bf16_n8192 (the reference GEMM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target oracle time for each line's cpu_baseline")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps (lets the GPU clock ramp up)")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="graph: capture the K timed steps into a HIP graph and replay it (default); eager: call them "
                         "one by one from Python")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, run --steps plain device-to-device copies of this many bytes "
                         "(the reference kernel for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-rocprof", metavar="DIR", default=None,
                    help="write profiles/<kernel>_<workload>.md and profiles/traffic_<workload>.json from the "
                         "rocprofv3 passes under DIR (one subdirectory per pass, see PROFILE_PASSES); no GPU")
    ap.add_argument("--kernel", default=None,
                    help="with --summarize-rocprof: summarise the kernel whose name contains this instead of the "
                         "workload's dominant one")
    ap.add_argument("--print-profile-commands", metavar="DIR", default=None,
                    help="print the rocprofv3 commands whose output --summarize-rocprof DIR reads")
    args = ap.parse_args()
    global LAUNCH
    LAUNCH = args.launch
    if args.summarize_rocprof:
        return summarize_rocprof(args.summarize_rocprof, args.workload, os.path.join(ROOT, "profiles"),
                                 kernel=args.kernel)
    if args.print_profile_commands:
        for cmd in PROFILE_PASSES.values():
            print(cmd.format(dir=args.print_profile_commands, w=args.workload))
        return 0
    if args.gpus != 1:
        print("bench.py: this forward runs on one GPU; --gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.copy_bytes:
        return copy_probe(args.copy_bytes, args.steps)
    if args.workload == GEMM_WORKLOAD:
        return gemm_ceiling(args.steps, args.warmup, args.prewarm_s)
    import fa_inputs
    if args.workload == "configs":
        names = list(CONFIG_WORKLOADS)
    elif args.workload == "all":
        extra = [n for n in list(fa_inputs.WORKLOADS) + list(fa_inputs.PAGED_WORKLOADS) +
                 list(fa_inputs.VARLEN_WORKLOADS) if n not in CONFIG_WORKLOADS]
        names = CONFIG_WORKLOADS[:-1] + extra + [DEFAULT_WORKLOAD]
    else:
        names = [args.workload]
    for name in names:
        print("bench: %s" % name, file=sys.stderr, flush=True)
        rec = run_workload(name, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline,
                           cpu_target_s=args.cpu_seconds, prewarm_s=args.prewarm_s)
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
