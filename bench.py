"""Benchmark of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one call of the forward (``fa_fwd``; ``fa_fwd_splitkv`` for the
decode workload; ``fa_fwd_paged_decode`` for the paged-cache decode) over one
batch of seeded synthetic inputs already resident in device memory.  The GPU's clock ramps up over the first tens of
milliseconds of sustained load after idle, so untimed steps run for at least
``--prewarm-s`` seconds (0.3 by default) before the W untimed warmup steps;
then K timed steps are bracketed by ``torch.cuda.synchronize()``.  Each step
is also bracketed by events on the stream the kernels run on, which gives
the per-launch kernel time used for the roofline fraction.

The default workload is causal bf16 prefill, B=8, H=16, N=4096, d=128.
FLOPs follow the convention 4*B*H*Nq*Nk*d (the two contractions), halved
under the causal mask; bytes are one read of Q, K, V and one write of O and
LSE.  One JSON line per workload goes to stdout.

The ``cpu_baseline`` leg times the fp64 oracle (test infrastructure) on a
bounded sample of query rows of the same workload on the host cores.
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
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector (packed)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# the sources each workload's dominant kernel is built from (a committed
# traffic record is used only while their hash is unchanged)
_COMMON = ["io_aware_amd/csrc/fa_layout.h", "io_aware_amd/csrc/fa_device.h"]
KERNEL_SOURCES = {
    "prefill": ["io_aware_amd/csrc/fa_prefill.hip"] + _COMMON,
    "f32": ["io_aware_amd/csrc/fa_f32.hip"],
    "decode": ["io_aware_amd/csrc/fa_decode.hip"],
    "backward": ["io_aware_amd/csrc/fa_backward.hip"] + _COMMON,
    "fp8": ["io_aware_amd/csrc/fa_fp8.hip"] + _COMMON,
}


def workload_kernel(name: str):
    """(source family, name pattern of the dominant kernel) of a workload."""
    import fa_inputs
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


def bwd_cpu_baseline(w, q, k, v, target_s: float):
    """Time the fp64 backward oracle on whole heads (all query and key rows),
    growing the number of heads until about ``target_s`` of work."""
    import numpy as np
    import oracle
    import fa_inputs
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    gf = fa_inputs.make_dout(w.B, w.H, w.Nq, w.d, w.dtype, w.seed).float().numpy()
    n = 1
    while True:
        t0 = time.perf_counter()
        oracle.attention_bwd(qf, kf, vf, gf, w.scale, w.causal, heads=np.arange(n), threads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= w.B * w.H:
            break
        n = min(w.B * w.H, max(n + 1, int(n * target_s / max(dt, 1e-3) * 1.1)))
    flops = workload_flops(w) / (w.B * w.H) * n
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "heads 0..%d of %d, all rows, %.1f s, fp64 backward oracle" % (n - 1, w.B * w.H, dt)}


def cpu_baseline(w, q, k, v, target_s: float):
    """Time the fp64 oracle on a sample of rows; returns the baseline object."""
    import numpy as np
    import oracle
    import fa_inputs
    if w.backward:
        return bwd_cpu_baseline(w, q, k, v, target_s)
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))   # exact widening, outside the timing
    total_rows = w.B * w.H * w.Nq
    n = min(total_rows, 256)
    elapsed, flops, rows_done = 0.0, 0.0, 0
    while True:
        rows = np.sort(np.random.default_rng(n).choice(total_rows, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention(qf, kf, vf, w.scale, w.causal, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        vis = oracle.visible_keys(w.Nq, w.Nk, w.causal, rows)
        elapsed, flops, rows_done = dt, float(4.0 * w.d * vis.sum()), n
        if dt >= target_s or n >= total_rows:
            break
        n = min(total_rows, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
    what = ("all %d query rows" % total_rows if rows_done == total_rows else
            "%d of %d query rows drawn uniformly (numpy seed %d)" % (rows_done, total_rows, rows_done))
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%s, %.1f s, fp64 three-pass oracle" % (what, elapsed)}


def time_steps(step, steps, warmup, prewarm_s):
    """(ms per step over the timed region, mean per-step kernel ms from the
    events, {median, min} of those per-step times)."""
    import torch
    dev = torch.device("cuda:0")
    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:   # clock ramp-up: untimed
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = sorted(s.elapsed_time(e) for s, e in ev)
    n = len(t)
    spread = {"kernel_ms_median": t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), "kernel_ms_min": t[0]}
    return wall * 1e3 / steps, sum(t) / n, spread


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
        qms, _, _ = time_steps(lambda: fa.fa_quantize_fp8(qd, kd, vd, signs=signs, pack=pack), 5, 1, 0.0)
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

    ms_per_step, kernel_ms, spread = time_steps(step, steps, warmup, prewarm_s)
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
        "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3" if w.fp8 else w.dtype,
        "data": "synthetic (seeded randn, cast with RNE)",
        "config": {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "dtype": w.dtype, "q_sigma": w.q_sigma, "num_splits": w.num_splits,
                   "flop_per_step": flops, "algorithmic_bytes_per_step": nbytes},
        "roofline": roof,
    }
    rec.update(extra)
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, cpu_target_s)
    return rec


def paged_cpu_baseline(w, q, kc, vc, table, lens, target_s: float):
    """Time the fp64 paged oracle (gather, then three-pass attention) on a
    prefix of the sequences."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    qf, kf, vf = (t.float() for t in (q, kc, vc))   # exact widening, outside the timing
    n = 1
    while True:
        t0 = time.perf_counter()
        oracle.paged_decode(qf, kf, vf, table, lens, w.scale, seqs=range(n), threads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= w.B:
            break
        n = min(w.B, max(n + 1, int(n * target_s / max(dt, 1e-3) * 1.1)))
    keys = int(lens[:n].clamp(min=0).sum())
    flops = 4.0 * w.H * w.d * keys
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "sequences 0..%d of %d (%d keys x %d heads), %.1f s, gather + fp64 three-pass oracle"
                      % (n - 1, w.B, keys, w.H, dt)}


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

    ms_per_step, kernel_ms, spread = time_steps(step, steps, warmup, prewarm_s)
    es = 2
    keys = int(lens.clamp(min=0).sum())
    flops = 4.0 * w.H * w.d * keys
    nbytes = float(2 * es * w.H * w.d * keys + 2 * es * w.B * w.H * w.d + 4 * w.B * w.H
                   + 4 * table.numel() + 4 * w.B)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(name)}
    rec = {
        "metric": "attention fwd TFLOP/s (and % of MI355X bf16 MFMA/HBM roofline) per config",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded randn, shuffled block table)",
        "config": {"workload": name, "B": w.B, "H": w.H, "d": w.d, "block_size": w.block_size,
                   "max_len": w.max_len, "keys_total": keys, "num_blocks": int(kc.shape[0]),
                   "num_splits": w.num_splits, "dtype": w.dtype, "flop_per_step": flops,
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": roof,
    }
    if with_cpu:
        rec["cpu_baseline"] = paged_cpu_baseline(w, q, kc, vc, table, lens, cpu_target_s)
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

    ms_per_step, kernel_ms, spread = time_steps(step, steps, warmup, prewarm_s)
    lq = (cq[1:] - cq[:-1]).tolist()
    lk = (ck[1:] - ck[:-1]).tolist()
    flops = 4.0 * w.d * w.H * varlen_pairs(w, lq, lk)
    nbytes = float(2 * w.H * w.d * (2 * sum(lq) + 2 * sum(lk)) + 4 * w.H * sum(lq))
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s (and % of MI355X bf16 MFMA/HBM roofline) per config",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, **spread, "prewarm_s": prewarm_s,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded randn, seeded length mix)",
        "config": {"workload": name, "S": w.S, "H": w.H, "d": w.d, "causal": w.causal, "dtype": w.dtype,
                   "seq_lens": lq, "total_q": sum(lq), "flop_per_step": flops,
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(name)},
    }
    if with_cpu:
        import oracle
        threads = len(os.sched_getaffinity(0))
        # the shortest sequences first until about cpu_target_s of oracle work
        order = list(np.argsort(lq))
        qf, kf, vf = (t.float() for t in (q, k, v))
        done, t_total, pairs = [], 0.0, 0
        for sidx in order:
            t0 = time.perf_counter()
            oracle.varlen_attention(qf, kf, vf, cq, ck, w.scale, w.causal, seqs=[int(sidx)], threads=threads)
            t_total += time.perf_counter() - t0
            done.append(int(sidx))
            pairs += varlen_pairs(w, [lq[sidx]], [lk[sidx]])
            if t_total >= cpu_target_s:
                break
        rec["cpu_baseline"] = {"value": 4.0 * w.d * w.H * pairs / t_total / 1e12, "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": "%d of %d sequences, shortest first (lengths %s), %.1f s, fp64 oracle"
                                         % (len(done), w.S, [lq[i] for i in done], t_total)}
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps (lets the GPU clock ramp up)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, run --steps plain device-to-device copies of this many bytes "
                         "(the reference kernel for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this forward runs on one GPU; --gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.copy_bytes:
        return copy_probe(args.copy_bytes, args.steps)
    import fa_inputs
    names = (list(fa_inputs.WORKLOADS) + list(fa_inputs.PAGED_WORKLOADS) + list(fa_inputs.VARLEN_WORKLOADS)
             if args.workload == "all" else [args.workload])
    for i, name in enumerate(names):
        rec = run_workload(name, args.steps, args.warmup,
                           with_cpu=(not args.no_cpu_baseline) and (i == 0 or args.workload != "all"),
                           cpu_target_s=args.cpu_seconds, prewarm_s=args.prewarm_s)
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
