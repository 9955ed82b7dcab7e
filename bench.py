"""Benchmark of block-sparse attention layer calls on one MI355X.

Default workload: the Wan2.1-1.3B 480p attention call -- B=1, H=12, d=128, bf16, token grid
21 x 30 x 52 = 32760, 4x4x8 blocks (336 x 336), block-mean scoring, top-p 0.9. A step is one
pass of the whole path over resident inputs: pool(Q), pool(K), score, select, sparse attention.

Other workloads (--config): 1 tiny fp32; 3 calibrate-then-reuse (one exact-mass calibration and
selection, then ten sparse steps; a step is their mean); 4 HunyuanVideo 720p with the per-head
minimum count; 5 Wan2.1-14B training (per layer: pool, head-global score and selection, forward
and backward; a step is the mean over the 1D/2D/3D layer cycle).

Prints one JSON line. `value` is selected-block TFLOP/s of the whole step (forward FLOPs
sum over selected (I, J) of 4 |I| |J| d, plus 8 |I| |J| d for the backward where there is one)
divided by the measured step time; `ms_per_step` is ms per layer call. `roofline` covers the
dominant kernel (the sparse attention forward) against the bf16 dense MFMA peak, timed with
events on the stream it runs on. `cpu_baseline` times the fp64 CPU oracle on a bounded sample of
the same layer (one GPU only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
METRIC = "ms/attention-layer + selected-block TFLOP/s (% bf16 MFMA peak), Wan-1.3B 480p"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle's attention sample")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scaling)")
    return ap.parse_args()


def read_traffic(kernel_src, workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source for this workload; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    with open(kernel_src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(rows, qsizes, kvsizes, d, per_pair=4):
    nq = len(qsizes)
    tot = 0
    for r, sel in enumerate(rows):
        if len(sel):
            tot += per_pair * int(qsizes[r % nq]) * int(kvsizes[sel].sum()) * d
    return tot


class Timer:
    """Per-stage event pairs on the launch stream; elapsed times read after a synchronize."""

    def __init__(self, stream):
        import torch
        self.torch, self.stream, self.marks = torch, stream, {}

    def __call__(self, name):
        timer = self

        class _Ctx:
            def __enter__(self_):
                self_.a = timer.torch.cuda.Event(enable_timing=True)
                self_.b = timer.torch.cuda.Event(enable_timing=True)
                self_.a.record(timer.stream)

            def __exit__(self_, *exc):
                self_.b.record(timer.stream)
                timer.marks.setdefault(name, []).append((self_.a, self_.b))
        return _Ctx()

    def mean_ms(self, name):
        ev = self.marks.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ev) / max(len(ev), 1)

    def reset(self):
        self.marks = {}


def cpu_baseline(w, x, rows, total_flops, target_s):
    """Time the oracle: pool + score + select over the whole layer, attention over a sample of
    query blocks, extrapolated to the layer's selected FLOPs."""
    import numpy as np
    import oracle
    from gen import bf16_bits_to_f64
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (bf16_bits_to_f64(x[n]) if x[n].dtype == np.uint16 else x[n].astype(np.float64)
               for n in ("q", "k", "v"))
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    hs = x["head_scale"].astype(np.float64)
    S = oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb), hs)
    rows_o = oracle.select_row(S, w.p)
    t_pss = time.perf_counter() - t0
    rp, ci = oracle.to_csr(rows_o)
    qs, ks = oracle.block_sizes(qb), oracle.block_sizes(kb)
    nq = len(qb)
    order = np.random.default_rng(0).permutation(len(rows_o))
    t1 = time.perf_counter()
    done_flops, n = 0, 0
    for r in order:
        b, h, i = r // (w.H * nq), (r // nq) % w.H, r % nq
        oracle.attention_fwd(Q, K, V, hs, qb, kb, rp, ci, rows=[(b, h, i)])
        done_flops += attention_flops([rows_o[r]], qs[i:i + 1], ks, w.d)
        n += 1
        if time.perf_counter() - t1 >= target_s:
            break
    t_att = time.perf_counter() - t1
    est = t_pss + t_att * (total_flops / max(done_flops, 1))
    return {"value": total_flops / est / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle: pool+score+select over the whole layer "
                       f"({t_pss:.1f} s) plus attention for {n} of {len(rows_o)} query blocks "
                       f"({t_att:.1f} s), extrapolated by selected FLOPs to one layer call "
                       f"({est:.1f} s)"),
            "ms_per_layer": est * 1e3}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has "
              f"no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import oracle
    from gen import CONFIGS, drift_step, kv_partition_for_layer, make_inputs
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention

    w = CONFIGS[args.config]
    x = make_inputs(w, tensors=("q", "k", "v", "do") if w.backward else ("q", "k", "v"))
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                     if a.dtype == np.uint16 else torch.from_numpy(a).cuda())
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    stream = torch.cuda.current_stream()
    tm = Timer(stream)
    kvparts = [kv_partition_for_layer(w, l) for l in range(3)] if w.kv_cycle else [w.kvpart]
    layers = [BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, kp, dtype=w.dtype,
                                   head_scale=x["head_scale"]) for kp in kvparts]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    do = dev(x["do"]) if w.backward else None
    head = w.mode == "head"
    mink = 2 if w.mode == "hybrid" else 0

    if w.mode == "calib":
        # later steps run on drifted inputs with the indices frozen at the calibration step
        masters = {n: x[n + "32"].copy() for n in ("q", "k", "v")}
        drift = drift_step(w, masters, 1)
        qd, kd, vd = dev(drift["q"]), dev(drift["k"]), dev(drift["v"])

    def step():
        if w.mode == "calib":
            L = layers[0]
            with tm("calibrate"):
                L.calibrate(q, k)
            with tm("select"):
                L.select(w.p)
            for _ in range(w.drift_steps):
                with tm("attn"):
                    L.attention(qd, kd, vd, out=out, lse=lse)
            return
        for L in layers:
            with tm("pool"):
                L.pool(q, k)
            with tm("score"):
                L.score(1 if head else 0)
            with tm("select"):
                L.select(w.p, 1 if head else 0, mink)
            with tm("attn"):
                L.attention(q, k, v, out=out, lse=lse)
            if w.backward:
                with tm("bwd"):
                    L.backward(q, k, v, out, do, lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fwd_flops, dens = [], []
    for L in layers:
        rp, ci = L.csr_host()
        rows = oracle.csr_rows(rp, ci)
        qs, ks = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
        f = attention_flops(rows, qs, ks, w.d)
        fwd_flops.append(f)
        dens.append(f / (4.0 * w.B * w.H * w.N * w.N * w.d))
    tm.reset()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1) / args.steps
    n_layers = len(layers)
    stages = {s: tm.mean_ms(s) for s in tm.marks}
    if w.mode == "calib":
        per_call = total_ms / (1 + w.drift_steps)            # (calibration + 10 steps) / 11
        step_flops = fwd_flops[0] * w.drift_steps / (1 + w.drift_steps)
        attn_flops = fwd_flops[0]
    else:
        per_call = total_ms / n_layers
        f_fwd = float(np.mean(fwd_flops))
        step_flops = f_fwd * (3.0 if w.backward else 1.0)   # fwd 4 + bwd 8 per pair
        attn_flops = f_fwd
    attn_ms = stages.get("attn", float("nan"))
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    value = step_flops / (per_call * 1e-3) / 1e12
    kernel_src = os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc", "attn_fwd.hip")
    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": per_call,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded smooth 3D field + 3D RoPE for Q/K, N(0,1) V)"
                if w.smooth else "synthetic (seeded iid N(0,1))",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "grid": list(w.grid),
                   "tokens": w.N, "qpart": str(w.qpart),
                   "kvpart": [str(p) for p in kvparts] if n_layers > 1 else str(w.kvpart),
                   "p": w.p, "mode": w.mode, "density": [round(d_, 4) for d_ in dens],
                   "selected_tflop_fwd": [f / 1e12 for f in fwd_flops]},
        "stage_ms": {s: round(v_, 4) for s, v_ in stages.items()},
        "attn_tflops": achieved,
        "pct_bf16_peak_step": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(kernel_src, w.name)},
    }
    if w.backward:
        res["bwd_tflops"] = 2 * attn_flops / (stages["bwd"] * 1e-3) / 1e12
    if args.copy_ref_mib:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline and w.mode in ("row", "hybrid") and args.config in (1, 2):
        L = layers[0]
        rp, ci = L.csr_host()
        res["cpu_baseline"] = cpu_baseline(w, x, oracle.csr_rows(rp, ci), fwd_flops[0],
                                           args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
