"""Benchmark of one block-sparse attention layer call on one MI355X.

Workload (default): the Wan2.1-1.3B 480p attention call -- B=1, H=12, d=128, bf16, token grid
21 x 30 x 52 = 32760, 4x4x8 blocks (336 x 336), block-mean scoring, top-p 0.9. A step is one
pass of the whole path over resident inputs: pool(Q), pool(K), score, select, sparse attention.

Prints one JSON line. `value` is the selected-block attention TFLOP/s of the whole layer call
(sum over selected (I, J) of 4 |I| |J| d, divided by the measured step time); `ms_per_step` is
ms per layer call. `roofline` covers the dominant kernel (sparse attention forward) against the
bf16 dense MFMA peak. `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
layer (rank 0, one GPU only).
"""
import argparse
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


def read_traffic(kernel_src):
    """HBM traffic per attention launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_wan480p_counters.txt")
    if not os.path.exists(path):
        return None
    with open(kernel_src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(rows, qsizes, kvsizes, d):
    nq = len(qsizes)
    tot = 0
    for r, sel in enumerate(rows):
        if len(sel):
            tot += 4 * int(qsizes[r % nq]) * int(kvsizes[sel].sum()) * d
    return tot


def cpu_baseline(w, x, rows_gpu, total_flops, target_s):
    """Time the oracle: pool + score + select over the whole layer, attention over a sample of
    query blocks, extrapolated to the layer's selected FLOPs."""
    import numpy as np
    import oracle
    from gen import bf16_bits_to_f64
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (bf16_bits_to_f64(x[n]) for n in ("q", "k", "v"))
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    hs = x["head_scale"].astype(np.float64)
    S = oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb), hs)
    rows = oracle.select_row(S, w.p)
    t_pss = time.perf_counter() - t0
    rp, ci = oracle.to_csr(rows)
    qs, ks = oracle.block_sizes(qb), oracle.block_sizes(kb)
    nq = len(qb)
    order = np.random.default_rng(0).permutation(len(rows))
    t1 = time.perf_counter()
    done_flops, n = 0, 0
    for r in order:
        b, h, i = r // (w.H * nq), (r // nq) % w.H, r % nq
        oracle.attention_fwd(Q, K, V, hs, qb, kb, rp, ci, rows=[(b, h, i)])
        done_flops += attention_flops([rows[r]], qs[i:i + 1], ks, w.d)
        n += 1
        if time.perf_counter() - t1 >= target_s:
            break
    t_att = time.perf_counter() - t1
    est = t_pss + t_att * (total_flops / max(done_flops, 1))
    return {"value": total_flops / est / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle: pool+score+select over the whole layer "
                       f"({t_pss:.1f} s) plus attention for {n} of {len(rows)} query blocks "
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
    from gen import CONFIGS, make_inputs
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention

    w = CONFIGS[args.config]
    x = make_inputs(w)
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                     if a.dtype == np.uint16 else torch.from_numpy(a).cuda())
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart, dtype=w.dtype,
                                 head_scale=x["head_scale"])
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    mode = "head" if w.mode == "head" else "row"
    mink = 2 if w.mode == "hybrid" else 0
    stream = torch.cuda.current_stream()

    def step(ev=None):
        layer.pool(q, k)
        layer.score(1 if mode == "head" else 0)
        layer.select(w.p, 1 if mode == "head" else 0, mink)
        if ev is not None:
            ev[0].record(stream)
        layer.attention(q, k, v, out=out, lse=lse)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows = oracle.csr_rows(rp, ci)
    _, qstart = layer.plan.blocks(0)
    _, kvstart = layer.plan.blocks(1)
    qs, ks = np.diff(qstart), np.diff(kvstart)
    flops = attention_flops(rows, qs, ks, w.d)
    density = flops / (4.0 * w.B * w.H * w.N * w.N * w.d)

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg = float(np.mean(attn_ms))
    achieved = flops / (attn_avg * 1e-3) / 1e12

    if args.copy_ref_mib:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kernel_src = os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc", "attn_fwd.hip")
    traffic = read_traffic(kernel_src)
    res = {
        "metric": METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded smooth 3D field + 3D RoPE for Q/K, N(0,1) V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d,
                   "grid": list(w.grid), "tokens": w.N, "qpart": str(w.qpart),
                   "kvpart": str(w.kvpart), "p": w.p, "mode": w.mode,
                   "density": round(density, 4), "selected_tflop": flops / 1e12},
        "attn_ms": attn_avg,
        "attn_tflops": achieved,
        "pct_bf16_peak_layer": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, rows, flops, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
