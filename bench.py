"""Benchmark of block-sparse attention layer calls on one MI355X.

Default workload: the Wan2.1-1.3B 480p attention call -- B=1, H=12, d=128, bf16, token grid
21 x 30 x 52 = 32760, 4x4x8 blocks (336 x 336), block-mean scoring, top-p 0.9. A step is one
pass of the whole path over resident inputs: pool(Q), pool(K), score, select, sparse attention.

Other workloads (--config): 1 tiny fp32; 3 calibrate-then-reuse (one dense step that returns the
exact block masses with its attention output, the selection, then ten sparse steps; a step is
their mean); 4 HunyuanVideo 720p with the per-head
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
from contextlib import nullcontext
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
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the untimed extra measurements (entropy-routed, Local + TopK and "
                         "per-token selection, attention with LSE), e.g. under a profiler")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scaling)")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only measure the MFMA and copy ceilings (bsa_probe_mfma, "
                         "bsa_probe_copy) and print them")
    ap.add_argument("--score-path", choices=("fused", "unfused"), default="unfused",
                    help="ROW-pool workloads: scores and selection in one kernel "
                         "(bsa_score_select) or bsa_score then bsa_select")
    return ap.parse_args()


def source_sha16(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def sources_sha16():
    """{attn_fwd.hip: hash, csrc: one hash over every source and header of the library in name
    order}, recorded with each line so that a profile can name the sources it was taken on."""
    import glob
    csrc = os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc")
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(csrc, "*"))):
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return {"attn_fwd.hip": source_sha16(os.path.join(csrc, "attn_fwd.hip")),
            "csrc": h.hexdigest()[:16]}


def read_traffic(kernel_src, workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source for this workload; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    sha = source_sha16(kernel_src)
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = (v.split() or [""])[0].strip("`")
    if vals.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def entropy_routed(w, L, q, k, v, out, tm, group_size=4, calls=5):
    """The same layer with EG-Sparse's entropy-routed selection (bsa_select_eg) in place of the
    per-row one, timed outside the step: pooled heads, the selection's time, the density and
    the output-only attention time on its block sets. theta is the median of the heads'
    entropies, so about half of the heads compete in a pool of group_size heads."""
    import numpy as np
    import torch
    L.pool(q, k)
    L.score(0)
    L.select_eg(w.p, float("-inf"), group_size)          # entropies only
    torch.cuda.synchronize()
    ent = L.head_entropy.cpu().numpy().astype(np.float64)
    theta = float(np.median(ent))
    for _ in range(calls):
        with tm("select_eg"):
            L.select_eg(w.p, theta, group_size)
        with tm("attn_eg"):
            L.attention(q, k, v, out=out, with_lse=False)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    qs, ks = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    f = attention_flops(csr_rows(rp, ci), qs, ks, w.d)
    attn_ms = tm.mean_ms("attn_eg")
    return {"group_size": group_size, "theta": theta,
            "pooled_heads": int(L.head_pooled.sum().item()), "heads": int(ent.size),
            "select_ms": round(tm.mean_ms("select_eg"), 4),
            "density": round(f / (4.0 * w.B * w.H * w.N * w.N * w.d), 4),
            "empty_row_fraction": round(float(np.mean(np.diff(rp) == 0)), 4),
            "attn_ms": round(attn_ms, 4), "attn_tflops": f / (attn_ms * 1e-3) / 1e12}


def local_topk(w, L, q, k, v, out, tm, ks=(2, 6, 18), calls=5):
    """VMoBA's training-free Local + TopK selection (BSA_POOL_LOCAL_TOPK) for k = 2, 6, 18,
    timed outside the step: the selection's time, the density and the output-only attention
    time on its block sets."""
    import numpy as np
    import torch
    from block_sparse_attention_bsa_amd import BSA_POOL_LOCAL_TOPK
    L.pool(q, k)
    L.score(0)
    qs, ksz = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    res = {}
    for kk in ks:
        for _ in range(calls):
            with tm(f"select_lt{kk}"):
                L.select(w.p, pool=BSA_POOL_LOCAL_TOPK, fixed_k=kk)
            with tm(f"attn_lt{kk}"):
                L.attention(q, k, v, out=out, with_lse=False)
        torch.cuda.synchronize()
        rp, ci = L.csr_host()
        f = attention_flops(csr_rows(rp, ci), qs, ksz, w.d)
        attn_ms = tm.mean_ms(f"attn_lt{kk}")
        res[str(kk)] = {"select_ms": round(tm.mean_ms(f"select_lt{kk}"), 4),
                        "density": round(f / (4.0 * w.B * w.H * w.N * w.N * w.d), 4),
                        "attn_ms": round(attn_ms, 4),
                        "attn_tflops": f / (attn_ms * 1e-3) / 1e12}
    return res


def token_topk(w, L, q, k, v, out, tm, ks=(2, 6, 18), calls=3):
    """Per-token Local + TopK (bsa_select_tokens + bsa_attn_fwd_tokens) for k = 2, 6, 18, timed
    outside the step. FLOPs: `token` counts each token's own selected keys (4 d per query-key
    pair), `executed` the union blocks its query block streams."""
    import numpy as np
    import torch
    L.pool(q, k)
    qs, ksz = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    res = {}
    for kk in ks:
        for _ in range(calls):
            with tm(f"select_tok{kk}"):
                sel = L.select_tokens(q, kk)
            with tm(f"attn_tok{kk}"):
                L.attention_tokens(q, k, v, sel, kk, out=out, with_lse=False)
        torch.cuda.synchronize()
        keys_per_token = ksz[sel.cpu().numpy()].sum(-1)          # [B, H, N]
        f_tok = 4.0 * w.d * float(keys_per_token.sum())
        rp, ci = L.csr_host()
        f_exec = attention_flops(csr_rows(rp, ci), qs, ksz, w.d)
        attn_ms = tm.mean_ms(f"attn_tok{kk}")
        dense = 4.0 * w.B * w.H * w.N * w.N * w.d
        res[str(kk)] = {"select_ms": round(tm.mean_ms(f"select_tok{kk}"), 4),
                        "density_token": round(f_tok / dense, 4),
                        "density_executed": round(f_exec / dense, 4),
                        "attn_ms": round(attn_ms, 4),
                        "attn_tflops_token": f_tok / (attn_ms * 1e-3) / 1e12,
                        "attn_tflops_executed": f_exec / (attn_ms * 1e-3) / 1e12}
    return res


def token_global(w, L, q, k, v, out, tm, tau=0.25, calls=5):
    """VMoBA's per-token global threshold selection (bsa_select_tokens_global, tau = 0.25 of the
    review's free parameters) on the same inputs, timed outside the step: the selection's time,
    the token-level density (pairs each token attends / N^2), the density the union walk
    executes, the share of tokens that keep no block, and the output-only attention time over
    the per-token bitmaps."""
    import numpy as np
    import torch
    L.pool(q, k)
    for _ in range(calls):
        with tm("select_tg"):
            bits = L.select_tokens_global(q, tau)
        with tm("attn_tg"):
            L.attention_token_bits(q, k, v, bits, out=out, with_lse=False)
    torch.cuda.synchronize()
    qs, ksz = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    nkv = len(ksz)
    b = np.ascontiguousarray(bits.cpu().numpy().reshape(-1, bits.shape[-1])).view(np.uint32)
    keys, empty = 0.0, 0
    for r0 in range(0, b.shape[0], 1 << 16):  # token rows in chunks (720p: 2.85 M rows)
        flags = np.unpackbits(b[r0:r0 + (1 << 16)].view(np.uint8), axis=1,
                              bitorder="little")[:, :nkv]
        keys += float((flags.astype(np.float64) @ ksz.astype(np.float64)).sum())
        empty += int((flags.sum(axis=1) == 0).sum())
    f_tok = 4.0 * w.d * keys
    rp, ci = L.csr_host()
    f_exec = attention_flops(csr_rows(rp, ci), qs, ksz, w.d)
    attn_ms = tm.mean_ms("attn_tg")
    dense = 4.0 * w.B * w.H * w.N * w.N * w.d
    return {"tau": tau, "select_ms": round(tm.mean_ms("select_tg"), 4),
            "density_token": round(f_tok / dense, 4), "density_executed": round(f_exec / dense, 4),
            "empty_token_fraction": round(empty / b.shape[0], 4),
            "attn_ms": round(attn_ms, 4),
            "attn_tflops_token": f_tok / (attn_ms * 1e-3) / 1e12,
            "attn_tflops_executed": f_exec / (attn_ms * 1e-3) / 1e12}


def dense_reference(w, L, q, k, v, out, tm, calls=3):
    """The same attention kernel with every block selected (a per-head minimum of nkv blocks
    keeps every block of every row), timed outside the step: the cost of the sparse walk without
    sparsity, to compare the step's selected-block rate with."""
    import numpy as np
    import torch
    from block_sparse_attention_bsa_amd import BSA_MINK_FIXED
    L.pool(q, k)
    L.score()
    L.select(1.0, min_k_mode=BSA_MINK_FIXED, fixed_k=L.plan.nkv)
    for _ in range(calls):
        with tm("attn_dense"):
            L.attention(q, k, v, out=out, with_lse=False)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    qs, ksz = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    f = attention_flops(csr_rows(rp, ci), qs, ksz, w.d)
    attn_ms = tm.mean_ms("attn_dense")
    tfl = f / (attn_ms * 1e-3) / 1e12
    return {"density": round(f / (4.0 * w.B * w.H * w.N * w.N * w.d), 4),
            "attn_ms": round(attn_ms, 4), "attn_tflops": tfl,
            "frac": tfl / PEAK_BF16_TFLOPS}


def p_sweep(w, L, q, k, v, out, tm, ps=(0.3, 0.6), calls=3):
    """The same layer at lower thresholds p (sparser block sets than the workload's p), timed
    outside the step: the attention kernel's selected-block rate across densities."""
    import numpy as np
    import torch
    L.pool(q, k)
    L.score()
    qs, ksz = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
    res = {}
    for p in ps:
        L.select(p)
        for _ in range(calls):
            with tm(f"attn_p{p}"):
                L.attention(q, k, v, out=out, with_lse=False)
        torch.cuda.synchronize()
        rp, ci = L.csr_host()
        f = attention_flops(csr_rows(rp, ci), qs, ksz, w.d)
        ms = tm.mean_ms(f"attn_p{p}")
        res[str(p)] = {"density": round(f / (4.0 * w.B * w.H * w.N * w.N * w.d), 4),
                       "attn_ms": round(ms, 4), "attn_tflops": f / (ms * 1e-3) / 1e12}
    return res


def measured_peaks(tm, copy_mib=1024, reps=3):
    """The ceilings on this GPU: the bf16 MFMA rate of back-to-back v_mfma_f32_32x32x16_bf16 and
    v_mfma_f32_16x16x32_bf16 loops (bsa_probe_mfma), and the read + write rate of a 16-byte grid-stride copy of copy_mib
    MiB (bsa_probe_copy) and of torch's device copy of the same tensors. Best of reps calls."""
    import torch
    from block_sparse_attention_bsa_amd import bsa_probe_copy, bsa_probe_mfma
    wgs = 2048
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    n = copy_mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    flops = 0.0
    for _ in range(reps + 1):
        with tm("probe_mfma"):
            flops = bsa_probe_mfma(0, wgs, 256, sink)
        with tm("probe_mfma16"):
            bsa_probe_mfma(1, wgs, 256, sink)
        with tm("probe_copy"):
            bsa_probe_copy(src, dst, n)
        with tm("probe_torch_copy"):
            dst.copy_(src)
    # the forward's instruction mix at its occupancy (768 workgroups: three per CU, one
    # wavefront of each per SIMD): per round 16 MFMAs and/or 32 exponentials or FMAs
    mix_wgs, mix_iters = 768, 4000
    mix_names = {2: "mfma", 3: "mfma_exp", 4: "exp", 5: "mfma_fma", 6: "fma"}
    for _ in range(reps + 1):
        for shape, name in mix_names.items():
            with tm("probe_mix_" + name):
                bsa_probe_mfma(shape, mix_wgs, mix_iters, sink)
    torch.cuda.synchronize()
    best = lambda k: min(a.elapsed_time(b) for a, b in tm.marks[k][1:])  # skip the first call
    # ns per round of every SIMD (its three wavefronts each run mix_iters rounds)
    mix = {name: round(best("probe_mix_" + name) * 1e6 / mix_iters, 1)
           for name in mix_names.values()}
    r32 = flops / (best("probe_mfma") * 1e-3) / 1e12
    r16 = flops / (best("probe_mfma16") * 1e-3) / 1e12
    return {"mfma_bf16_tflops": round(max(r32, r16), 1),
            "mfma_32x32x16_tflops": round(r32, 1), "mfma_16x16x32_tflops": round(r16, 1),
            "copy_kernel_gbs": round(2 * n / (best("probe_copy") * 1e-3) / 1e9, 1),
            "copy_torch_gbs": round(2 * n / (best("probe_torch_copy") * 1e-3) / 1e9, 1),
            "copy_bytes_moved": 2 * n,
            "mix_ns_per_round": mix,
            "method": "bsa_probe_mfma (v_mfma_f32_32x32x16_bf16 and 16x16x32 loops, 2048 x 256 "
                      "threads; the faster counts) and bsa_probe_copy / torch copy_ of 1 GiB, "
                      "best of 3 calls after one warm-up; mix_ns_per_round: shapes 2-6 at "
                      "768 x 256 threads (three wavefronts per SIMD), 4000 rounds, ns per round "
                      "of 3 x 16 MFMAs and/or 3 x 32 exponentials or FMAs per SIMD"}


def score_paths(w, L, q, k, mink, tm, calls=10):
    """Scores and selection as one kernel (bsa_score_select: S never goes through memory, except
    for the per-head minimum's top-up) against bsa_score followed by bsa_select, on the same
    pooled inputs; both give the same CSR."""
    import torch
    L.pool(q, k)
    for _ in range(2):
        L.score_select(w.p, min_k_mode=mink)
        L.score(0)
        L.select(w.p, 0, mink)
    for _ in range(calls):
        with tm("sp_fused"):
            L.score_select(w.p, min_k_mode=mink)
        with tm("sp_score"):
            L.score(0)
        with tm("sp_select"):
            L.select(w.p, 0, mink)
    torch.cuda.synchronize()
    f, a, b = tm.mean_ms("sp_fused"), tm.mean_ms("sp_score"), tm.mean_ms("sp_select")
    return {"fused_ms": round(f, 4), "score_ms": round(a, 4), "select_ms": round(b, 4),
            "unfused_ms": round(a + b, 4), "speedup": round((a + b) / f, 2)}


def csr_rows(row_ptr, col_idx):
    """The CSR's rows as a list of index arrays (for the FLOP count of the selected blocks)."""
    return [col_idx[row_ptr[r]:row_ptr[r + 1]] for r in range(len(row_ptr) - 1)]


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

    def stats_ms(self, name):
        """Median, p10 and p90 of the individual calls."""
        import numpy as np
        t = np.array([a.elapsed_time(b) for a, b in self.marks.get(name, [])])
        if not len(t):
            return None
        return {"median": round(float(np.median(t)), 4),
                "p10": round(float(np.percentile(t, 10)), 4),
                "p90": round(float(np.percentile(t, 90)), 4), "calls": int(len(t))}

    def reset(self):
        self.marks = {}


def host_info():
    """CPU model and the BLAS numpy is built on (reported with the oracle's timing)."""
    import numpy as np
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        blas = np.__config__.CONFIG["Build Dependencies"]["blas"]
        blas = f"{blas.get('name')} {blas.get('version')}"
    except Exception:  # older numpy: no structured config
        blas = "unknown"
    return model, blas


def cpu_baseline(w, x, total_flops, target_s, threads=None):
    """Time the oracle: pool + score + select over the whole layer, attention over a sample of
    query blocks, extrapolated to the layer's selected FLOPs. threads=1 limits BLAS to one
    thread (otherwise it uses every core this process may run on)."""
    import numpy as np
    import oracle
    from gen import bf16_bits_to_f64
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            r = cpu_baseline(w, x, total_flops, target_s)
        r["cores"] = threads
        return r
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    Q, K, V = (bf16_bits_to_f64(x[n]) if x[n].dtype == np.uint16 else x[n].astype(np.float64)
               for n in ("q", "k", "v"))
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    hs = x["head_scale"].astype(np.float64)
    ta = time.perf_counter()
    Qb, Kb = oracle.pool(Q, qb), oracle.pool(K, kb)
    tb = time.perf_counter()
    S = oracle.score_row(Qb, Kb, hs)
    tc = time.perf_counter()
    rows_o = oracle.select_row(S, w.p)
    td = time.perf_counter()
    t_pss = td - t0
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
    model, blas = host_info()
    return {"value": total_flops / est / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": model, "blas": blas,
            "stage_s": {"pool": round(tb - ta, 4), "score": round(tc - tb, 4),
                        "select": round(td - tc, 4),
                        "attn_extrapolated": round(t_att * total_flops / max(done_flops, 1), 3)},
            "sample": (f"fp64 numpy oracle: pool+score+select over the whole layer "
                       f"({t_pss:.1f} s) plus attention for {n} of {len(rows_o)} query blocks "
                       f"({t_att:.1f} s), extrapolated by selected FLOPs to one layer call "
                       f"({est:.1f} s)"),
            "ms_per_layer": est * 1e3}


def retained_mass(w, x, L, dev):
    """Calibrate-then-reuse quality: the exact attention mass the frozen block set keeps on each
    of the drifted steps. Exact block masses of step s come from the calibration kernel run on
    that step's inputs; the retained mass of a row is the sum of its masses over the blocks frozen
    at step 0. Reported as the mean and minimum over rows, per step."""
    import numpy as np
    from gen import drift_step
    rp, ci = L.csr_host()
    nq, nkv = L.plan.nq, L.plan.nkv
    sel = np.zeros((len(rp) - 1, nkv), dtype=bool)
    for r in range(len(rp) - 1):
        sel[r, ci[rp[r]:rp[r + 1]]] = True
    def kept_stats(M, s):
        kept = (M.reshape(-1, nkv) * sel).sum(axis=1)
        return {"step": s, "mean": round(float(kept.mean()), 5), "min": round(float(kept.min()), 5)}
    out = [kept_stats(L.S.cpu().numpy(), 0)]  # the calibration step itself (>= p by construction)
    masters = {n: x[n + "32"].copy() for n in ("q", "k", "v")}
    for s in range(1, w.drift_steps + 1):
        d = drift_step(w, masters, s)
        out.append(kept_stats(L.calibrate(dev(d["q"]), dev(d["k"])).cpu().numpy(), s))
    return {"threshold": w.p, "source": "exact block masses of each drifted step (calibration "
            "kernel); blocks frozen at step 0", "retained_mass": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has "
              f"no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.peaks_only:
        print(json.dumps({"measured_peaks": measured_peaks(Timer(torch.cuda.current_stream())),
                          "sources_sha256_16": sources_sha16()}), flush=True)
        return

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
    # per-layer stage names for the 1D / 2D / 3D cycle (temporal, spatial, spatio-temporal)
    tags = ["@1D", "@2D", "@3D"] if w.kv_cycle else [""]
    layers = [BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, kp, dtype=w.dtype,
                                   head_scale=x["head_scale"]) for kp in kvparts]
    out = torch.empty_like(q)
    # The LSE is an output of the training layer (the backward consumes it); an inference layer
    # requests O only, which runs the output-only attention kernel.
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda") if w.backward else None
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
            # the dense step: exact block masses and that step's dense attention output together
            L = layers[0]
            with tm("dense_step"):
                L.calibrate_attention(q, k, v, out=out, lse=lse)
            with tm("select"):
                L.select(w.p)
            for _ in range(w.drift_steps):
                with tm("attn"):
                    L.attention(qd, kd, vd, out=out, lse=lse, with_lse=w.backward)
            return
        for L, tag in zip(layers, tags):
            with tm("pool"):
                L.pool(q, k)
            if head or args.score_path == "unfused":
                with tm("score"):
                    L.score(1 if head else 0)
                with tm("select"):
                    L.select(w.p, 1 if head else 0, mink)
            else:
                with tm("score_select"):
                    L.score_select(w.p, min_k_mode=mink)
            with tm("attn"), (tm("attn" + tag) if tag else nullcontext()):
                L.attention(q, k, v, out=out, lse=lse, with_lse=w.backward)
            if w.backward:
                with tm("bwd"), (tm("bwd" + tag) if tag else nullcontext()):
                    L.backward(q, k, v, out, do, lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fwd_flops, dens, empty = [], [], []
    for L in layers:
        rp, ci = L.csr_host()
        rows = csr_rows(rp, ci)
        qs, ks = np.diff(L.plan.blocks(0)[1]), np.diff(L.plan.blocks(1)[1])
        f = attention_flops(rows, qs, ks, w.d)
        fwd_flops.append(f)
        dens.append(f / (4.0 * w.B * w.H * w.N * w.N * w.d))
        empty.append(float(np.mean(np.diff(rp) == 0)))
    tm.reset()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        with tm("step"):
            step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1) / args.steps
    n_layers = len(layers)
    stages = {s: tm.mean_ms(s) for s in tm.marks if s != "step"}
    stage_stats = {s: tm.stats_ms(s) for s in tm.marks}
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
        "call_stats_ms": stage_stats,
        "empty_row_fraction": [round(e, 4) for e in empty],
        "attn_tflops": achieved,
        "sources_sha256_16": sources_sha16(),
        "pct_bf16_peak_step": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(kernel_src, w.name),
                     "kernel_source_sha256_16": source_sha16(kernel_src)},
    }
    if w.backward:
        res["bwd_tflops"] = 2 * attn_flops / (stages["bwd"] * 1e-3) / 1e12
        # per member of the 1D / 2D / 3D cycle: forward, backward and their sum
        res["per_partition_ms"] = {
            (t[1:] or "single"): {"fwd": round(stages["attn" + t], 4),
                                  "bwd": round(stages["bwd" + t], 4),
                                  "fwd+bwd": round(stages["attn" + t] + stages["bwd" + t], 4)}
            for t in tags}
    if "pool" in stages:
        elt = 2 if w.dtype == "bf16" else 4
        L = layers[0]
        pool_bytes = (2 * w.B * w.H * w.N * w.d * elt
                      + (L.plan.nq + L.plan.nkv) * w.B * w.H * w.d * 4)
        gbs = pool_bytes / (stages["pool"] * 1e-3) / 1e9
        res["pool"] = {"GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
                       "bytes": pool_bytes}
    if w.mode == "hybrid":
        hk = layers[0].head_k.cpu().numpy()
        res["head_k"] = {"min": int(hk.min()), "median": float(np.median(hk)),
                         "max": int(hk.max()), "nkv": layers[0].plan.nkv}
    if w.mode == "calib":
        for _ in range(3):  # the masses alone (no dense output), for comparison
            with tm("calibrate_masses_only"):
                layers[0].calibrate(q, k)
        torch.cuda.synchronize()
        res["stage_ms"]["calibrate_masses_only"] = round(tm.mean_ms("calibrate_masses_only"), 4)
        res["calibrate_then_reuse"] = retained_mass(w, x, layers[0], dev)
    if not w.backward and not args.no_extras:
        # the same attention call with the LSE requested as well (the training kernel), untimed
        # in the step
        lse_x = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        qa, ka, va = (qd, kd, vd) if w.mode == "calib" else (q, k, v)
        for _ in range(5):
            with tm("attn_with_lse"):
                layers[0].attention(qa, ka, va, out=out, lse=lse_x)
        torch.cuda.synchronize()
        res["attn_with_lse"] = {"ms": round(tm.mean_ms("attn_with_lse"), 4),
                                "tflops": attn_flops / (tm.mean_ms("attn_with_lse") * 1e-3)
                                / 1e12}
    if w.mode in ("row", "hybrid") and not args.no_extras:
        res["score_paths"] = score_paths(w, layers[0], q, k, mink, tm)
    if w.mode in ("row", "hybrid") and w.dtype == "bf16" and not args.no_extras:
        # other selections on the same inputs (they replace the layer's CSR: keep them last)
        res["entropy_routed"] = entropy_routed(w, layers[0], q, k, v, out, tm)
        res["local_topk"] = local_topk(w, layers[0], q, k, v, out, tm)
        res["token_topk"] = token_topk(w, layers[0], q, k, v, out, tm)
        if layers[0].plan.nkv <= 2048:  # the per-token bitmap attention's limit
            res["token_global"] = token_global(w, layers[0], q, k, v, out, tm)
        res["p_sweep"] = p_sweep(w, layers[0], q, k, v, out, tm)
        res["dense_reference"] = dense_reference(w, layers[0], q, k, v, out, tm)
    if not args.no_extras:
        res["measured_peaks"] = mp = measured_peaks(tm)
        res["roofline"]["frac_of_measured"] = achieved / mp["mfma_bf16_tflops"]
        res["roofline"]["measured_peak"] = mp["mfma_bf16_tflops"]
        if "pool" in res:
            res["pool"]["pct_of_measured_copy"] = round(
                100 * res["pool"]["GB/s"] / max(mp["copy_kernel_gbs"], mp["copy_torch_gbs"]), 1)
    if args.copy_ref_mib:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline and w.mode in ("row", "hybrid") and args.config in (1, 2):
        res["cpu_baseline"] = cpu_baseline(w, x, fwd_flops[0], args.cpu_seconds)
        if args.config == 1:
            res["cpu_baseline_1thread"] = cpu_baseline(w, x, fwd_flops[0], args.cpu_seconds,
                                                       threads=1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
