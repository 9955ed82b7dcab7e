"""Text summaries of rocprofv3 output, for the committed profiles.

    python -m block_sparse_attention_bsa_amd.profsum trace DB "COMMAND" [BENCH_LOG]
        Kernel table (calls, average and total microseconds, share) from the SQLite database of a
        `rocprofv3 --kernel-trace --stats` run; with the profiled run's output (BENCH_LOG), also
        the stage times bench.py measured with events in that same run.

    python -m block_sparse_attention_bsa_amd.profsum counters FETCH_CSV WRITE_CSV WORKLOAD \
        "FETCH_COMMAND" "WRITE_COMMAND"
        HBM traffic of one bsa_attn_fwd call (the two K/V permutations plus the attention kernel)
        from two `rocprofv3 --pmc` runs of bench.py with --copy-ref-mib: FETCH_SIZE and
        WRITE_SIZE (KiB per dispatch) are scaled by what the same counter reads for the plain
        device copy of known size that bench.py runs last. Writes the markdown that bench.py's
        read_traffic() parses (kernel_source_sha256_16, hbm_bytes_per_launch).
"""
import collections
import csv
import hashlib
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# The attention kernel of the call measured: the output-only kernel (an inference layer) when
# the run has it, else the one that also writes the LSE.
ATTN_KERNELS = ("attn_mfma_d128<4>", "attn_mfma_d128<0>")
PERM = "permute_rows_kernel"
COPY = "__amd_rocclr_copyBuffer"


def short(name):
    s = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", s)


def trace(db, cmd, bench_log=None):
    con = sqlite3.connect(db)
    print(f"Command: `{cmd}`\n")
    print("Durations from rocprofv3's top_kernels view (microseconds).\n")
    print("| kernel | calls | avg us | total us | % |")
    print("|---|---|---|---|---|")
    q = "select name, total_calls, total_duration, average, percentage from top_kernels"
    for name, calls, tot, avg, pct in con.execute(q):
        print(f"| {short(name)} | {calls} | {avg:.1f} | {tot:.1f} | {pct:.2f} |")
    if bench_log:
        import json
        with open(bench_log) as f:
            lines = [l for l in f if l.startswith("{")]
        if lines:
            r = json.loads(lines[-1])
            print("\nbench.py's own event timing in the same (profiled) run, ms per stage call: "
                  + ", ".join(f"{k} {v}" for k, v in r["stage_ms"].items())
                  + f"; attention {r['attn_tflops']:.1f} TFLOP/s.")


def per_dispatch(path, counter):
    """{kernel: [value per dispatch]} for one counter of a --pmc CSV."""
    out = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def counters(fetch_csv, write_csv, workload, cmd_f, cmd_w, copy_mib=1024):
    fe = per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = per_dispatch(write_csv, "WRITE_SIZE")
    ref_kib = copy_mib * 1024.0
    f_scale = ref_kib / max(fe[COPY])       # the largest copy dispatch is the reference copy
    w_scale = ref_kib / max(wr[COPY])
    mean = lambda v: sum(v) / len(v)
    ATTN = next(k for k in ATTN_KERNELS if fe.get(k) and wr.get(k))
    f_attn, w_attn = mean(fe[ATTN]) * f_scale, mean(wr[ATTN]) * w_scale
    f_perm, w_perm = mean(fe[PERM]) * f_scale, mean(wr[PERM]) * w_scale
    per_call_kib = f_attn + w_attn + 2 * (f_perm + w_perm)
    src = os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc", "attn_fwd.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    print(f"# HBM traffic of one bsa_attn_fwd call, {workload}\n")
    print(f"FETCH_SIZE run: `{cmd_f}`\n")
    print(f"WRITE_SIZE run: `{cmd_w}`\n")
    print(f"Scaling: the {copy_mib} MiB device copy that bench.py runs last reads "
          f"{max(fe[COPY]):.0f} KiB by FETCH_SIZE and writes {max(wr[COPY]):.0f} KiB by "
          f"WRITE_SIZE, so FETCH_SIZE is multiplied by {f_scale:.3f} and WRITE_SIZE by "
          f"{w_scale:.3f}.\n")
    print("| kernel | dispatches | FETCH KiB (scaled) | WRITE KiB (scaled) |")
    print("|---|---|---|---|")
    print(f"| {ATTN} | {len(fe[ATTN])} | {f_attn:.0f} | {w_attn:.0f} |")
    print(f"| {PERM} (x2 per call) | {len(fe[PERM])} | {f_perm:.0f} | {w_perm:.0f} |")
    print()
    print(f"- workload: {workload}")
    print(f"- kernel_source_sha256_16: {sha}")
    print(f"- hbm_bytes_per_launch: {per_call_kib * 1024:.0f}")


def main(argv):
    if len(argv) >= 3 and argv[0] == "trace":
        trace(argv[1], argv[2], argv[3] if len(argv) > 3 else None)
    elif len(argv) >= 6 and argv[0] == "counters":
        counters(argv[1], argv[2], argv[3], argv[4], argv[5])
    else:
        sys.stderr.write(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
