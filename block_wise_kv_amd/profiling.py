"""rocprofv3 post-processing for the decoding kernels, and a plain copy
workload that calibrates the HBM byte counters. Nothing here runs on the
decoding path.

    # a known-size copy, to scale FETCH_SIZE / WRITE_SIZE
    python3 -m block_wise_kv_amd.profiling copy --mib 1024 --reps 4

    # attention / unmask sweep table from kernel_sweep's JSON and the trace
    # of a run of the same sweep (reads <dir>/**/*_kernel_trace.csv)
    python3 -m block_wise_kv_amd.profiling sweep --json J --trace DIR --reps R \
        --cmd-events "..." --cmd-trace "..." > profiles/attention_unmask_sweep.md

    # kernel-trace summary (reads <dir>/**/*_kernel_stats.csv)
    python3 -m block_wise_kv_amd.profiling stats DIR --title T --cmd "..." > profiles/x.md

    # HBM bytes per launch from counter runs (reads *_counter_collection.csv)
    python3 -m block_wise_kv_amd.profiling traffic --fetch D1 --write D2 \
        --copy-fetch D3 --copy-write D4 [--mfma D5 (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16)] --copy-mib 1024 --cmd "..." --out profiles/traffic.json

Kernel names from the trace are mapped onto the variant names the library's
own launch timer uses (gemm_<epilogue>_bm<rows>, attention, embed,
final_norm, unmask_stats, unmask_select), so counter, trace and event figures
line up.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EPILOGUES = ("qkv", "resid", "swiglu", "lmhead")
# sources whose change makes a kernel family's stored counter figures stale
SOURCES = {
    "gemm": ("gemm.hip", "common.h", "internal.h", "select.h"),
    "attention": ("attention.hip", "common.h", "internal.h"),
    "other": ("misc.hip", "unmask.hip", "common.h", "internal.h", "select.h"),
}


def family(variant: str) -> str:
    return "gemm" if variant.startswith("gemm_") else ("attention" if variant == "attention" else "other")


def source_hash(fam: str) -> str:
    h = hashlib.sha256()
    for f in SOURCES[fam]:
        with open(os.path.join(ROOT, "block_wise_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def variant(kernel_name: str) -> str | None:
    """Library variant name of a demangled kernel name (None: not ours)."""
    m = re.search(r"fdllm::gemm_kernel<fdllm::(?:BF16|F32), (\d+), (\d+), (\d+), (?:true|false)(?:, (?:true|false))?>", kernel_name)
    if m:
        return f"gemm_{EPILOGUES[int(m.group(3))]}_bm{m.group(1)}"
    for key, name in (("attn_kernel", "attention"), ("embed_kernel", "embed"),
                      ("final_norm_kernel", "final_norm"), ("unmask_stats_kernel", "unmask_stats"),
                      ("unmask_select_kernel", "unmask_select")):
        if f"fdllm::{key}" in kernel_name:
            return name
    return None


def _rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def kernel_stats(directory: str) -> dict:
    """{name: (calls, total_ns, avg_ns)} from rocprofv3 --stats output."""
    out = {}
    for r in _rows(directory, "_kernel_stats.csv"):
        out[r["Name"]] = (int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]))
    return out


def counters(directory: str, counter: str) -> dict:
    """{dispatch_id: (kernel_name, grid, value)} for one counter."""
    out = {}
    for r in _rows(directory, "_counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        prev = out.get(did)
        v = float(r["Counter_Value"]) + (prev[2] if prev else 0.0)
        grid = next((int(float(r[k])) for k in r if k.startswith("Grid_Size") and r[k]), 0)
        out[did] = (r["Kernel_Name"], grid, v)
    return out


def per_variant(values: dict) -> dict:
    acc = defaultdict(lambda: [0, 0.0])
    for name, _, v in values.values():
        var = variant(name)
        if var:
            acc[var][0] += 1
            acc[var][1] += v
    return acc


def copy_kib(values: dict) -> float:
    """Counter value (KiB) of the calibration copy: mean over the dispatches
    of the largest-grid kernel that is not one of ours."""
    cand = [(g, v) for n, g, v in values.values() if variant(n) is None]
    if not cand:
        raise SystemExit("no copy dispatch found")
    gmax = max(g for g, _ in cand)
    vals = [v for g, v in cand if g == gmax]
    return sum(vals) / len(vals)


# ----------------------------------------------------------------------------

def cmd_copy(a) -> int:
    import torch
    n = a.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        torch.neg(src, out=dst)  # one elementwise kernel: reads and writes mib MiB
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": a.mib, "reps": a.reps}), flush=True)
    return 0


def cmd_stats(a) -> int:
    st = kernel_stats(a.dir)
    tot = sum(v[1] for v in st.values())
    by_var = defaultdict(lambda: [0, 0.0])
    print(f"# {a.title}\n")
    print("Command (from the repository root):\n")
    print(f"    {a.cmd}\n")
    print(f"Total kernel time {tot / 1e6:.2f} ms over {sum(v[0] for v in st.values())} dispatches.\n")
    print("| kernel | variant | calls | total ms | avg us | share |")
    print("|---|---|---|---|---|---|")
    for name, (calls, tns, avg) in sorted(st.items(), key=lambda kv: -kv[1][1])[:a.top]:
        var = variant(name) or "-"
        short = re.sub(r"\(.*\)$", "", name).replace("fdllm::", "")[:80]
        print(f"| `{short}` | {var} | {calls} | {tns / 1e6:.3f} | {avg / 1e3:.2f} | {100 * tns / tot:.1f}% |")
    for name, (calls, tns, _) in st.items():
        var = variant(name)
        if var:
            by_var[var][0] += calls
            by_var[var][1] += tns
    print("\nBy library variant (the names the launch timer uses):\n")
    print("| variant | calls | total ms | avg us |")
    print("|---|---|---|---|")
    for var, (calls, tns) in sorted(by_var.items(), key=lambda kv: -kv[1][1]):
        print(f"| {var} | {calls} | {tns / 1e6:.3f} | {tns / calls / 1e3:.2f} |")
    return 0


def cmd_traffic(a) -> int:
    cf, cw = counters(a.copy_fetch, "FETCH_SIZE"), counters(a.copy_write, "WRITE_SIZE")
    known_kib = a.copy_mib * 1024.0
    f_fetch = known_kib / copy_kib(cf)
    f_write = known_kib / copy_kib(cw)
    fetch = per_variant(counters(a.fetch, "FETCH_SIZE"))
    write = per_variant(counters(a.write, "WRITE_SIZE"))
    mfma = {}
    if a.mfma:
        util = per_variant(counters(a.mfma, "MfmaUtil"))
        mops = per_variant(counters(a.mfma, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        for var in util:
            # MfmaUtil: percent of SIMD cycles with the matrix core busy, per
            # dispatch; averaged over the variant's dispatches
            mfma[var] = {"mfma_util_pct": round(util[var][1] / util[var][0], 2),
                         "mfma_bf16_issued_flops_per_launch":
                             round(mops[var][1] * 512 / mops[var][0]) if var in mops else None}
    kernels = {}
    for var in sorted(set(fetch) & set(write)):
        n = fetch[var][0]
        fb = fetch[var][1] / n * 1024.0 * f_fetch
        wb = write[var][1] / write[var][0] * 1024.0 * f_write
        kernels[var] = {"launches": n, "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                        "bytes_per_launch": round(fb + wb), **mfma.get(var, {})}
    out = {"source_hash": {f: source_hash(f) for f in SOURCES}, "command": a.cmd, "copy_mib": a.copy_mib,
           "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4), "kernels": kernels}
    text = json.dumps(out, indent=1)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
    print(text)
    return 0


def trace_durations(directory: str) -> list:
    """[(variant, duration_us)] of our dispatches in dispatch order."""
    rows = sorted(_rows(directory, "_kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    out = []
    for r in rows:
        var = variant(r["Kernel_Name"])
        if var:
            out.append((var, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return out


def cmd_sweep(a) -> int:
    """Markdown table of the kernel sweep. The traced run makes, per case,
    buffer_sets warm-up calls and then `reps` timed calls, in the order of the
    JSON; the kernel columns average the trace durations of the timed calls."""
    with open(a.json) as fh:
        res = json.load(fh)
    tr = trace_durations(a.trace)
    attn = [d for v, d in tr if v == "attention"]
    stats = [d for v, d in tr if v == "unmask_stats"]
    sel = [d for v, d in tr if v == "unmask_select"]
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    print("# Attention and logits-in unmask over their sweep shapes\n")
    print("Event-timed figures (per call, launch stream, operand sets rotated so each call reads HBM):\n")
    print(f"    {a.cmd_events}\n")
    print(f"Kernel durations from the trace of the same sweep (the {a.reps} timed calls of each case):\n")
    print(f"    {a.cmd_trace}\n")
    print("## Block attention: batch 8, 32 query rows, 32 heads x 128, bf16\n")
    print("| KV length | algorithmic MB | floor at 8 TB/s (us) | event-timed (us) | GB/s | fraction of HBM peak "
          "| kernel (trace, us) | kernel GB/s | kernel fraction |")
    print("|---|---|---|---|---|---|---|---|---|")
    i = 0
    for r in res.get("attention", []):
        n = r["buffer_sets"] + a.reps
        k = mean(attn[i + r["buffer_sets"]:i + n])
        i += n
        kg = r["bytes"] / k / 1e3
        print(f"| {r['kv_len']} | {r['bytes'] / 1e6:.1f} | {r['floor_us']} | {r['us']} | {r['GBps']} | {r['frac_hbm']} "
              f"| {k:.1f} | {kg:.0f} | {kg / 8000:.3f} |")
    print("\n## Confidence unmask from bf16 logits [8][32][126464]: two launches (chunk statistics, then selection)\n")
    print("Only rows still masked are read; the algorithmic bytes count those rows' logits.\n")
    print("| scale | masked fraction | tau | rows read | algorithmic MB | event-timed (us) | GB/s | fraction of HBM peak "
          "| stats kernel (trace, us) | select kernel (trace, us) | stats kernel fraction |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    i = 0
    for r in res.get("unmask_logits", []):
        n = r["buffer_sets"] + a.reps
        ks, kq = mean(stats[i + r["buffer_sets"]:i + n]), mean(sel[i + r["buffer_sets"]:i + n])
        i += n
        print(f"| {r['scale']} | {r['masked_frac']} | {r['tau']} | {r['rows_read']} | {r['bytes'] / 1e6:.1f} | {r['us']} "
              f"| {r['GBps']} | {r['frac_hbm']} | {ks:.1f} | {kq:.1f} | {r['bytes'] / ks / 1e3 / 8000:.3f} |")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", default="rocprofv3 kernel trace")
    s.add_argument("--cmd", default="")
    s.add_argument("--top", type=int, default=25)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--mfma")
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--cmd", default="")
    t.add_argument("--out")
    w = sub.add_parser("sweep")
    w.add_argument("--json", required=True)
    w.add_argument("--trace", required=True)
    w.add_argument("--reps", type=int, required=True)
    w.add_argument("--cmd-events", default="")
    w.add_argument("--cmd-trace", default="")
    a = ap.parse_args(argv)
    return {"copy": cmd_copy, "stats": cmd_stats, "traffic": cmd_traffic, "sweep": cmd_sweep}[a.cmd_name](a)


if __name__ == "__main__":
    sys.exit(main())
