"""Turn rocprofv3 CSV output of ``bench.py`` into the short text and JSON
summaries kept under ``profiles/``.

    python -m weights_ttt_layer_amd.profile_summary stats   <rocprof dir> <out.txt> --cmd "<command>"
    python -m weights_ttt_layer_amd.profile_summary traffic <fetch dir> <write dir> <workload> --cmd "<cmd>" --cmd "<cmd>"

``stats`` reads ``*kernel_stats.csv`` (``rocprofv3 --kernel-trace --stats
--output-format csv``) and writes the per-kernel call count and durations of
this library's kernels.

``traffic`` reads two counter runs (``rocprofv3 --pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` over ``bench.py --copy-calibration``). FETCH_SIZE and
WRITE_SIZE are KiB per dispatch of traffic between the L2 and memory. The
calibration step of the bench copies COPY_BYTES with a plain device-to-device
copy kernel; the ratio (known bytes / counted bytes) of that copy scales the
counts of this library's kernels, giving HBM bytes per launch. The record
carries a digest of the kernel sources so that a later change of the kernels
makes the bench report the traffic as unknown rather than stale.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weights_ttt_layer_amd", "csrc")

# plain copy used to calibrate the memory-traffic counters (bench.py --copy-calibration)
COPY_BYTES = 512 * 1024 * 1024
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# kernel sources behind each path; their digest tags a traffic record
KERNEL_SOURCES = {
    "plain": ["smallb_linear.hip", "smallb_common.h", "device_common.h"],
    "ln": ["smallb_chain.hip", "device_common.h"],
    "mlp": ["smallb_mlp.hip", "gelu.h", "smallb_common.h", "device_common.h"],
    "large": ["large_chunk.hip", "device_common.h"],
    "block_before": ["large_chunk.hip", "device_common.h"],
    "block_after": ["large_chunk.hip", "device_common.h"],
    "decode": ["decode.hip", "device_common.h"],
    "layer": ["outer_layer.hip", "smallb_chain.hip", "device_common.h"],
    "backward": ["backward.hip", "device_common.h"],
}

OUR_KERNELS = ("smallb_linear_kernel", "smallb_chain_kernel", "smallb_mlp_kernel", "midb_linear_kernel",
               "mlp_generic_kernel", "lc_gram_kernel", "lc_scan_kernel", "lc_chunk_kernel", "lc_apply_kernel",
               "decode_kernel", "layer_gemm_kernel", "layer_outprep_kernel", "bwd_linear_kernel",
               "bwd_gamma_beta_kernel")

# kernel-name prefixes launched by one call of each path
PATH_KERNELS = {
    "plain": ("smallb_linear_kernel<0,",),
    "ln": ("smallb_chain_kernel<1, 1,",),
    "mlp": ("smallb_mlp_kernel",),
    "large": ("lc_gram_kernel", "lc_scan_kernel", "lc_chunk_kernel"),
    "block_before": ("lc_gram_kernel", "lc_scan_kernel", "lc_apply_kernel<false>"),
    "block_after": ("lc_gram_kernel", "lc_scan_kernel", "lc_apply_kernel<true>"),
    "decode": ("decode_kernel",),
    "layer": ("layer_gemm_kernel", "layer_outprep_kernel", "smallb_chain_kernel<1, 2,"),
    "backward": ("bwd_linear_kernel", "bwd_gamma_beta_kernel"),
}


def source_digest(path_key: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path_key]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(full: str) -> str:
    """'void ttt::(anonymous namespace)::lc_out_kernel<true>(int, ...)' -> 'lc_out_kernel<true>'."""
    s = full.replace("(anonymous namespace)::", "").replace("void ", "").replace("ttt::", "")
    depth, out = 0, []
    for ch in s:
        if ch == "(" and depth == 0:
            break
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        out.append(ch)
    return "".join(out).strip()


def is_ours(name: str) -> bool:
    return any(k in name for k in OUR_KERNELS)


def find_one(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def stats(args):
    path = find_one(args.dir, "*kernel_stats.csv")
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if is_ours(r["Name"]):
                rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]),
                             float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    lines = [f"# rocprofv3 kernel statistics: {args.title or os.path.basename(args.out)}", "",
             "Command (from the repository root):", ""]
    lines += [f"    {c}" for c in args.cmd]
    lines += ["", "| kernel | calls | average us | min us | max us | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for n, c, avg, mn, mx, pct in rows:
        lines.append(f"| {n} | {c} | {avg/1e3:.1f} | {mn/1e3:.1f} | {mx/1e3:.1f} | {pct:.1f} |")
    if args.note:
        lines += ["", args.note]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_counter(d: str, counter: str):
    path = find_one(d, "*counter_collection.csv")
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def traffic(args):
    sys.path.insert(0, ROOT)
    from weights_ttt_layer_amd import workloads as wlm
    from bench import algorithmic_bytes, bwd_algorithmic_bytes, layer_algorithmic

    layers = {w.name: w for w in wlm.LAYER_WORKLOADS}
    if args.workload in layers:
        wl = layers[args.workload]
        path_key = "layer"
        alg = layer_algorithmic(wl)[0]
    else:
        wl = wlm.BY_NAME[args.workload]
        path_key = "large" if wl.b >= 256 else wl.kind
        alg = bwd_algorithmic_bytes(wl) if args.variant == "backward" else algorithmic_bytes(wl)
    if args.variant != "dual":
        path_key = args.variant
    suffix = "" if args.variant == "dual" else f"_{args.variant}"
    fetch = load_counter(args.fetch_dir, "FETCH_SIZE")
    write = load_counter(args.write_dir, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024.0
    # the calibration copies are the copy dispatches that moved about COPY_BYTES
    cf = [v for v in fetch.get(COPY_KERNEL, []) if 0.5 * copy_kib < v < 2.0 * copy_kib]
    cw = [v for v in write.get(COPY_KERNEL, []) if 0.5 * copy_kib < v < 2.0 * copy_kib]
    if not cf or not cw:
        raise SystemExit("no calibration copy found in the counter runs")
    f_fac = copy_kib / (sum(cf) / len(cf))
    w_fac = copy_kib / (sum(cw) / len(cw))
    kernels = {}
    total = 0.0
    for name in sorted(set(fetch) | set(write)):
        if not name.startswith(PATH_KERNELS[path_key]):
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        hbm = (fk * f_fac + wk * w_fac) * 1024.0
        kernels[name] = {"fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
                         "hbm_bytes_per_dispatch": hbm, "dispatches": len(fetch[name])}
        total += hbm
    if not kernels:
        raise SystemExit(f"no dispatch of the {path_key} path's kernels in the counter runs")
    rec = {
        "workload": wl.name,
        "variant": args.variant,
        "kernels": kernels,
        "hbm_bytes_per_launch": total,
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": total / alg,
        "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib_counted": sum(cf) / len(cf),
                        "write_kib_counted": sum(cw) / len(cw), "fetch_factor": f_fac,
                        "write_factor": w_fac},
        "source_digest": source_digest(path_key),
        "commands": args.cmd,
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl.name}{suffix}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic per launch: {wl.name} ({args.variant})", "", "Commands (from the repository root):", ""]
    lines += [f"    {c}" for c in args.cmd]
    lines += ["", f"Calibration: a plain device copy of {COPY_BYTES} bytes counted "
              f"FETCH_SIZE {sum(cf)/len(cf):.0f} KiB and WRITE_SIZE {sum(cw)/len(cw):.0f} KiB "
              f"(expected {copy_kib:.0f} KiB each): factors {f_fac:.4f} and {w_fac:.4f}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (calibrated) |", "|---|---|---|---|"]
    for n, k in kernels.items():
        lines.append(f"| {n} | {k['fetch_kib_per_dispatch']:.0f} | {k['write_kib_per_dispatch']:.0f} | "
                     f"{k['hbm_bytes_per_dispatch']/1e6:.2f} |")
    lines += ["", f"Per launch: {total/1e6:.2f} MB measured vs {alg/1e6:.2f} MB algorithmic "
              f"(ratio {total/alg:.3f}). Source digest {rec['source_digest']}."]
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl.name}{suffix}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def gpu_geometry(d: str):
    """(SIMDs, XCDs) of the GPU agent in a rocprofv3 output directory."""
    path = find_one(d, "*agent_info.csv")
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Agent_Type"] == "GPU":
                return int(r["Simd_Count"]), int(r["Num_Xcc"])
    raise SystemExit(f"no GPU agent in {path}")


def counters(args):
    """Per-kernel matrix-core and issue counters from two --pmc runs.

    The values are device totals per dispatch. GRBM_GUI_ACTIVE is summed over
    the XCDs (so / XCDs = active clock cycles of the dispatch);
    SQ_VALU_MFMA_BUSY_CYCLES is summed over all SIMDs (a 32x32x16 bf16 MFMA
    keeps its SIMD's matrix pipe busy 32 cycles); SQ_INSTS_VALU_MFMA_MOPS_* x 512
    is the executed MFMA flops; SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU and
    SQ_WAIT_INST_ANY count in units of four cycles (one VALU instruction of a
    wave of 64 takes one such unit)."""
    simds, xcds = gpu_geometry(args.mfma_dir)
    keys_m = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
              "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")
    keys_i = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU",
              "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")
    m = {k: load_counter(args.mfma_dir, k) for k in keys_m}
    i = {k: load_counter(args.issue_dir, k) for k in keys_i}
    avg = lambda v: sum(v) / len(v)
    names = [n for n in m["GRBM_GUI_ACTIVE"] if is_ours(n) and n in i["SQ_WAVES"]]
    lines = [f"# Matrix-core and issue counters per kernel: {args.title}", "",
             "Commands (from the repository root):", ""]
    lines += [f"    {c}" for c in args.cmd]
    lines += ["", f"GPU: {simds} SIMDs in {xcds} XCDs. Per dispatch (averaged over dispatches):",
              "cycles = GRBM_GUI_ACTIVE / XCDs; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles);",
              "MFMA TFLOP/s = executed MFMA flops / (cycles / 2.4 GHz) is at the nominal clock;",
              "per wave: VALU and LDS instructions, VALU issue and waiting as fractions of the wave's",
              "cycles, LDS bank-conflict cycles per LDS instruction.", "",
              "| kernel | dispatches | cycles | MFMA instr | MFMA busy | executed MFMA GFLOP | MFMA TFLOP/s | "
              "waves | VALU/wave | LDS/wave | VALU issue | waiting | conflict cyc/LDS |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for n in names:
        cyc = avg(m["GRBM_GUI_ACTIVE"][n]) / xcds
        busy = avg(m["SQ_VALU_MFMA_BUSY_CYCLES"][n]) / (simds * cyc) if cyc else 0.0
        flops = (avg(m["SQ_INSTS_VALU_MFMA_MOPS_BF16"][n]) + avg(m["SQ_INSTS_VALU_MFMA_MOPS_F32"][n])) * 512
        tfs = flops / (cyc / 2.4e9) / 1e12 if cyc else 0.0
        waves = avg(i["SQ_WAVES"][n])
        wc = avg(i["SQ_WAVE_CYCLES"][n])
        lds = avg(i["SQ_INSTS_LDS"][n])
        lines.append(f"| {n} | {len(m['GRBM_GUI_ACTIVE'][n])} | {cyc:.0f} | {avg(m['SQ_INSTS_MFMA'][n]):.3g} | "
                     f"{100 * busy:.1f}% | {flops / 1e9:.2f} | {tfs:.0f} | {waves:.0f} | "
                     f"{avg(i['SQ_INSTS_VALU'][n]) / waves:.0f} | {lds / waves:.0f} | "
                     f"{100 * avg(i['SQ_ACTIVE_INST_VALU'][n]) / wc:.0f}% | "
                     f"{100 * avg(i['SQ_WAIT_INST_ANY'][n]) / wc:.0f}% | "
                     f"{(avg(i['SQ_LDS_BANK_CONFLICT'][n]) / lds if lds else 0):.2f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--cmd", action="append", default=[])
    s.add_argument("--title", default="")
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("workload")
    t.add_argument("--variant", default="dual", choices=sorted(KERNEL_SOURCES.keys() - {"plain", "ln", "mlp", "large"}) + ["dual"])
    t.add_argument("--cmd", action="append", default=[])
    k = sub.add_parser("counters")
    k.add_argument("mfma_dir")
    k.add_argument("issue_dir")
    k.add_argument("out")
    k.add_argument("--title", default="")
    k.add_argument("--cmd", action="append", default=[])
    args = ap.parse_args(argv)
    {"stats": stats, "traffic": traffic, "counters": counters}[args.what](args)


if __name__ == "__main__":
    main()
