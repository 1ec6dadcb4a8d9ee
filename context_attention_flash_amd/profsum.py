"""Summaries of rocprofv3 CSV output for the profiles/ folder.

    python -m context_attention_flash_amd.profsum stats TRACE_kernel_stats.csv \
        --cmd "<the rocprofv3 command>" --title "..." --out profiles/NAME.md
    python -m context_attention_flash_amd.profsum traffic \
        --fetch F_counter_collection.csv --write W_counter_collection.csv \
        --copy-fetch CF_counter_collection.csv --copy-write CW_counter_collection.csv \
        --copy-bytes N --kernel bwd_dkdv_bf16_kernel --cmds "..." --out profiles/NAME.md
    python -m context_attention_flash_amd.profsum mfma M_counter_collection.csv \
        --cmd "..." --title "..." --out profiles/NAME.md

`mfma` turns SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 matrix ops / 512 per
dispatch), SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE into the bf16 flops
each kernel issued per launch, its matrix-core busy fraction and its average
clock, with the same source hash per kernel.

`power` turns samples of `amd-smi metric -p -c` (socket power and the clock
of every XCD), taken while bench.py holds a pass of the workload running back
to back (`--sustain`), into a table per pass.

`traffic` turns the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch, as
rocprofv3 reports them) of one kernel into bytes per launch.  Each counter is
scaled by the factor that maps what it reads for a plain copy kernel of known
size (N bytes read and N bytes written per dispatch) onto N.  The summary
records a hash of the kernel's sources; bench.py reports the traffic only while
that hash still matches the sources in the tree.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel (substring of the dispatched symbol) -> the sources it is built from
KERNEL_SOURCES = {
    "fwd_step_bf16_kernel": ["fwd_bf16.hip", "kernel_common.h", "kernel_args.h"],
    "bwd_dkdv_bf16_kernel": ["bwd_bf16.hip", "kernel_common.h", "kernel_args.h"],
    "bwd_dq_bf16_kernel": ["bwd_bf16.hip", "kernel_common.h", "kernel_args.h"],
    "bwd_dq_ds_bf16_kernel": ["bwd_bf16.hip", "kernel_common.h", "kernel_args.h"],
    "lse_merge_kernel": ["elementwise.hip", "kernel_common.h", "kernel_args.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str, n: int = 70) -> str:
    name = re.sub(r"\(.*\)$", "", name.replace("void ", "", 1)) if name.startswith("void ") else name
    return name if len(name) <= n else name[: n - 3] + "..."


def stats_md(csv_path: str, cmd: str, title: str, top: int = 10) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```", cmd, "```",
           "", "| kernel | calls | total (us) | average (us) | min (us) | max (us) | % of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(csv_path: str, kernel: str, counter: str):
    """Counter value (KiB) of every dispatch whose kernel name contains `kernel`."""
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[int(r["Dispatch_Id"])] = vals.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel!r} in {csv_path}")
    return list(vals.values())


def traffic_md(a) -> str:
    fetch = _per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    write = _per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cf = _per_dispatch(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw = _per_dispatch(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    # the copy kernel moves copy_bytes each way per dispatch; take the median
    # dispatch (the first one may see cold caches)
    f_scale = a.copy_bytes / (statistics.median(cf) * 1024.0)
    w_scale = a.copy_bytes / (statistics.median(cw) * 1024.0)
    fetch_b = statistics.mean(fetch) * 1024.0 * f_scale
    write_b = statistics.mean(write) * 1024.0 * w_scale
    total = fetch_b + write_b
    out = [f"# HBM traffic of `{a.kernel}`: {a.title}", "",
           "Commands (from the repository root, one MI355X; one counter per run):", "", "```",
           *a.cmds.split(" ;; "), "```", "",
           f"- dispatches of the kernel: {len(fetch)} (FETCH_SIZE run), {len(write)} (WRITE_SIZE run)",
           f"- FETCH_SIZE per dispatch: mean {statistics.mean(fetch):.0f} KiB "
           f"(min {min(fetch):.0f}, max {max(fetch):.0f})",
           f"- WRITE_SIZE per dispatch: mean {statistics.mean(write):.0f} KiB "
           f"(min {min(write):.0f}, max {max(write):.0f})",
           f"- copy kernel (`{a.copy_kernel}`, {a.copy_bytes} bytes read and written per dispatch): "
           f"FETCH_SIZE median {statistics.median(cf):.0f} KiB, WRITE_SIZE median "
           f"{statistics.median(cw):.0f} KiB -> scale {f_scale:.4f} (fetch), {w_scale:.4f} (write)",
           f"- scaled bytes per launch: fetch {fetch_b:.4g}, write {write_b:.4g}, total {total:.4g}",
           "", "Machine-readable (bench.py reads these; the hash covers the kernel's sources):", "",
           "```", f"kernel: {a.kernel}", f"kernel_source_sha256_16: {source_hash(a.kernel)}",
           f"fetch_bytes_per_launch: {fetch_b:.6g}", f"write_bytes_per_launch: {write_b:.6g}",
           f"traffic_bytes_per_launch: {total:.6g}", "```"]
    return "\n".join(out) + "\n"


def read_traffic(md_path: str, kernel: str):
    """Traffic bytes per launch from a summary written by `traffic`, or None when
    the file is missing, is for another kernel, or the kernel's sources changed."""
    if not os.path.exists(md_path):
        return None
    kv = {}
    for line in open(md_path):
        m = re.match(r"^([a-z_0-9]+): (\S+)$", line.strip())
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel") != kernel or kv.get("kernel_source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _per_dispatch_all(csv_path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} over every kernel."""
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = vals.get(d, (r["Kernel_Name"], 0.0))
        vals[d] = (name, v + float(r["Counter_Value"]))
    return vals


def mfma_md(csv_path: str, cmd: str, title: str, n_xcd: int = 8, n_simd: int = 1024) -> str:
    mops = _per_dispatch_all(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = _per_dispatch_all(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _per_dispatch_all(csv_path, "GRBM_GUI_ACTIVE")
    ts = {}
    for r in csv.DictReader(open(csv_path)):
        ts[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = [f"# Issued bf16 MFMA work: {title}", "", "Command (from the repository root, one MI355X):",
           "", "```", cmd, "```", "",
           "| kernel | dispatches | issued GFLOP per launch | matrix cores busy | average clock (GHz) |",
           "|---|---|---|---|---|"]
    machine = []
    for kernel in KERNEL_SOURCES:
        ds = [d for d, (name, _) in mops.items() if kernel in name and "(" in name
              and name.split("(")[0].split("<")[0].endswith(kernel)]
        if not ds:
            continue
        fl = statistics.mean(mops[d][1] * 512.0 for d in ds)
        util = statistics.mean(busy[d][1] / (gui[d][1] / n_xcd * n_simd) for d in ds if d in busy and d in gui)
        clk = statistics.mean(gui[d][1] / n_xcd / ts[d] for d in ds if d in gui and ts.get(d))
        out.append(f"| `{kernel}` | {len(ds)} | {fl / 1e9:.1f} | {100 * util:.1f}% | {clk:.2f} |")
        machine += [f"kernel: {kernel}", f"kernel_source_sha256_16: {source_hash(kernel)}",
                    f"issued_flops_per_launch: {fl:.6g}", ""]
    out += ["", "Clock = GRBM_GUI_ACTIVE / 8 XCDs / kernel duration; busy = SQ_VALU_MFMA_BUSY_CYCLES /",
            "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).", "",
            "Machine-readable (bench.py reads these; each hash covers that kernel's sources):", "",
            "```", *machine, "```"]
    return "\n".join(out) + "\n"


# Per-SIMD and per-CU normalisations of the SQ counters (rocprofv3 sums them
# over the shader engines of the chip): 8 XCDs, 256 CUs, 1024 SIMDs.
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def counters_md(csv_paths, kernels, cmds: str, title: str) -> str:
    """Average per dispatch of every counter in the given CSVs (one rocprofv3
    --pmc run each) for each kernel, plus derived fractions."""
    per = {}   # kernel -> counter -> [values per dispatch]
    dur = {}
    for path in csv_paths:
        acc = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            k = next((k for k in kernels if k in name), None)
            if k is None:
                continue
            key = (k, int(r["Dispatch_Id"]), r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
            dur.setdefault(k, {})[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for (k, d, c), v in acc.items():
            per.setdefault(k, {}).setdefault(c, []).append(v)
    out = [f"# SQ counters: {title}", "", "Commands (from the repository root, one MI355X; one run per "
           "counter set):", "", "```", *cmds.split(" ;; "), "```", ""]
    for k in kernels:
        if k not in per:
            continue
        c = {n: statistics.mean(v) for n, v in per[k].items()}
        ndisp = max(len(v) for v in per[k].values())
        out += [f"## `{k}` ({ndisp} dispatches per counter set)", "", "| counter | mean per dispatch |",
                "|---|---|"]
        out += [f"| {n} | {c[n]:.4g} |" for n in sorted(c)]
        gui = c.get("GRBM_GUI_ACTIVE")
        der = []
        if gui:
            cyc = gui / N_XCD   # cycles of one XCD's clock over the dispatch
            ns = statistics.mean(dur[k].values())
            der.append(f"- average clock: {cyc / ns:.2f} GHz (GRBM_GUI_ACTIVE / 8 / duration)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                der.append(f"- matrix cores busy: {100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.1f}% "
                           "of SIMD-cycles")
            if "SQ_LDS_IDX_ACTIVE" in c:
                der.append(f"- LDS busy (indexed access): {100 * c['SQ_LDS_IDX_ACTIVE'] / (cyc * N_CU):.1f}% "
                           "of CU-cycles")
            if "SQ_LDS_BANK_CONFLICT" in c:
                der.append(f"- LDS stalled on bank conflicts: "
                           f"{100 * c['SQ_LDS_BANK_CONFLICT'] / (cyc * N_CU):.1f}% of CU-cycles")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            der.append(f"- VALU issued while the matrix cores were busy: "
                       f"{100 * c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}% of "
                       "their busy cycles")
        wc = c.get("SQ_WAVE_CYCLES")
        if wc:
            for n in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                      "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                      "SQ_WAIT_INST_LDS"):
                if n in c:
                    der.append(f"- {n} / SQ_WAVE_CYCLES: {c[n] / wc:.3f}")
        if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c and c["SQ_INSTS_MFMA"]:
            der.append(f"- VALU instructions per MFMA: {c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f} "
                       "(SQ_INSTS_VALU counts the MFMAs too)")
        if "SQ_INSTS_LDS" in c and c.get("SQ_INSTS_MFMA"):
            der.append(f"- LDS instructions per MFMA: {c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:.2f}")
        if der:
            out += ["", "Derived:", "", *der]
        out.append("")
    return "\n".join(out) + "\n"


def parse_smi_samples(text: str):
    """(socket watts, [GFX clock MHz of each XCD]) of every `amd-smi metric -p
    -c` sample in `text`."""
    out = []
    for chunk in re.split(r"^GPU: \d+\s*$", text, flags=re.M)[1:]:
        pw = re.search(r"SOCKET_POWER:\s*(\d+(?:\.\d+)?)\s*W", chunk)
        clks = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+(?:\.\d+)?)\s*MHz", chunk)]
        if pw and clks:
            out.append((float(pw.group(1)), clks))
    return out


def power_md(files, labels, cmds: str, title: str) -> str:
    lines = [f"# Power and clocks under a sustained load: {title}", "",
             "Commands (from the repository root, one MI355X):", "", "```"]
    lines += [c.strip() for c in cmds.split(" ;; ")]
    lines += ["```", "", "| pass | sample | socket power (W) | XCD clocks (MHz) | mean clock (MHz) |",
              "|---|---|---|---|---|"]
    for path, label in zip(files, labels):
        with open(path) as fh:
            samples = parse_smi_samples(fh.read())
        for i, (w, clks) in enumerate(samples):
            lines.append(f"| {label} | {i} | {w:.0f} | {', '.join(f'{c:.0f}' for c in clks)} | "
                         f"{statistics.mean(clks):.0f} |")
    lines.append("")
    return "\n".join(lines)


def read_issued(md_path: str, kernel: str):
    """Issued bf16 MFMA flops per launch of `kernel` from a summary written by
    `mfma`, or None when missing or the kernel's sources changed."""
    if not os.path.exists(md_path):
        return None
    cur = {}
    for line in open(md_path):
        m = re.match(r"^([a-z_0-9]+): (\S+)$", line.strip())
        if not m:
            continue
        if m.group(1) == "kernel":
            cur = {"kernel": m.group(2)}
        else:
            cur[m.group(1)] = m.group(2)
        if cur.get("kernel") == kernel and "issued_flops_per_launch" in cur:
            if cur.get("kernel_source_sha256_16") != source_hash(kernel):
                return None
            return float(cur["issued_flops_per_launch"])
    return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("csv")
    mf.add_argument("--cmd", required=True)
    mf.add_argument("--title", required=True)
    mf.add_argument("--out", required=True)
    cn = sub.add_parser("counters")
    cn.add_argument("csv", nargs="+")
    cn.add_argument("--kernels", required=True, help="comma-separated kernel name substrings")
    cn.add_argument("--title", required=True)
    cn.add_argument("--cmds", required=True, help="the commands, separated by ' ;; '")
    cn.add_argument("--out", required=True)
    pw = sub.add_parser("power")
    pw.add_argument("files", nargs="+", help="amd-smi outputs, one per pass")
    pw.add_argument("--labels", required=True, help="comma-separated pass names")
    pw.add_argument("--title", required=True)
    pw.add_argument("--cmds", required=True, help="the commands, separated by ' ;; '")
    pw.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="elementwise_kernel")
    t.add_argument("--kernel", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--cmds", required=True, help="the commands, separated by ' ;; '")
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.mode == "stats":
        text = stats_md(a.csv, a.cmd, a.title)
    elif a.mode == "mfma":
        text = mfma_md(a.csv, a.cmd, a.title)
    elif a.mode == "counters":
        text = counters_md(a.csv, a.kernels.split(","), a.cmds, a.title)
    elif a.mode == "power":
        text = power_md(a.files, a.labels.split(","), a.cmds, a.title)
    else:
        text = traffic_md(a)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    sys.exit(main())
