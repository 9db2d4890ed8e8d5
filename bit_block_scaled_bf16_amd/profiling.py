"""Measurement helpers: summaries of rocprofv3 output for profiles/.

Usage (after the rocprofv3 runs that bench.py's docstring lists):

  python -m bit_block_scaled_bf16_amd.profiling stats  <kernel_stats.csv> <out.md> <command>
  python -m bit_block_scaled_bf16_amd.profiling traffic <fetch_dir> <write_dir> <copy_bytes> \
        <out.md> <command>
  python -m bit_block_scaled_bf16_amd.profiling counters <pmc_dir> <out.md> <command>

`stats` condenses a --kernel-trace --stats CSV into a table of average kernel
durations. `traffic` turns two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB
per dispatch) into bytes per launch, each scaled by what the same counter
reads for a copy-like kernel of known size (torch's elementwise bitwise_not,
which reads and writes the same number of bytes, run by bench.py
--copy-calibration-mib). The traffic summary carries the SHA-256 of
each kernel source it covers; bench.py reports the figure only while the
source is unchanged. `counters` turns one --pmc run of COUNTERS into per-
dispatch clock, MFMA and VALU busy fractions and instructions per wave.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Name fragment of the copy-like calibration kernel (bench.py
# --copy-calibration-mib runs torch.bitwise_not on int32 tensors of that size).
CALIBRATION_KERNEL = "bitwise_not"

# Kernel name fragment -> source file whose hash the traffic figure covers.
KERNEL_SOURCES = {
    "gemm_kernel": "gemm.hip",
    "quantize_kernel": "quantize.hip",
    "amax_flat_kernel": "quantize.hip",
    "amax_tile_kernel": "quantize.hip",
    "rht_amax_mfma_kernel": "quantize.hip",
    "rht_quantize_mfma_kernel": "quantize.hip",
    "mxfp4": "mxfp4.hip",
    "fp8": "fp8.hip",
    "f8f6f4_gemm": "f8f6f4_gemm.hip",
    "fp8_quantize_kernel": "fp8.hip",
    "block_gemm_kernel": "f8f6f4_gemm.hip",
}


def source_hash(fname: str) -> str:
    """SHA-256 of a kernel source together with the library's shared headers
    (csrc/*.h), so that a change to either invalidates its figures."""
    h = hashlib.sha256()
    for name in [fname] + sorted(n for n in os.listdir(CSRC) if n.endswith(".h")):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without namespaces, return type and parameter list."""
    name = name.replace("nvfp4::(anonymous namespace)::", "").replace("nvfp4::", "")
    if name.startswith("void "):
        name = name[5:]
    if "<" in name and name.index("<") < name.find("(") if "(" in name else False:
        return name[: name.index(">") + 1]
    return name.split("(")[0]


def stats_summary(csv_path: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [
        "# Kernel durations (rocprofv3 --kernel-trace --stats)",
        "",
        f"Command: `{command}`",
        "",
        "| kernel | calls | average us | min us | max us | share % |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(
            f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
            f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
            f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(run_dir: str, counter: str):
    path = None
    for root, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                path = os.path.join(root, fn)
    if path is None:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    agg = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        agg[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(d, names[d], agg[d]) for d in sorted(agg)]


# One --pmc pass (6 SQ counters and 1 GRBM counter, within one pass's limits).
COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
            "SQ_INSTS_VALU", "SQ_INSTS_MFMA")
# MI355X: 256 CUs x 4 SIMDs; GRBM_GUI_ACTIVE is summed over the 8 XCDs.
SIMDS = 1024
XCDS = 8


def counters_summary(run_dir: str, out_md: str, command: str) -> None:
    """Per dispatch: duration, average clock (GUI-active cycles / duration),
    the fraction of SIMD-cycles with an MFMA busy, the fraction with a VALU
    instruction active (SQ_ACTIVE_INST_VALU counts in units of 4 cycles, the
    issue time of a wave64 VALU instruction), and VALU / MFMA instructions
    per wave."""
    path = None
    for root, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                path = os.path.join(root, fn)
    if path is None:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    meta = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        agg[d][r["Counter_Name"]] += float(r["Counter_Value"])
        meta[d] = (short_name(r["Kernel_Name"]),
                   (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [
        "# Busy fractions per dispatch (rocprofv3 --pmc)",
        "",
        f"Command: `{command}`",
        "",
        f"Counters (one pass): {' '.join(COUNTERS)}. clock = GRBM_GUI_ACTIVE / {XCDS} / "
        f"duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GUI cycles); "
        f"VALU busy = 4 x SQ_ACTIVE_INST_VALU / ({SIMDS} x GUI cycles). MFMA busy x clock / "
        "2.4 GHz is the share of the chip's dense MFMA peak that the busy cycles represent. "
        "The counters cover a window slightly longer than the dispatch, so clock and busy "
        "fractions of dispatches shorter than about 100 us are approximate (a clock above "
        "2.4 GHz marks them).",
        "",
        "| dispatch | kernel | us | clock GHz | MFMA busy | MFMA busy x clk/2.4 | VALU busy | "
        "VALU inst/wave | MFMA inst/wave |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    result = {
        "command": command,
        "sources": {k: source_hash(v) for k, v in sorted(set(KERNEL_SOURCES.items()))},
        "kernels": {},
    }
    for d in sorted(agg):
        name, us = meta[d]
        if "Fill" in name or "copyBuffer" in name or CALIBRATION_KERNEL in name:
            continue
        c = agg[d]
        gui = c["GRBM_GUI_ACTIVE"] / XCDS
        if gui <= 0 or us <= 0:
            continue
        clk = gui / (us * 1e3)
        mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * gui)
        valu = 4.0 * c["SQ_ACTIVE_INST_VALU"] / (SIMDS * gui)
        waves = max(c["SQ_WAVES"], 1.0)
        lines.append(f"| {d} | `{name}` | {us:.1f} | {clk:.2f} | {mfma:.3f} | {mfma * clk / 2.4:.3f} | "
                     f"{valu:.2f} | {c['SQ_INSTS_VALU'] / waves:.0f} | "
                     f"{c['SQ_INSTS_MFMA'] / waves:.0f} |")
        result["kernels"].setdefault(name, []).append({
            "us": round(us, 1), "clock_ghz": round(clk, 3), "mfma_busy": round(mfma, 4),
            "mfma_peak_share": round(mfma * clk / 2.4, 4), "valu_busy": round(valu, 4),
            "valu_inst_per_wave": round(c["SQ_INSTS_VALU"] / waves, 1),
            "mfma_inst_per_wave": round(c["SQ_INSTS_MFMA"] / waves, 1)})
    lines += ["", "```json", json.dumps(result, indent=1), "```", ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


def traffic_summary(fetch_dir: str, write_dir: str, copy_bytes: int, out_md: str,
                    command: str) -> dict:
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    # the calibration kernel: torch's elementwise bitwise_not over int32, which
    # reads and writes copy_bytes each, like a plain copy
    copy_f = [v for _, n, v in fetch if CALIBRATION_KERNEL in n]
    copy_w = [v for _, n, v in write if CALIBRATION_KERNEL in n]
    kib_f = max(copy_f)
    kib_w = max(copy_w)
    f_read = copy_bytes / (kib_f * 1024.0)
    f_write = copy_bytes / (kib_w * 1024.0)
    per_kernel = collections.defaultdict(lambda: {"fetch": [], "write": []})
    for _, n, v in fetch:
        per_kernel[short_name(n)]["fetch"].append(v * 1024.0 * f_read)
    for _, n, v in write:
        per_kernel[short_name(n)]["write"].append(v * 1024.0 * f_write)
    result = {
        "command": command,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": kib_f,
        "copy_write_kib": kib_w,
        "read_factor": f_read,
        "write_factor": f_write,
        "sources": {k: source_hash(v) for k, v in sorted(set(KERNEL_SOURCES.items()))},
        "kernels": {},
    }
    for name, d in per_kernel.items():
        if not d["fetch"] or not d["write"]:
            continue
        n = min(len(d["fetch"]), len(d["write"]))
        result["kernels"][name] = {
            "dispatches": n,
            "fetch_bytes": [round(x) for x in d["fetch"][:n]],
            "write_bytes": [round(x) for x in d["write"][:n]],
        }
    lines = [
        "# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)",
        "",
        f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`",
        "",
        f"Calibration: a plain copy of {copy_bytes} bytes reads FETCH_SIZE = {kib_f:.0f} KiB and "
        f"WRITE_SIZE = {kib_w:.0f} KiB, so the counters are scaled by {f_read:.3f} (reads) and "
        f"{f_write:.3f} (writes).",
        "",
        "| kernel | dispatch | fetched MB | written MB |",
        "|---|---|---|---|",
    ]
    for name, d in result["kernels"].items():
        for i, (fb, wb) in enumerate(zip(d["fetch_bytes"], d["write_bytes"])):
            lines.append(f"| `{name}` | {i} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    lines += ["", "```json", json.dumps(result, indent=1), "```", ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    return result


def load_traffic(md_path: str):
    """The JSON block of a traffic or counters summary, or None."""
    if not os.path.exists(md_path):
        return None
    text = open(md_path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


def _sources_current(data, source_key) -> bool:
    for key in (source_key,) if isinstance(source_key, str) else source_key:
        src = KERNEL_SOURCES.get(key)
        if src is None or data["sources"].get(key) != source_hash(src):
            return False
    return True


def kernel_counters(md_path: str, kernels, source_key):
    """Busy fractions of one call's kernels from a counters summary: a dict
    short-name fragment -> that dispatch's clock, MFMA / VALU busy and
    instructions per wave. None when the summary is missing, has none of the
    kernels, or the source of source_key changed since it was taken."""
    data = load_traffic(md_path)
    if data is None or not _sources_current(data, source_key):
        return None
    out = {}
    for frag, idx in kernels:
        for name, rows in data["kernels"].items():
            if frag in name and idx < len(rows):
                out[frag.rstrip(",")] = rows[idx]
                break
    return out or None


def kernel_traffic(md_path: str, kernels, source_key):
    """HBM bytes (read + write) of one call: the sum over `kernels`, a list of
    (short-name fragment, dispatch index) pairs, of that dispatch of the
    first kernel whose short name contains the fragment. None when the
    summary is missing, none of the kernels is in it, or the source of
    source_key (one key or a tuple of keys) changed since it was taken."""
    data = load_traffic(md_path)
    if data is None or not _sources_current(data, source_key):
        return None
    total, found = 0, False
    for frag, idx in kernels:
        for name, d in data["kernels"].items():
            if frag in name and idx < d["dispatches"]:
                total += d["fetch_bytes"][idx] + d["write_bytes"][idx]
                found = True
                break
    return total if found else None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "counters":
        counters_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        r = traffic_summary(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6])
        print(json.dumps({k: v for k, v in r.items() if k != "kernels"}, indent=1))
    else:
        raise SystemExit(__doc__)
