"""Measurement helpers: HBM traffic of one kernel from rocprofv3 counters.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report KiB per
dispatch as the memory side sees them.  Their scale is calibrated against a
plain device-to-device copy of known size run in the same process (bench.py
``--copy-calibration``: 256 MiB read and 256 MiB written by the runtime's copy
kernel), so traffic = FETCH_SIZE / (copy FETCH_SIZE / copy bytes) + the same for
WRITE_SIZE.  A measurement is tied to a digest of the kernel's sources and
build flags; bench.py reports it only while the digest still matches.

    python -m linear_attention_sequence_kda_amd.profiling traffic \\
        --fetch <dir of the FETCH_SIZE pass> --write <dir of the WRITE_SIZE pass> \\
        --kernel kda_inter_scalar_kernel --workload <name> --out profiles/traffic.json
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")

COPY_BYTES = 256 << 20          # bench.py --copy-calibration: one 256 MiB copy
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# sources whose change changes the kernel's memory traffic
KERNEL_SOURCES = {
    "kda_intra_kernel": ["kda_intra.hip", "kda_rev_record.h"],
    "kda_inter_kernel": ["kda_inter.hip"],
    "kda_inter_scalar_kernel": ["kda_inter_scalar.hip"],
    "kda_inter_wide_kernel": ["kda_inter_wide.hip"],
    "kda_inter_quad_kernel": ["kda_inter_wide.hip"],
    "kda_decode_kernel": ["kda_decode.hip"],
    "kda_bwd_kernel": ["kda_bwd.hip"],
    # chunkwise gradients: the gradient kernel and the wide state pass in its
    # scan forms (forward, reverse), which rocprofv3 lists as
    # kda_inter_wide_kernel instances (traffic --match); the reverse records
    # are built by the intra-chunk kernel's gradient form
    "kda_chunk_grad_kernel": ["kda_chunk_bwd.hip"],
    "kda_inter_wide_scan": ["kda_inter_wide.hip"],
    "kda_inter_wide_scan_rev": ["kda_inter_wide.hip"],
}
COMMON_SOURCES = ["kda_device.h", "kda_internal.h"]
# the prefill kernels' launch shapes (spans, column slices) are set by the ABI layer
PREFILL_HOST = ["kda_api.cpp"]


def source_digest(kernel: str) -> str:
    """sha256 over the kernel's source files, the shared headers and build.py."""
    h = hashlib.sha256()
    names = KERNEL_SOURCES[kernel] + COMMON_SOURCES
    if kernel != "kda_decode_kernel":
        names = names + PREFILL_HOST
    files = [os.path.join(CSRC, f) for f in names]
    files.append(os.path.join(PKG, "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(pass_dir: str) -> List[dict]:
    paths = glob.glob(os.path.join(pass_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no *counter_collection.csv under {pass_dir}")
    rows: List[dict] = []
    for p in paths:
        with open(p, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def per_dispatch_kib(pass_dir: str, counter: str, match: str, also: str = "",
                     first: int = 0, last: int = -1) -> List[float]:
    """Counter value (KiB) of every dispatch whose kernel name contains `match`
    (and `also`), with a dispatch id in [first, last] (last < 0: no bound)."""
    vals: Dict[str, float] = {}
    for r in _rows(pass_dir):
        d = int(r["Dispatch_Id"])
        if d < first or (last >= 0 and d > last):
            continue
        if r["Counter_Name"] == counter and match in r["Kernel_Name"] and also in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def first_dispatch(pass_dir: str, match: str, also: str = "") -> int:
    """Dispatch id of the first dispatch whose kernel name contains `match` and `also`."""
    ids = [int(r["Dispatch_Id"]) for r in _rows(pass_dir)
           if match in r["Kernel_Name"] and also in r["Kernel_Name"]]
    if not ids:
        raise ValueError(f"no dispatch of {match} {also} under {pass_dir}")
    return min(ids)


def traffic(fetch_dir: str, write_dir: str, kernel: str, also: str = "",
            window=((0, -1), (0, -1))) -> dict:
    """HBM bytes per dispatch of `kernel` (every dispatch whose name contains
    `kernel` and `also`: one template instance when a run launches several;
    `window`: the dispatch-id ranges of the fetch and the write pass, one leg
    of a run that launches the same instance in several legs)."""
    fk = per_dispatch_kib(fetch_dir, "FETCH_SIZE", kernel, also, *window[0])
    wk = per_dispatch_kib(write_dir, "WRITE_SIZE", kernel, also, *window[1])
    fc = per_dispatch_kib(fetch_dir, "FETCH_SIZE", COPY_KERNEL)
    wc = per_dispatch_kib(write_dir, "WRITE_SIZE", COPY_KERNEL)
    if not fk or not wk:
        raise ValueError(f"no dispatch of {kernel} in the counter files")
    if not fc or not wc:
        raise ValueError("no calibration copy in the counter files (run bench.py with "
                         "--copy-calibration)")
    # the calibration copy is the first copy of the run (later copies are the
    # benchmark's own, e.g. restoring a decode state)
    f_factor = fc[0] * 1024.0 / COPY_BYTES   # counter bytes per real byte read
    w_factor = wc[0] * 1024.0 / COPY_BYTES
    fetch = sum(fk) / len(fk) * 1024.0 / f_factor
    write = sum(wk) / len(wk) * 1024.0 / w_factor
    return {"fetch_bytes": fetch, "write_bytes": write, "bytes": fetch + write,
            "fetch_kib_per_dispatch": sum(fk) / len(fk),
            "write_kib_per_dispatch": sum(wk) / len(wk),
            "dispatches": len(fk), "copy_fetch_factor": f_factor,
            "copy_write_factor": w_factor}


# MFMA-busy pass: one rocprofv3 run with these counters (all in the SQ and
# GRBM blocks, within one pass's limits)
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
SIMDS = 256 * 4   # MI355X: 256 CUs x 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the 8 XCDs


def mfma(pass_dir: str, kernel: str) -> List[dict]:
    """MFMA utilisation of one kernel's dispatches, grouped by template
    instance and grid size (one group per workload and instance): the MFMA
    pipes' busy cycles summed over all SIMDs /
    (the GPU's active cycles x SIMDs), and the bf16 and fp32 MFMA flops the SQ
    counted (MOPS x 512).  rocprofv3 gives one row per dispatch and counter;
    GRBM_GUI_ACTIVE is the sum of the XCDs' counts, so one XCD's active
    cycles are that / 8."""
    disp: Dict[str, dict] = {}
    for r in _rows(pass_dir):
        if kernel not in r["Kernel_Name"]:
            continue
        d = disp.setdefault(r["Dispatch_Id"], {"grid": int(r["Grid_Size"]), "name": r["Kernel_Name"],
                                                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    groups: Dict[tuple, List[dict]] = {}
    for d in disp.values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("GRBM_GUI_ACTIVE", 0) > 0:
            groups.setdefault((d["grid"], d["name"]), []).append(d)
    if not groups:
        raise ValueError(f"no dispatch of {kernel} with MFMA counters under {pass_dir}")
    out = []
    for (grid, name), ds in sorted(groups.items()):
        n = len(ds)
        avg = lambda key: sum(d.get(key, 0.0) for d in ds) / n
        util = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
                   for d in ds) / n
        out.append({"kernel": kernel, "instance": name, "grid_size": grid, "dispatches": n,
                    "avg_dispatch_us": avg("ns") / 1e3,
                    "mfma_busy_cycles": avg("SQ_VALU_MFMA_BUSY_CYCLES"),
                    "gui_active_cycles_per_xcd": avg("GRBM_GUI_ACTIVE") / XCDS,
                    "mfma_util": util,
                    "bf16_mfma_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512,
                    "f32_mfma_flops": avg("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512})
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True, help="directory of the MFMA counter pass")
    m.add_argument("--kernel", required=True, action="append")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--also", default="", help="a further substring of the kernel name "
                   "(one template instance, e.g. Lb1ELb1E for the KDA intra-chunk kernel "
                   "writing MFMA-order records)")
    t.add_argument("--match", default="", help="the kernel name to look for in the counter "
                   "files when it differs from --kernel (the scan forms of the wide state pass)")
    t.add_argument("--from-kernel", default="", help="count only dispatches from the first "
                   "dispatch of this kernel-name substring on (a later leg of the run)")
    t.add_argument("--until-kernel", default="", help="count only dispatches before the "
                   "first dispatch of this kernel-name substring (an earlier leg)")
    a = ap.parse_args()
    if a.cmd == "mfma":
        for k in a.kernel:
            for rec in mfma(a.pmc, k):
                print(json.dumps(rec))
        return
    win = []
    for d in (a.fetch, a.write):
        lo = first_dispatch(d, *a.from_kernel.split("+", 1)) if a.from_kernel else 0
        hi = first_dispatch(d, *a.until_kernel.split("+", 1)) - 1 if a.until_kernel else -1
        win.append((lo, hi))
    rec = traffic(a.fetch, a.write, a.match or a.kernel, a.also, tuple(win))
    rec["source_sha256"] = source_digest(a.kernel)
    data = {}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            data = json.load(fh)
    data[f"{a.kernel}|{a.workload}"] = rec
    with open(a.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
