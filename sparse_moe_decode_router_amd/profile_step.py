"""Drive and summarise hardware-counter runs of the decode step.

``run``: a short program for rocprofv3 to wrap: eager steps of one workload
(rotating inputs), then a plain f32 copy of known size (``--copy-mib``), the
calibration dispatch that says what FETCH_SIZE and WRITE_SIZE read for a
known number of bytes moved; with ``--read-mb``, read-only reference launches
(torch's sum) of given sizes.

``summarize``: reads the counter CSVs of two rocprofv3 runs (one with
FETCH_SIZE, one with WRITE_SIZE), scales each kernel's mean per-dispatch
reading by the copy's ratio of counter to bytes, and writes
``profiles/traffic.json`` (per workload and kernel symbol: HBM bytes per
launch, tied to the device sources by their digest).

``busy``: per-kernel means of an SQ / GRBM counter run and the MFMA and
VALU utilisation they imply.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- \\
        python3 -m sparse_moe_decode_router_amd.profile_step run --workload k3_b1
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- \\
        python3 -m sparse_moe_decode_router_amd.profile_step run --workload k3_b1
    python3 -m sparse_moe_decode_router_amd.profile_step summarize \\
        --workload k3_b1 --fetch OUT/fetch --write OUT/write
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# name -> (layer recipe, batch, top_k, seed)
WORKLOADS = {
    "k3_b1": ("k3", 1, 16, 0),
    "k3_zipf_b8": ("k3_zipf", 8, 16, 0),
    "k3_flat_b64": ("k3_flat", 64, 16, 0),
    "k3_b64": ("k3", 64, 16, 0),
    "k3_tp8_b1": ("k3_tp8", 1, 16, 1000),
    "k3_tp8_b8": ("k3_tp8", 8, 16, 1000),
    "k3_tp8_b64": ("k3_tp8", 64, 16, 1000),
}
MODES = ("four_launches", "late_routing", "dense_routing", "ordered", "side_stream", "two_launches",
         "fused")
COPY_KERNEL = "elementwise"  # torch's kernel for the calibration copy


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def run(args) -> None:
    import numpy as np
    import torch

    from . import binding, synth

    recipe_name, B, k, seed = WORKLOADS[args.workload]
    recipe = synth.RECIPES[recipe_name]
    log(f"[profile] generating {args.workload}")
    layer = synth.make_layer(recipe, seed)
    torch.cuda.set_device(0)
    dev = binding.DeviceLayer(layer)
    ctx = binding.MoEDecode(dev, B, k)
    mode = "fused" if args.fused else args.mode
    ctx.set_mode({"four_launches": binding.MODE_FOUR_LAUNCHES,
                  "late_routing": binding.MODE_LATE_ROUTING,
                  "dense_routing": binding.MODE_DENSE_ROUTING,
                  "ordered": binding.MODE_ORDERED,
                  "side_stream": binding.MODE_SIDE_STREAM,
                  "two_launches": binding.MODE_TWO_LAUNCHES, "fused": binding.MODE_FUSED}[mode])
    xs = [torch.from_numpy(synth.make_tokens(layer.dims, seed, B, draw=r).view(np.int16)).cuda()
          for r in range(args.rotate)]
    out = torch.empty((B, layer.dims.hidden), dtype=torch.int16, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((B, k), dtype=torch.float32, device="cuda")
    for i in range(args.steps):
        ctx.step(xs[i % args.rotate], k, out, idx, wts)
    torch.cuda.synchronize()
    log(f"[profile] {args.steps} steps done; dispatch {ctx.last_dispatch()}")
    assert ctx.read_flags() == 0
    n = args.copy_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.copies):
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_mib MiB
    torch.cuda.synchronize()
    log(f"[profile] calibration copy: {args.copies} x {args.copy_mib} MiB")
    # Read-only reference launches: torch's sum over buffers of the given
    # sizes (MB), e.g. the bytes of one launch of the step, so that a
    # kernel trace shows what one plain streaming launch of that size takes.
    for mb in args.read_mb:
        buf = torch.ones(int(mb * 1e6) // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(args.copies):
            buf.sum()
        torch.cuda.synchronize()
        log(f"[profile] read reference: {args.copies} x {mb} MB")
        del buf
    ctx.close()


def read_counters(d: str, counter: str):
    """kernel name -> list of per-dispatch values (KiB) of `counter`."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = defaultdict(lambda: defaultdict(float))
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if not row["Counter_Name"].startswith(counter):
                    continue
                key = (fn, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[row["Kernel_Name"]][key] += float(row["Counter_Value"])
    return {name: list(v.values()) for name, v in per.items()}


def symbol_of(kernel_name: str):
    m = re.search(r"moe::(k_\w+)", kernel_name)
    return m.group(1) if m else None


def summarize(args) -> None:
    from .build import source_digest

    fetch = read_counters(args.fetch, "FETCH_SIZE")
    write = read_counters(args.write, "WRITE_SIZE")
    copy_bytes = args.copy_mib * (1 << 20)

    def copy_ratio(c):
        vals = [v for name, vs in c.items() if COPY_KERNEL in name for v in vs]
        big = [v for v in vals if v * 1024 > copy_bytes / 2]
        if not big:
            raise SystemExit("calibration copy not found in the counters")
        return (sum(big) / len(big)) * 1024 / copy_bytes

    rf, rw = copy_ratio(fetch), copy_ratio(write)
    entry = {}
    for name in sorted(set(fetch) | set(write)):
        sym = symbol_of(name)
        if sym is None:
            continue
        f = fetch.get(name, [])
        w = write.get(name, [])
        fb = (sum(f) / len(f)) * 1024 / rf if f else 0.0
        wb = (sum(w) / len(w)) * 1024 / rw if w else 0.0
        e = entry.setdefault(sym, {"kernels": [], "fetch_bytes": 0.0, "write_bytes": 0.0,
                                   "dispatches": 0})
        e["kernels"].append(name)
        e["fetch_bytes"] += fb
        e["write_bytes"] += wb
        e["dispatches"] = max(e["dispatches"], len(f), len(w))
    digest = source_digest()
    for sym, e in entry.items():
        e["fetch_bytes"] = int(e["fetch_bytes"])
        e["write_bytes"] = int(e["write_bytes"])
        e["bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
        e["source_digest"] = digest
    path = os.path.join(ROOT, "profiles", "traffic.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    table[args.workload] = entry
    table["calibration"] = {"copy_mib": args.copy_mib, "fetch_kib_per_kib_moved": round(rf, 4),
                            "write_kib_per_kib_moved": round(rw, 4)}
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps({"workload": args.workload, "calibration": table["calibration"],
                      "kernels": {s: e["bytes_per_launch"] for s, e in entry.items()}}))


def busy(args) -> None:
    """Per-kernel means of the SQ / GRBM counters of one rocprofv3 --pmc run
    (directory args.dir), with the utilisations they imply, by rocprofv3's
    own derived-counter formulas (MfmaUtil, VALUBusy) on MI355X (8 XCDs, 256
    compute units, 1024 SIMDs):
      mfma_util = sum SQ_VALU_MFMA_BUSY_CYCLES / (GUI x 1024),
      valu_busy = sum SQ_ACTIVE_INST_VALU / 256 / GUI,
    where GUI is the busiest XCD's GRBM_GUI_ACTIVE (the CSV holds the sum over
    the 8 XCDs, each active for the whole dispatch: GUI = sum / 8); printed as
    one JSON line."""
    files = glob.glob(os.path.join(args.dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {args.dir}")
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                sym = symbol_of(row["Kernel_Name"])
                if sym is None:
                    continue
                key = (fn, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[row["Kernel_Name"]][row["Counter_Name"]][key] += float(row["Counter_Value"])
    out = {}
    for name, counters in per.items():
        mean = {c: sum(v.values()) / len(v) for c, v in counters.items()}
        e = {"dispatches": max(len(v) for v in counters.values()), "mean": mean}
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui:
            gui /= args.xcds
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                e["mfma_util"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * args.cus * 4), 4)
            if "SQ_ACTIVE_INST_VALU" in mean:
                e["valu_busy"] = round(mean["SQ_ACTIVE_INST_VALU"] / args.cus / gui, 4)
            if "SQ_INSTS_MFMA" in mean and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                e["mfma_cycles_per_inst"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                  max(1.0, mean["SQ_INSTS_MFMA"]), 2)
        out[name] = e
    print(json.dumps({"dir": args.dir, "kernels": out}))


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="k3_b1", choices=sorted(WORKLOADS))
    r.add_argument("--steps", type=int, default=16)
    r.add_argument("--rotate", type=int, default=8)
    r.add_argument("--fused", action="store_true", help="the one-launch mode (same as --mode fused)")
    r.add_argument("--mode", default="four_launches", choices=MODES)
    r.add_argument("--copy-mib", type=int, default=512)
    r.add_argument("--copies", type=int, default=3)
    r.add_argument("--read-mb", type=float, nargs="*", default=[],
                   help="sizes (MB) of read-only reference launches (torch sum)")
    s = sub.add_parser("summarize")
    s.add_argument("--workload", default="k3_b1", choices=sorted(WORKLOADS))
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-mib", type=int, default=512)
    b = sub.add_parser("busy")
    b.add_argument("--dir", required=True)
    b.add_argument("--cus", type=int, default=256)
    b.add_argument("--xcds", type=int, default=8)
    args = ap.parse_args()
    if args.cmd == "run":
        run(args)
    elif args.cmd == "busy":
        busy(args)
    else:
        summarize(args)


if __name__ == "__main__":
    main()
