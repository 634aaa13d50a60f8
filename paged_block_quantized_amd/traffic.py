"""HBM traffic of one decode step (paged_attn_decode_append: the current
token's store and the attention), from rocprofv3 counters.

Two steps, each a command of its own:

``python -m paged_block_quantized_amd.traffic run --workload W``
    the program to profile: sets up workload W, makes ``--calls`` decode
    steps cycling through ``--rotate`` copies of the pool (as bench.py times
    them), then ``--copies`` passes of a plain elementwise kernel that reads
    1 GiB and writes 1 GiB (bitwise not of a uint8 tensor; a torch copy_
    would go to the DMA engine, which the counters do not see).  Run it
    under ``rocprofv3 --pmc FETCH_SIZE`` and, separately, under
    ``rocprofv3 --pmc WRITE_SIZE`` (CSV output).

``python -m paged_block_quantized_amd.traffic summarize --workload W
  --fetch DIR --write DIR --out profiles/traffic_W.json``
    reads the two counter_collection CSV files, takes the median counter per
    dispatch of the step's kernels (partition, reduce, and the store kernel
    where the step launches it; the last --calls dispatches) and of the
    calibration kernel, scales each counter by (known bytes / calibration
    counter), and writes bytes per decode call with the hash of the kernel
    source.

The counters are read in KiB per dispatch; the copy calibration makes the
unit question moot because the same factor converts both.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
DECODE_KERNELS = ("attn_partition_", "attn_reduce", "quantize_store")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("paged_attn.hip", "quantize_store.hip", "store_tile.h", "device_common.h"):
        with open(os.path.join(ROOT, "paged_block_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run(args):
    import torch

    sys.path.insert(0, ROOT)
    from paged_block_quantized_amd import runner, workloads as W

    w = W.WORKLOADS[args.workload]
    if w.q_len:   # a multi-query workload: its calls re-read one pool
        setup = runner.setup_multi(w)
        for _ in range(args.calls):
            setup.run()
    elif w.store_only:   # quantize-and-store of every prompt, the same call repeated
        setup = runner.setup_prefill_store(w)
        for _ in range(args.calls):
            setup.run()
    else:
        setup = runner.setup_decode(w)
        if args.rotate > 1:
            setup.add_replicas(args.rotate - 1)
        for i in range(args.calls):
            setup.step(r=i % max(1, args.rotate))
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.copies):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(f"traffic run: {args.calls} decode calls ({w.name}), {args.copies} copies of "
          f"{COPY_BYTES} B", flush=True)


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_kernel(rows, counter):
    """{kernel name: [(dispatch id, counter value)]} in dispatch order (values
    summed over the dimensions rocprofv3 reports for one dispatch)."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], int(r.get("Dispatch_Id") or r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, did), v in sorted(per.items(), key=lambda kv: kv[0][1]):
        out.setdefault(name, []).append((did, v))
    return out


def _copy_kernel(per):
    """The calibration kernel (reads and writes COPY_BYTES)."""
    cands = [n for n in per if "bitwise_not" in n]
    if len(cands) != 1:
        raise SystemExit("calibration kernel not found among: " + ", ".join(per))
    return cands[0]


def _step_kernels(per, calls):
    """{kernel: median counter per step} over the dispatches of the steps:
    those from the first partition-kernel dispatch on (the pool is built by
    store dispatches alone; a step may hold several partition kernels), or
    for a store-only workload its last `calls` store dispatches."""
    parts = [d for n, v in per.items() if "attn_partition_" in n for d, _ in v]
    if parts:
        if len(parts) < calls:
            raise SystemExit("fewer partition-kernel dispatches than steps")
        first = min(parts)
    else:   # a store-only workload: its last `calls` store dispatches
        stores = sorted(d for n, v in per.items() if "quantize_store" in n for d, _ in v)
        if len(stores) < calls:
            raise SystemExit("fewer store dispatches than calls")
        first = stores[-calls]
    out = {}
    for n, v in per.items():
        if any(k in n for k in DECODE_KERNELS):
            vals = [x for d, x in v if d >= first]
            if vals:
                out[n] = statistics.median(vals)
    return out


def summarize(args):
    res = {"workload": args.workload, "kernel_hash": kernel_source_hash()}
    total = 0.0
    for counter, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        known = COPY_BYTES
        per = _per_kernel(_counter_rows(d), counter)
        ck = _copy_kernel(per)
        copy_val = statistics.median(x for _, x in per[ck])
        scale = known / copy_val
        dec = _step_kernels(per, args.calls)
        if not dec:
            raise SystemExit("decode kernels not found")
        dec_bytes = sum(v * scale for v in dec.values())
        total += dec_bytes
        res[counter] = {
            "copy_kernel": ck, "copy_counter_per_dispatch": copy_val, "known_copy_bytes": known,
            "scale_bytes_per_unit": scale,
            "decode_kernels_counter_median": dec,
            "bytes_per_decode": round(dec_bytes),
        }
    res["bytes_per_decode"] = round(total)
    if args.algorithmic:
        res["algorithmic_bytes_per_decode"] = args.algorithmic
        res["traffic_over_algorithmic"] = round(total / args.algorithmic, 4)
    with open(args.out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="llama7b")
    r.add_argument("--calls", type=int, default=8)
    r.add_argument("--rotate", type=int, default=4)
    r.add_argument("--copies", type=int, default=3)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", default="llama7b")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--algorithmic", type=int, default=0)
    s.add_argument("--calls", type=int, default=8)
    args = ap.parse_args()
    (run if args.cmd == "run" else summarize)(args)


if __name__ == "__main__":
    main()
