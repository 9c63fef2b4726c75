"""Summarise rocprofv3 output of bench.py runs into text the repository keeps.

    python -m transformer_megakernel_persistent_amd.profile_counters \
        --workload llama1b --fetch DIR --write DIR --trace DIR --command-* "..."

Inputs are the CSV directories of three rocprofv3 runs of the same bench
command: one `--pmc FETCH_SIZE`, one `--pmc WRITE_SIZE` (the counters need
separate passes), one `--kernel-trace --stats`.  bench.py was run with
`--copy-calibration BYTES`, so each counter run also holds three
device-to-device copies of a known size; the ratio of the copy's known bytes
to its counter reading scales the decode kernel's reading to bytes.

Writes profiles/counters_<workload>.json (read back by bench.py for the
`roofline.traffic` field, only while its kernel_hash matches the sources) and
profiles/<kernel>_<workload>.md (the figures and the commands).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_TAG = "mk_decode_kernel"


def _rows(directory: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    out = []
    for pth in paths:
        with open(pth, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _template_args(name: str):
    a, b = name.find("<"), name.find(">")
    return [x.strip() for x in name[a + 1:b].split(",")] if 0 <= a < b else []


def _is_decode(name: str) -> bool:
    # the token-producing instantiation: its fourth template argument (LOGITS)
    # is true; decode launches that fill the cache have false
    args = _template_args(name)
    return DECODE_TAG in name and len(args) >= 4 and args[3] == "true"


def _is_copy(name: str) -> bool:
    n = name.lower()
    return "copy" in n and DECODE_TAG not in n and "prelayout" not in n


def counter_per_dispatch(directory: str, counter: str):
    """(mean KiB per decode dispatch, median KiB per calibration copy, n_decode, n_copy, copy kernel name)."""
    per_dispatch = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name = r.get("Kernel_Name", "")
        per_dispatch.setdefault(key, [name, 0.0])
        per_dispatch[key][1] += float(r["Counter_Value"])
    dec = [v for n, v in per_dispatch.values() if _is_decode(n)]
    # the calibration copies are the last three copy dispatches of the run
    # (earlier ones are the runtime's small staging copies)
    ids = sorted((int(k), n, v) for k, (n, v) in per_dispatch.items() if _is_copy(n))
    cpy = [(n, v) for _, n, v in ids[-3:]]
    if not dec or not cpy:
        names = sorted({n for n, _ in per_dispatch.values()})
        raise RuntimeError(f"{counter}: found {len(dec)} decode and {len(cpy)} copy dispatches in {directory}; "
                           f"kernels seen: {names}")
    return statistics.mean(dec), statistics.median(v for _, v in cpy), len(dec), len(cpy), cpy[0][0]


def kernel_stats(directory: str):
    rows = _rows(directory, "kernel_stats.csv")
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                    "total_ms": float(r["TotalDurationNs"]) / 1e6, "pct": float(r["Percentage"])})
    return sorted(out, key=lambda x: -x["total_ms"])


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", default=None, help="CSV directory of the --pmc FETCH_SIZE run")
    ap.add_argument("--write", default=None, help="CSV directory of the --pmc WRITE_SIZE run")
    ap.add_argument("--trace", required=True, help="CSV directory of the --kernel-trace --stats run")
    ap.add_argument("--copy-bytes", type=int, required=True, help="bytes of each calibration copy")
    ap.add_argument("--command-fetch", default=None)
    ap.add_argument("--command-write", default=None)
    ap.add_argument("--command-trace", required=True)
    ap.add_argument("--bench-json", default=None, help="the JSON line the traced bench run printed")
    ap.add_argument("--dram", default=None, help="CSV directory of a --pmc TCC_EA0_RDREQ_DRAM_sum run (optional)")
    ap.add_argument("--command-dram", default=None)
    ap.add_argument("--note", default=None, help="a line for the summary (e.g. why a counter pass is missing)")
    args = ap.parse_args(argv)
    if (args.fetch is None) != (args.write is None):
        ap.error("--fetch and --write go together")

    sys.path.insert(0, ROOT)
    import synth
    from bench import kernel_hash

    stats = kernel_stats(args.trace)
    dec = [s for s in stats if _is_decode(s["name"])]
    cfg = synth.CONFIGS[args.workload]
    bench = json.loads(args.bench_json) if args.bench_json else None
    pos0 = bench["config"]["decode_positions"][0] if bench else cfg.context
    alg = cfg.step_bytes(pos0)
    rec = None
    if args.fetch:
        f_dec, f_cpy, n_f, n_fc, copy_name = counter_per_dispatch(args.fetch, "FETCH_SIZE")
        w_dec, w_cpy, n_w, n_wc, _ = counter_per_dispatch(args.write, "WRITE_SIZE")
        kib = args.copy_bytes / 1024.0
        f_scale, w_scale = kib / f_cpy, kib / w_cpy
        fetch_b = f_dec * f_scale * 1024.0
        write_b = w_dec * w_scale * 1024.0
        rec = {"workload": args.workload, "kernel_hash": kernel_hash(), "kernel": DECODE_TAG + "<..., LOGITS=true>",
               "hbm_bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b,
               "write_bytes_per_launch": write_b, "fetch_kib_raw": f_dec, "write_kib_raw": w_dec,
               "copy_bytes": args.copy_bytes, "copy_fetch_kib_raw": f_cpy, "copy_write_kib_raw": w_cpy,
               "fetch_scale": f_scale, "write_scale": w_scale, "decode_dispatches": [n_f, n_w],
               "algorithmic_bytes_per_launch": alg, "commands": {"fetch": args.command_fetch,
                                                                 "write": args.command_write}}
        if args.dram:
            # read requests the memory-side caches passed on to DRAM, summed over
            # the L2 channels, scaled by the same counter's reading for the copy
            d_dec, d_cpy, n_d, n_dc, _ = counter_per_dispatch(args.dram, "TCC_EA0_RDREQ_DRAM_sum")
            rec["dram_read_requests_per_launch"] = d_dec
            rec["dram_read_requests_per_copy"] = d_cpy
            rec["dram_read_bytes_per_launch_scaled"] = d_dec * (args.copy_bytes / d_cpy) if d_cpy else None
            rec["commands"]["dram"] = args.command_dram
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if rec is not None:
        with open(os.path.join(ROOT, "profiles", f"counters_{args.workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")

    lines = [f"# {DECODE_TAG} on {args.workload}", "",
             f"Kernel sources hash: `{kernel_hash()}`", "",
             "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{args.command_trace}`", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for s in stats[:8]:
        nm = s["name"] if len(s["name"]) < 90 else s["name"][:87] + "..."
        lines.append(f"| `{nm}` | {s['calls']} | {s['avg_us']:.2f} | {s['min_us']:.2f} | {s['max_us']:.2f} | "
                     f"{s['total_ms']:.2f} | {s['pct']:.2f} |")
    if dec:
        lines += ["", f"Decode kernel (token-producing instantiation): {dec[0]['calls']} calls, "
                      f"average {dec[0]['avg_us']:.2f} us; algorithmic bytes at position {pos0}: {alg} "
                      f"-> {alg / (dec[0]['avg_us'] * 1e-6) / 1e9:.1f} GB/s."]
    if bench:
        lines += ["", f"The traced bench run printed: value {bench['value']:.1f} tokens/s, mean event-timed step "
                      f"{bench['us_per_token_mean']:.2f} us, roofline.achieved {bench['roofline']['achieved']:.1f} GB/s."]
    if args.note:
        lines += ["", args.note]
    if rec is None:
        out_md = os.path.join(ROOT, "profiles", f"{DECODE_TAG}_{args.workload}.md")
        with open(out_md, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(json.dumps({"counters": None, "md": out_md}))
        return
    lines += ["", "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
              f"FETCH_SIZE command: `{args.command_fetch}`", "",
              f"WRITE_SIZE command: `{args.command_write}`", "",
              f"Calibration: a device-to-device copy (`{copy_name}`) of {args.copy_bytes} bytes reads FETCH_SIZE "
              f"{f_cpy:.0f} KiB and WRITE_SIZE {w_cpy:.0f} KiB per dispatch (median of {n_fc}/{n_wc}), against "
              f"{kib:.0f} KiB moved each way: scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
              "| per decode launch | raw KiB | scaled bytes |", "|---|---|---|",
              f"| FETCH_SIZE | {f_dec:.0f} | {fetch_b:.4g} |", f"| WRITE_SIZE | {w_dec:.0f} | {write_b:.4g} |",
              f"| total | | {fetch_b + write_b:.4g} |", "",
              f"Algorithmic bytes per launch (every weight once + K/V rows of positions 0..{pos0}): {alg:.4g}; "
              f"measured / algorithmic = {(fetch_b + write_b) / alg:.3f}.", ""]
    if args.dram:
        lines += ["## DRAM read requests (rocprofv3 --pmc TCC_EA0_RDREQ_DRAM_sum)", "",
                  f"Command: `{args.command_dram}`", "",
                  f"Per decode launch {rec['dram_read_requests_per_launch']:.4g} requests; per calibration copy "
                  f"{rec['dram_read_requests_per_copy']:.4g}; scaled by the copy's {args.copy_bytes} bytes: "
                  f"{rec['dram_read_bytes_per_launch_scaled']:.4g} bytes read from DRAM per launch "
                  f"({rec['dram_read_bytes_per_launch_scaled'] / alg:.3f} x the algorithmic bytes).", ""]
    out_md = os.path.join(ROOT, "profiles", f"{DECODE_TAG}_{args.workload}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"counters": rec["hbm_bytes_per_launch"], "md": out_md}))


if __name__ == "__main__":
    main()
