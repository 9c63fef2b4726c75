"""Stage timeline of one decode step, from the kernel's own trace.

    python -m transformer_megakernel_persistent_amd.stage_timeline llama1b [llama70b:6 ...]
        [--prefetch-depth D] [--stage-drain]

A workload name may carry ':N' to keep only its first N layers.  The handle is
created with tuning trace=1 (mk_read_trace), weights are seeded synthetic
(loaded a layer at a time), the cache holds synthetic values up to the
workload's context, and a few decode steps run; the last one is summarised:

  - per stage kind (QKV, attention, O, gate/up, down), averaged over the
    inner layers and taking the median workgroup: the boundary epilogue, the
    wait for the stage's cross-workgroup inputs, loading them, and the data
    steps (the stage's weight or cache slots);
  - the skew of the workgroups at the end of each layer's feed-forward
    stages against the median, grouped by XCD (workgroup w runs on XCD
    w mod 8 under an ordinary launch);
  - consumer 0's arithmetic time and barrier interval for each data step of
    layer 1.

Times are wall-clock ticks of the device (100 MHz) converted to us.  Tracing
adds a few percent to the step.
"""
from __future__ import annotations

import argparse
import dataclasses
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

from .mk import KVCache, MegaKernel, upload_weights  # noqa: E402

SHAPE_KEYS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "rms_eps", "rope_theta",
              "dtype", "tied")
STAGES = ("QKV", "attn", "O", "GU", "down")
TICK_US = 0.01


def load(cfg, shape, max_seq, tuning):
    mk = MegaKernel(shape, None, max_seq, tuning=tuning)
    for l in range(cfg.n_layers):
        lw = synth.gen_layer(cfg, 0, l)  # (with the per-row scales of an INT8 model)
        mk.load_weights(upload_weights({"layers": [lw]}), first_layer=l)
    head = {"embed": synth.gen_tensor(cfg, 0, "embed"), "final_norm": synth.gen_tensor(cfg, 0, "final_norm")}
    if not cfg.tied:
        head["lm_head"] = synth.gen_tensor(cfg, 0, "lm_head")
        if cfg.dtype == "w8":
            head["lm_head_scale"] = synth.gen_scale(cfg, 0, "lm_head")
    mk.load_weights(upload_weights(head))
    return mk


def summarise(name: str, tuning: dict, steps: int = 6) -> None:
    base, _, nl = name.partition(":")
    cfg = synth.CONFIGS[base]
    if nl:
        cfg = cfg.with_(n_layers=int(nl))
    shape = {k: v for k, v in dataclasses.asdict(cfg).items() if k in SHAPE_KEYS}
    ctx = cfg.context
    max_seq = ctx + steps
    mk = load(cfg, shape, max_seq, dict(tuning, trace=1))
    kv = KVCache(shape, max_seq, fill=None)
    std = synth.kv_std(cfg)
    kv.k.normal_(0.0, std)
    kv.v.normal_(0.0, std)
    logits = torch.empty(cfg.vocab, device="cuda")
    wall = []
    for i in range(steps):
        torch.cuda.synchronize()
        t = time.perf_counter()
        mk.decode_step(1 + i, ctx + i, kv, logits)
        torch.cuda.synchronize()
        wall.append(time.perf_counter() - t)
    if mk.device_error() != 0:
        raise RuntimeError("device error")
    tr = mk.read_trace().astype(np.int64)  # [grid][5L+2][4]
    L, G = cfg.n_layers, tr.shape[0]
    inner = range(1, L - 1) if L > 2 else range(L)
    print(f"== {name}: traced step {np.median(wall) * 1e6:.0f} us (wall, median of {steps})")
    for k, st in enumerate(STAGES):
        parts = np.zeros(4)
        for l in inner:
            b = 5 * l + k
            parts += [np.median(tr[:, b, e + 1] - tr[:, b, e]) for e in range(3)] + \
                     [np.median(tr[:, b + 1, 0] - tr[:, b, 3])]
        parts *= TICK_US / len(inner)
        print(f"  {st:5s} epilogue {parts[0]:7.2f}  wait {parts[1]:7.2f}  load {parts[2]:6.2f}  "
              f"data {parts[3]:7.2f}  total {parts.sum():7.2f} us")
    starts = [np.median(tr[:, 5 * l, 0]) for l in range(L + 1)] + [np.median(tr[:, 5 * L + 1, 0])]
    print(f"  per layer {np.mean(np.diff(starts[:L + 1])) * TICK_US:.2f} us; LM head "
          f"{(starts[L + 1] - starts[L]) * TICK_US:.2f} us")
    if L > 2:
        ends = np.stack([tr[:, 5 * l, 0] - np.median(tr[:, 5 * l, 0]) for l in range(2, L + 1)], 1) * TICK_US
        print(f"  feed-forward end vs median: per-layer max {ends.max(0).mean():.2f} us")
        print("  by XCD (mean, max): " + ", ".join(f"{x}: {ends[x::8].mean():+.2f}/{ends[x::8].max():.2f}"
                                                for x in range(min(8, G))))
    st_ = mk.last_steps.astype(np.int64)
    n = int((st_[0, :, 0] > 0).sum())
    if n > 1:
        comp = np.median(st_[:, :n, 1] - st_[:, :n, 0], 0) * TICK_US
        intv = np.median(np.diff(st_[:, :n, 0], axis=1), 0) * TICK_US
        print("  layer-1 data steps, arithmetic / barrier interval (us): " +
              " ".join(f"{a:.2f}/{b:.2f}" for a, b in zip(comp[:-1], intv)))
    ld = mk.last_loader.astype(np.int64)
    m = int((ld[0, :, 0] > 0).sum())
    if m > 1:
        # loader 0 at the barriers of layer 1: time spent waiting in the
        # barrier (arrival to exit) and the interval between its exits.  A
        # short wait means the loader arrives last (the loads pace the step).
        wait = np.median(ld[:, :m, 1] - ld[:, :m, 0], 0) * TICK_US
        gap = np.median(np.diff(ld[:, :m, 1], axis=1), 0) * TICK_US
        print("  layer-1 loader barriers, wait / interval (us): " +
              " ".join(f"{a:.2f}/{b:.2f}" for a, b in zip(wait[:-1], gap)))
    mk.close()


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--prefetch-depth", type=int, default=0)
    ap.add_argument("--stage-drain", action="store_true")
    args = ap.parse_args(argv)
    tuning = {"prefetch_depth": args.prefetch_depth, "stage_drain": int(args.stage_drain)}
    for name in args.workloads:
        summarise(name, tuning)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
