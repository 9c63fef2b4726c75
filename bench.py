"""Decode benchmark: batch-1 greedy decoding through the persistent megakernel.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama1b]

A step is one decode step of the whole path (embedding -> all layers ->
LM head -> greedy argmax), launched as ONE kernel through the C ABI
(mk_decode_step_device_token): each launch reads the token the previous
launch wrote, so the timed loop runs with no host round trip.  The headline
workload is the Llama-3.2-1B-shaped decoder with a 2048-token context and
128 greedy steps; weights are seeded N(0, 0.02) bf16 (synthetic, random
init) and the context is filled by mk_prefill_kv from seeded token ids.
The Llama-3-8B shape (2048-token context), the 1B shape at a 32768-token
context, and the 1B and 8B shapes with weight-only INT8 matrices (int8 codes
with per-row fp32 scales, bf16 cache) are measured in the same run and
reported under `extra_workloads`.

Each workload is timed in `--runs` (3) runs of K steps; the median run gives
`value` (tokens/s, wall clock, inputs resident in HBM) and the roofline
figure, p50/P99 pool the steps of every run.  Prints ONE JSON line.
`roofline` divides the algorithmic bytes of a step (every weight once + the
K/V rows read at that position) by the average kernel duration measured
with events on the launch stream; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
SHAPE_KEYS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "rms_eps", "rope_theta",
              "dtype", "tied")
KERNEL_SOURCES = ("transformer_megakernel_persistent_amd/csrc/mk_kernel.hip",
                  "transformer_megakernel_persistent_amd/csrc/mk_prelayout.hip",
                  "transformer_megakernel_persistent_amd/csrc/mk_internal.h")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


HOST_ORACLE_MAX_BYTES = 40e9


def load_model(mkp, synth, cfg, shape, max_seq, tuning, seed, dev, keep_host):
    """A handle made by mk_create_deferred; each layer is generated on the
    host, uploaded, pre-laid out by mk_load_weights and freed, so the device
    never holds more than one layer twice (an 80-layer hidden-8192 model
    would not fit twice).  Returns the handle and, if keep_host, the host
    weights (for the oracle baseline)."""
    mk = mkp.MegaKernel(shape, None, max_seq, tuning=tuning)
    host_layers = []
    for l in range(cfg.n_layers):
        lw = synth.gen_layer(cfg, seed, l)  # (with the per-row scales of an INT8 model)
        part = mkp.upload_weights({"layers": [lw]}, dev)
        mk.load_weights(part, first_layer=l)
        del part
        if keep_host:
            host_layers.append(lw)
        if l % 16 == 15:
            print(f"[bench] loaded layer {l + 1}/{cfg.n_layers}", file=sys.stderr, flush=True)
    head = {"embed": synth.gen_tensor(cfg, seed, "embed"), "final_norm": synth.gen_tensor(cfg, seed, "final_norm")}
    if not cfg.tied:
        head["lm_head"] = synth.gen_tensor(cfg, seed, "lm_head")
        if cfg.dtype == "w8":
            head["lm_head_scale"] = synth.gen_scale(cfg, seed, "lm_head")
    part = mkp.upload_weights(head, dev)
    mk.load_weights(part)
    del part
    if not keep_host:
        return mk, None
    head["layers"] = host_layers
    return mk, head


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    k = (len(xs) - 1) * q
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def cpu_baseline(cfg, host_w, shape, budget_s: float):
    """The oracle (plain float64 C) on this host: decode steps of the same
    model at the same context length, from a synthetic cache, until the
    time budget is used (at least one step)."""
    import numpy as np

    import oracle
    import synth
    ctx = cfg.context
    ref = oracle.Model(shape, host_w, ctx + 65)
    for l in range(cfg.n_layers):
        ref.k[l, :, :ctx] = synth.gen_kv_prefix(cfg, 7, ctx, "k", l)
        ref.v[l, :, :ctx] = synth.gen_kv_prefix(cfg, 7, ctx, "v", l)
    tok, n, t0 = 1, 0, time.perf_counter()
    while True:
        lg = ref.decode_step(tok, ctx + n)
        tok = int(np.argmax(lg))
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 64:
            break
    cores = oracle.num_threads()
    # one more step on a single thread (the same code; its row loops serial)
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    ref.decode_step(tok, ctx + n)
    el1 = time.perf_counter() - t1
    oracle.set_num_threads(cores)
    return {"value": n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} greedy decode steps of the same model from a synthetic {ctx}-token cache "
                      f"(positions {ctx}..{ctx + n - 1}), {el:.1f} s, float64; one more step on 1 thread "
                      f"took {el1:.1f} s",
            "value_1_thread": 1.0 / el1}


PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def prefill_record(cfg, n, seconds, info):
    """Prefill throughput and its roofline: the algorithmic flops of n
    prompt positions (2 per weight of every layer matrix per token, plus the
    causal attention's 4 * n_heads * head_dim per (token, earlier position)
    pair per layer) over the wall time, against the bf16 matrix-core peak."""
    H, F = cfg.hidden, cfg.ffn
    per_layer = (cfg.q_dim + 2 * cfg.kv_dim) * H + H * cfg.q_dim + 3 * H * F
    flops = 2.0 * cfg.n_layers * per_layer * n + 4.0 * cfg.n_layers * cfg.q_dim * n * (n + 1) / 2
    tf = flops / seconds / 1e12
    rec = {"positions": n, "seconds": seconds, "tokens_per_s": n / seconds,
           "mode": f"batched, chunks of up to {info['prefill_chunk']} positions" if info["prefill_chunk"] else "decode launches",
           "warmup": "one untimed 16-token prefill first" if info["prefill_chunk"] else "none",
           "roofline": None}
    if info["prefill_chunk"]:  # the matrix-core path; decode launches are the decode step's own roofline
        rec["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tf / PEAK_MFMA_BF16_TFLOPS, "traffic": None, "flops": flops}
    return rec


def measure(name, args, dev, steps, warm, runs, cpu_budget, with_cpu):
    """One workload: load, prefill, `warm` untimed steps, then `runs` timed
    runs of `steps` chained device-token steps each.  Returns its record."""
    import torch

    import synth
    import transformer_megakernel_persistent_amd as mkp

    cfg = synth.CONFIGS[name]
    shape = {k: v for k, v in dataclasses.asdict(cfg).items() if k in SHAPE_KEYS}
    ctx = cfg.context
    max_seq = ctx + warm + runs * steps
    tuning = {"grid": args.grid, "ring_slots": args.ring, "attn_splits": args.splits,
              "cooperative": 1 if args.launch == "cooperative" else 2,
              "prefetch_depth": args.prefetch_depth, "stage_drain": 1 if args.stage_drain else 0,
              "prefill_chunk": args.prefill_chunk, "attn_pm_slots": args.attn_pm_slots,
              "slots_per_step": args.slots_per_step}
    # The oracle baseline needs every weight in host memory; past this size it
    # is not taken (the weights are streamed to the device a layer at a time).
    keep_host = with_cpu and cfg.weight_bytes_per_step() <= HOST_ORACLE_MAX_BYTES
    t = time.perf_counter()
    mk, host_w = load_model(mkp, synth, cfg, shape, max_seq, tuning, args.seed, dev, keep_host)
    print(f"[bench] {cfg.name}: weights generated and loaded in {time.perf_counter() - t:.1f}s", file=sys.stderr,
          flush=True)
    torch.cuda.empty_cache()
    info = mk.info()
    kv = mkp.KVCache(shape, max_seq, dev)
    prompt = synth.gen_tokens(args.seed, ctx + 1, cfg.vocab)
    if info["prefill_chunk"]:
        # one short prefill first, untimed (the first launch of each prefill
        # kernel loads its code); the timed prefill rewrites these rows
        mk.prefill_kv(prompt[:min(ctx, 16)], 0, kv)
    torch.cuda.synchronize()
    t = time.perf_counter()
    mk.prefill_kv(prompt[:ctx], 0, kv)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    print(f"[bench] {cfg.name}: prefill of {ctx} positions: {prefill_s:.2f}s", file=sys.stderr, flush=True)
    if mk.device_error() != 0:
        raise RuntimeError("device error during prefill")

    stream = torch.cuda.current_stream()
    n_tok = warm + runs * steps
    tok = torch.tensor([int(prompt[ctx])], dtype=torch.int32, device=dev)
    toks_out = torch.empty(n_tok, dtype=torch.int32, device=dev)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)

    def step(i):  # launch i of the chain: position ctx + i, token from launch i - 1
        src = toks_out[i - 1:i] if i > 0 else tok
        mk.decode_step_device_token(src, ctx + i, kv, logits, toks_out[i:i + 1], stream)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    run_recs = []
    for r in range(runs):
        i0 = warm + r * steps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(steps):
            step(i0 + i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_us = [ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(steps)]
        run_recs.append({"wall": wall, "step_us": step_us, "pos0": ctx + i0})
    if mk.device_error() != 0:
        raise RuntimeError("device error during the timed steps")
    tokens = toks_out[warm:].cpu().numpy()
    mk.close()
    del kv
    torch.cuda.empty_cache()

    # the median run (by wall time) carries the figures; p50/P99 pool every step
    order = sorted(range(runs), key=lambda r: run_recs[r]["wall"])
    med = run_recs[order[runs // 2]]
    all_us = [u for rr in run_recs for u in rr["step_us"]]
    p50, p99 = percentile(all_us, 0.5), percentile(all_us, 0.99)
    mean_us = sum(med["step_us"]) / steps
    bytes_per_step = [cfg.step_bytes(med["pos0"] + i) for i in range(steps)]
    mean_bytes = sum(bytes_per_step) / len(bytes_per_step)
    achieved = mean_bytes / (mean_us * 1e-6) / 1e9
    gbs_p50 = cfg.step_bytes(med["pos0"] + steps // 2) / (p50 * 1e-6) / 1e9
    traffic = traffic_from_profile(cfg.name)

    cpu = None
    if host_w is not None:
        cpu = cpu_baseline(cfg, host_w, shape, cpu_budget)
    return {
        "workload": f"{cfg.name}: {cfg.n_layers}L hidden {cfg.hidden}, {cfg.n_heads}q/{cfg.n_kv_heads}kv heads x "
                    f"{cfg.head_dim}, SwiGLU {cfg.ffn}, vocab {cfg.vocab}{' tied' if cfg.tied else ''}, "
                    f"{cfg.dtype} weights+KV, fp32 accumulate; {ctx}-token context, {steps} greedy steps per run, "
                    f"batch 1",
        "name": cfg.name,
        "value": steps / med["wall"],
        "runs_tokens_per_s": [steps / rr["wall"] for rr in run_recs],
        "ms_per_step": med["wall"] * 1000.0 / steps,
        "us_per_token_p50": p50,
        "us_per_token_p99": p99,
        "us_per_token_mean": mean_us,
        "gbs_p50": gbs_p50,
        "bytes_per_step": mean_bytes,
        "decode_positions": [ctx + warm, ctx + n_tok - 1],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
        "prefill": prefill_record(cfg, ctx, prefill_s, info),
        "info": info,
        "first_tokens": [int(x) for x in tokens[:8]],
        "dtype": {"bf16": "bf16", "f32": "f32", "w8": "int8 weights x bf16 activations, fp32 accumulate"}[cfg.dtype],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps per run (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--runs", type=int, default=3, help="timed runs; the median run is reported")
    ap.add_argument("--config", default="llama1b", help="the headline workload")
    ap.add_argument("--extra", default=None,
                    help="comma-separated further workloads reported in the same line (default with the llama1b "
                         "headline: llama8b,llama1b_32k; otherwise none)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--ring", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefetch-depth", type=int, default=0,
                    help="slots the loads run ahead (default: ring slots - 1); an ablation knob")
    ap.add_argument("--stage-drain", action="store_true",
                    help="ablation: no loads for a stage before its grid dependency is met")
    ap.add_argument("--prefill-chunk", type=int, default=0,
                    help="tokens per batched-prefill chunk (default 4096, or the context if smaller); -1: one decode launch per position")
    ap.add_argument("--slots-per-step", type=int, default=0,
                    help="16 KiB ring slots per data step, the stream's tile (default 1); a tunable")
    ap.add_argument("--attn-pm-slots", type=int, default=0,
                    help="position-major attention when a split holds at least this many KV slots "
                         "(default 0: always head-major)")
    ap.add_argument("--launch", choices=["cooperative", "ordinary"], default="ordinary",
                    help="cooperative launch (co-residency checked by the runtime) or an ordinary launch")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the run, copy BYTES device-to-device three times (a plain copy kernel of known "
                         "size, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU tensor-parallel design is described but not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if args.extra is None:
        extra = ["llama8b", "llama1b_32k", "llama1b_w8", "llama8b_w8"] if args.config == "llama1b" else []
    else:
        extra = [x for x in args.extra.split(",") if x]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    with_cpu = not args.no_cpu_baseline
    cfg = synth.CONFIGS[args.config]
    steps = args.steps if args.steps is not None else cfg.decode_steps
    head = measure(args.config, args, dev, steps, args.warmup, args.runs, args.cpu_budget, with_cpu)
    extras = []
    for name in extra:
        c = synth.CONFIGS[name]
        n = args.steps if args.steps is not None else c.decode_steps
        rec = measure(name, args, dev, n, args.warmup, args.runs, min(args.cpu_budget, 10.0), with_cpu)
        extras.append({k: rec[k] for k in ("name", "workload", "value", "runs_tokens_per_s", "ms_per_step",
                                           "us_per_token_p50", "us_per_token_p99", "us_per_token_mean", "gbs_p50",
                                           "bytes_per_step", "decode_positions", "roofline", "cpu_baseline",
                                           "prefill", "first_tokens", "dtype")} | {"unit": "tokens/s", "steps": n})
    info = head["info"]
    out = {
        "metric": "batch-1 decode tokens/s (us/token p50/P99) + achieved HBM GB/s vs peak",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic: seeded N(0,0.02) random-init weights, uniform random prompt tokens, greedy decode",
        "config": {
            "workload": head["workload"],
            "context": cfg.context, "global_batch": 1, "decode_positions": head["decode_positions"],
            "runs": args.runs, "launches_per_token": 1, "grid": info["grid"], "ring_slots": info["ring_slots"],
            "prefetch_slots": info["prefetch_slots"], "slots_per_step": info["slots_per_step"],
            "stage_drain": bool(args.stage_drain),
            "attn_splits": info["attn_splits"], "block_threads": info["block_threads"],
            "lds_bytes": info["lds_bytes"], "launch": args.launch, "parallelism": "single GPU"},
        "runs_tokens_per_s": head["runs_tokens_per_s"],
        "us_per_token_p50": head["us_per_token_p50"],
        "us_per_token_p99": head["us_per_token_p99"],
        "us_per_token_mean": head["us_per_token_mean"],
        "gbs_p50": head["gbs_p50"],
        "bytes_per_step": head["bytes_per_step"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "prefill": head["prefill"],
        "extra_workloads": extras,
        "kernel_hash": kernel_hash(),
        "first_tokens": head["first_tokens"],
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 3}), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
