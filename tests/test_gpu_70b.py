"""Full-depth parity for the Llama-2/3-70B shape (80 layers, hidden 8192, 64
query heads x 128, 8 KV heads, FFN 28672, vocab 128256; 139 GB of bf16
weights on one GPU): the 4096-token context is prefilled on the GPU
(batched), the oracle starts from a host copy of that cache, re-derives the
cache rows of the last prefilled position from the GPU's rows before it
(every layer and head, within 5e-2 and layer 0 within one bf16 step, as for
the other full-size runs), and one decode step's logits are compared at the
bf16 bar, with the greedy token.

It needs about 140 GB of host memory for the oracle's copy of the weights
and several minutes (weight generation, an fp64 step over 139 GB), so it
runs only when MK_TEST_70B=1 is set; its last result is recorded in the
design notes.  The default GPU suite checks the 70B widths with 2 of the 80
layers (test_gpu_fullsize.py)."""
import os

import numpy as np
import pytest

import synth

from test_gpu_parity import cache_f64, check_layer0_rounding, env, shape_of, to_host  # noqa: F401  (fixture)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("MK_TEST_70B") != "1",
                                 reason="opt-in (MK_TEST_70B=1): ~140 GB of host memory and several minutes")]


def test_llama70b_full_depth_one_step(env):
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["llama70b"]
    shape = shape_of(cfg)
    ctx, seed = cfg.context, 91
    max_seq = ctx + 1
    mk = mkp.MegaKernel(shape, None, max_seq)
    layers = []
    for l in range(cfg.n_layers):  # generate, upload, pre-lay out, keep the host copy for the oracle
        lw = {k: synth.gen_tensor(cfg, seed, k, layer=l) for k in synth.LAYER_KINDS}
        mk.load_weights(mkp.upload_weights({"layers": [lw]}), first_layer=l)
        layers.append(lw)
        if l % 20 == 19:
            print(f"[70b] loaded layer {l + 1}/{cfg.n_layers}", flush=True)
    head = {"embed": synth.gen_tensor(cfg, seed, "embed"), "final_norm": synth.gen_tensor(cfg, seed, "final_norm"),
            "lm_head": synth.gen_tensor(cfg, seed, "lm_head")}
    mk.load_weights(mkp.upload_weights(head))
    torch.cuda.empty_cache()
    kv = mkp.KVCache(shape, max_seq, fill=float("nan"))
    toks = synth.gen_tokens(seed, ctx + 1, cfg.vocab)
    mk.prefill_kv(toks[:ctx], 0, kv)
    logits = torch.full((cfg.vocab,), float("nan"), device="cuda")
    mk.decode_step(int(toks[ctx]), ctx, kv, logits)
    torch.cuda.synchronize()
    assert mk.device_error() == 0
    got = logits.cpu().numpy().astype(np.float64)
    print(f"[70b] GPU prefill of {ctx} positions and one step done", flush=True)
    ref = oracle.Model(shape, dict(head, layers=layers), max_seq)
    gk, gv = to_host(kv.k), to_host(kv.v)
    ref.k[:, :, :ctx] = gk[:, :, :ctx]
    ref.v[:, :, :ctx] = gv[:, :, :ctx]
    mk.close()
    # the batched prefill's rows at the last prefilled position
    p = ctx - 1
    ref.decode_step(int(toks[p]), p, want_logits=False)
    worst = 0.0
    for name, g, r in (("K", gk, ref.k), ("V", gv, ref.v)):
        got_r = cache_f64(oracle, cfg, g[:, :, p])
        want_r = cache_f64(oracle, cfg, r[:, :, p])
        d = float(np.abs(got_r - want_r).max())
        worst = max(worst, d)
        assert d <= 5e-2, f"{name} row {p}: max|d| {d:.3e}"
        check_layer0_rounding(got_r, want_r, f"{name} row {p}")
    ref.k[:, :, p] = gk[:, :, p]
    ref.v[:, :, p] = gv[:, :, p]
    print(f"[70b] prefill rows at position {p}: max|d| {worst:.3e}, layer 0 within one bf16 step", flush=True)
    want = ref.decode_step(int(toks[ctx]), ctx)
    err = float(np.abs(got - want).max())
    top2 = np.sort(np.partition(want, -2)[-2:])
    print(f"[70b] 80 layers, one step at position {ctx}: max|dlogit| {err:.3e}, greedy "
          f"{int(np.argmax(got))} vs oracle {oracle.argmax(want)}, oracle top-2 gap {top2[1] - top2[0]:.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert err <= 2e-2
    assert int(np.argmax(got)) == oracle.argmax(want) or top2[1] - top2[0] <= 2 * err
