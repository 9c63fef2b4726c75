"""mk_decode_step_device_token_noalloc (the step for callers that cannot
allocate device memory) against mk_decode_step_device_token, through the C
ABI: the same kernel with its cross-workgroup records in the library's static
scratch instead of the handle's own buffer, so the logits and the greedy
token must be identical bit for bit.  Two calls in a row on the static
scratch, the second with a smaller model (fewer layers, a narrower hidden
size, so a smaller record buffer over the first call's leftovers), each
checked against the allocating entry point; then a model whose records do
not fit the static scratch is refused with MK_ERR_SCRATCH."""
import numpy as np
import pytest

import synth

from test_gpu_parity import env, shape_of  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _step_both(env, cfg, seed, n_prompt):
    torch, oracle, mkp = env
    shape = shape_of(cfg)
    max_seq = n_prompt + 2
    host = synth.gen_weights(cfg, seed=seed, gains="random")
    mk = mkp.MegaKernel(shape, mkp.upload_weights(host), max_seq)
    info = mk.info()
    print(f"[noalloc] {cfg.name} L={cfg.n_layers} H={cfg.hidden}: record buffer {info['record_bytes']} bytes",
          flush=True)
    assert 0 < info["record_bytes"] <= mkp.mk.MK_STATIC_SCRATCH_BYTES
    toks = synth.gen_tokens(seed, n_prompt + 1, cfg.vocab)
    kv = mkp.KVCache(shape, max_seq)
    mk.prefill_kv(toks[:n_prompt], 0, kv)
    tin = torch.tensor([int(toks[n_prompt])], dtype=torch.int32, device="cuda")
    la = torch.full((cfg.vocab,), float("nan"), device="cuda")
    lb = torch.full((cfg.vocab,), float("nan"), device="cuda")
    ta = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tb = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    # the allocating entry point, then the static-scratch one on the same step
    # (it rewrites the same cache row with the same values)
    mk.decode_step_device_token(tin, n_prompt, kv, la, ta)
    mk.decode_step_device_token_noalloc(tin, n_prompt, kv, lb, tb)
    torch.cuda.synchronize()
    assert mk.device_error() == 0
    assert torch.isfinite(la).all()
    assert torch.equal(la, lb), float((la - lb).abs().max())
    assert int(ta.item()) == int(tb.item()) >= 0
    # and the same result as the oracle's step to the fp32 bar
    ref = oracle.Model(shape, host, max_seq)
    ref.prefill(toks[:n_prompt])
    want = ref.decode_step(int(toks[n_prompt]), n_prompt)
    err = float(np.abs(lb.cpu().numpy().astype(np.float64) - want).max())
    print(f"[noalloc] {cfg.name}: identical to the allocating step; max|dlogit| vs oracle {err:.3e}", flush=True)
    assert err <= 1e-4
    mk.close()


def test_noalloc_matches_allocating_step_twice_then_smaller(env):
    big = synth.CONFIGS["tiny"].with_(n_layers=4, hidden=512, n_heads=8, n_kv_heads=2, ffn=1024)
    small = synth.CONFIGS["tiny"]  # 2 layers, hidden 256: a smaller record buffer
    _step_both(env, big, seed=61, n_prompt=37)
    _step_both(env, small, seed=62, n_prompt=21)


def test_noalloc_refuses_records_beyond_the_static_scratch(env):
    torch, oracle, mkp = env
    # hidden 16384: the down-projection partials alone are 2 x grid x hidden x
    # 8 bytes = 64 MiB at 256 workgroups, beyond the static scratch.  Weights
    # are never loaded: the size check comes first.
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_layers=1, hidden=16384, n_heads=64, n_kv_heads=8,
                                      head_dim=128, ffn=1024, vocab=256, rope_theta=500000.0)
    mk = mkp.MegaKernel(shape_of(cfg), None, 8)
    assert mk.info()["record_bytes"] > mkp.mk.MK_STATIC_SCRATCH_BYTES
    kv = mkp.KVCache(shape_of(cfg), 8)
    tin = torch.zeros(1, dtype=torch.int32, device="cuda")
    tout = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mkp.MkError) as e:
        mk.decode_step_device_token_noalloc(tin, 0, kv, None, tout)
    assert e.value.status == mkp.mk.MK_ERR_SCRATCH
    mk.close()
