"""GPU parity: the HIP megakernel through the C ABI vs the CPU oracle, on the
same seeded inputs.  Bars: max|dlogit| <= 1e-4 for float32 weights, <= 2e-2
for bfloat16 weights, and greedy (teacher-forced) agreement on every step."""
import dataclasses

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

SHAPE_KEYS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "rms_eps", "rope_theta",
              "dtype", "tied")


def shape_of(cfg):
    d = dataclasses.asdict(cfg)
    return {k: d[k] for k in SHAPE_KEYS}


def tol_of(cfg):
    return 1e-4 if cfg.dtype == "f32" else 2e-2


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    import transformer_megakernel_persistent_amd as mkp
    mkp.load_library()
    return torch, oracle, mkp


def to_host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def cache_f64(oracle, cfg, a):
    """Cache contents (float32, or bfloat16 bits) as float64."""
    return a.astype(np.float64) if cfg.dtype == "f32" else oracle.f64_array_from_bf16(a)


def bf16_step(a):
    """Spacing of bfloat16 values at magnitude a (float64 array): 2^(e-7) for
    a in [2^e, 2^(e+1)), the subnormal spacing below the normal range."""
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_layer0_rounding(got, want, name):
    """Layer 0's cache rows depend on the token's embedding and the layer's
    weights only (no earlier row, no earlier layer), so both sides round the
    same real value to bfloat16 and may differ by at most one rounding step
    (fp32 against fp64 arithmetic only moves a value across a rounding
    boundary).  Deeper layers read earlier rows and layers, where a single
    flipped rounding propagates; they are held to the absolute bar.  The
    1e-4 floor covers entries near zero, where the sum cancels and fp32's
    absolute error (a few 1e-6 over 2048 products of size 0.02) exceeds the
    bf16 step at the entry's own magnitude."""
    g0, w0 = got[0], want[0]
    bad = np.abs(g0 - w0) > bf16_step(np.maximum(np.abs(g0), np.abs(w0))) + 1e-4
    assert not bad.any(), f"{name}: {int(bad.sum())} layer-0 entries more than one bf16 step apart"


def put_kv_prefix(cfg, seed, n_pos, ref, kv):
    """Same synthetic cache contents for positions [0, n_pos) on both sides."""
    import torch
    for l in range(cfg.n_layers):
        for which, host, dev in (("k", ref.k, kv.k), ("v", ref.v, kv.v)):
            a = synth.gen_kv_prefix(cfg, seed, n_pos, which, l)
            host[l, :, :n_pos, :] = a
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else \
                torch.from_numpy(a)
            dev[l, :, :n_pos, :] = t.to(dev.device)


def create_deferred(mkp, shape, host, max_seq, tuning=None, order=None):
    """A handle made by mk_create_deferred, its weights uploaded and loaded
    one layer at a time (in `order`), the head weights last."""
    mk = mkp.MegaKernel(shape, None, max_seq, tuning=tuning)
    for l in (order if order is not None else range(shape["n_layers"])):
        part = mkp.upload_weights({"layers": [host["layers"][l]]})
        mk.load_weights(part, first_layer=l)
        del part
    head = mkp.upload_weights({k: v for k, v in host.items() if k != "layers"})
    mk.load_weights(head)
    del head
    return mk


def run_pair(env, cfg, seed, n_prompt, n_steps, gains="random", tuning=None, use_prefill=True, poison=True,
             check_kv=True, deferred=False, expect_batched=None):
    """Prefill (or synthetic cache) then teacher-forced greedy steps on both
    sides; returns per-step max|dlogit| and the argmax agreement count."""
    torch, oracle, mkp = env
    print(f"[parity] {cfg.name} dtype={cfg.dtype} prompt={n_prompt} steps={n_steps} seed={seed} tuning={tuning}",
          flush=True)
    shape = shape_of(cfg)
    max_seq = n_prompt + n_steps
    host = synth.gen_weights(cfg, seed=seed, gains=gains)
    ref = oracle.Model(shape, host, max_seq)
    if deferred:
        mk = create_deferred(mkp, shape, host, max_seq, tuning)
    else:
        dev_w = mkp.upload_weights(host)
        mk = mkp.MegaKernel(shape, dev_w, max_seq, tuning=tuning)
        del dev_w
    if expect_batched is not None:  # which prefill path the handle takes
        assert (mk.info()["prefill_chunk"] > 0) == expect_batched, mk.info()
    kv = mkp.KVCache(shape, max_seq, fill=float("nan") if poison else 0.0)
    toks = synth.gen_tokens(seed, n_prompt + 1, cfg.vocab)
    if use_prefill:
        ref.prefill(toks[:n_prompt])
        mk.prefill_kv(toks[:n_prompt], 0, kv)
        torch.cuda.synchronize()
        assert mk.device_error() == 0
        if check_kv and n_prompt:
            for name, dev_c, host_c in (("K", kv.k, ref.k), ("V", kv.v, ref.v)):
                got = cache_f64(oracle, cfg, to_host(dev_c)[:, :, :n_prompt])
                want = cache_f64(oracle, cfg, host_c[:, :, :n_prompt])
                assert np.isfinite(got).all()
                kv_err = float(np.abs(got - want).max())
                print(f"[parity] prefilled {name} max|d| = {kv_err:.3e}", flush=True)
                assert kv_err <= (1e-4 if cfg.dtype == "f32" else 5e-2)
                if cfg.dtype != "f32":  # a bf16 cache (bf16 or int8 weights)
                    check_layer0_rounding(got, want, name)
    else:
        put_kv_prefix(cfg, seed + 100, n_prompt, ref, kv)
    logits = torch.empty(cfg.vocab, device="cuda")
    errs, agree = [], 0
    tok = int(toks[n_prompt])
    for s in range(n_steps):
        pos = n_prompt + s
        want = ref.decode_step(tok, pos)
        logits.fill_(float("nan"))
        mk.decode_step(tok, pos, kv, logits)
        torch.cuda.synchronize()
        assert mk.device_error() == 0
        got = logits.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        errs.append(float(np.abs(got - want).max()))
        nxt = oracle.argmax(want)
        agree += int(int(np.argmax(got)) == nxt)
        tok = nxt  # teacher forcing with the oracle's greedy token
    print(f"[parity] max|dlogit| per step: {['%.2e' % e for e in errs]}  agree {agree}/{n_steps}", flush=True)
    mk.close()
    return errs, agree


def test_tiny_fp32_prefill_and_greedy_decode(env):
    cfg = synth.CONFIGS["tiny"]
    errs, agree = run_pair(env, cfg, seed=1, n_prompt=cfg.context, n_steps=cfg.decode_steps)
    assert max(errs) <= 1e-4
    assert agree == cfg.decode_steps


def test_tiny_bf16_gqa4_tied(env):
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=8, n_kv_heads=2, head_dim=64, tied=True,
                                      rope_theta=500000.0)
    errs, agree = run_pair(env, cfg, seed=2, n_prompt=40, n_steps=8)
    assert max(errs) <= 2e-2
    assert agree == 8


def test_first_position_with_poisoned_cache(env):
    # pos = 0: attention over the single just-written position; the rest of
    # the cache holds NaN and must never be read.
    cfg = synth.CONFIGS["tiny"]
    errs, agree = run_pair(env, cfg, seed=3, n_prompt=0, n_steps=3)
    assert max(errs) <= 1e-4 and agree == 3


# depth: slots the loads run ahead (0: ring - 1); drain: no cross-stage prefetch
@pytest.mark.parametrize("grid,splits,ring,depth,drain", [(64, 8, 3, 0, 0), (37, 5, 4, 0, 0), (256, 1, 8, 0, 0),
                                                          (256, 1, 9, 0, 0), (64, 8, 3, 1, 0), (37, 5, 4, 2, 1),
                                                          (256, 1, 8, 1, 1), (256, 1, 8, 0, 1)])
def test_tiny_other_launch_shapes(env, grid, splits, ring, depth, drain):
    cfg = synth.CONFIGS["tiny"]
    errs, agree = run_pair(env, cfg, seed=4, n_prompt=21, n_steps=3,
                           tuning={"grid": grid, "attn_splits": splits, "ring_slots": ring, "prefetch_depth": depth,
                                   "stage_drain": drain})
    assert max(errs) <= 1e-4 and agree == 3


def test_prefetch_depth_beyond_ring_is_rejected(env):
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"]
    for tun in ({"ring_slots": 4, "prefetch_depth": 4},
                # two slots per data step: the depth must leave both slots of
                # a step unclaimed and cover both before the step's barrier
                {"ring_slots": 4, "prefetch_depth": 3, "slots_per_step": 2},
                {"ring_slots": 8, "prefetch_depth": 1, "slots_per_step": 2}):
        with pytest.raises(mkp.MkError) as e:
            _make(env, cfg, seed=0, max_seq=32, tuning=tun)
        assert e.value.status == mkp.mk.MK_ERR_TUNING, tun


# ---- the stream's tile: two ring slots per data step ----
# Every stage's slot count is odd or even somewhere in these shapes (1B: 3
# QKV slots; ragged shapes: partial pieces and row groups), so steps of one
# slot at a stage's end are covered; the ring sizes and depths cover the
# limits of depth 2 .. ring - 2; fp32 with prefill by decode launches runs
# the cache-append instantiation.

@pytest.mark.parametrize("case", ["fp32_mha_decode_launch_prefill", "bf16_gqa4_ring4", "bf16_long_context",
                                  "bf16_position_major", "bf16_group8_head128", "w8_ragged_small_grid",
                                  "bf16_stage_drain"])
def test_two_slots_per_step(env, case):
    tiny = synth.CONFIGS["tiny"]
    bf = dict(dtype="bf16", rope_theta=500000.0)
    tun = {"slots_per_step": 2}
    kw = {}
    if case == "fp32_mha_decode_launch_prefill":
        cfg, tol = tiny.with_(n_heads=4, n_kv_heads=4), 1e-4
        tun.update(prefill_chunk=-1)
        kw = dict(n_prompt=50, n_steps=4)
    elif case == "bf16_gqa4_ring4":
        cfg, tol = tiny.with_(n_heads=8, n_kv_heads=2, **bf), 2e-2
        tun.update(ring_slots=4, prefetch_depth=2)
        kw = dict(n_prompt=37, n_steps=4)
    elif case == "bf16_long_context":
        cfg, tol = tiny.with_(n_heads=8, n_kv_heads=2, **bf), 2e-2
        tun.update(grid=64, attn_splits=8)
        kw = dict(n_prompt=900, n_steps=4, use_prefill=False)
    elif case == "bf16_position_major":
        cfg, tol = tiny.with_(n_heads=8, n_kv_heads=2, **bf), 2e-2
        tun.update(grid=64, attn_splits=8, attn_pm_slots=1)
        kw = dict(n_prompt=900, n_steps=4, use_prefill=False)
    elif case == "bf16_group8_head128":
        cfg, tol = tiny.with_(n_heads=16, n_kv_heads=2, head_dim=128, **bf), 2e-2
        kw = dict(n_prompt=45, n_steps=4)
    elif case == "w8_ragged_small_grid":
        cfg, tol = tiny.with_(dtype="w8", rope_theta=500000.0, tied=False, hidden=264, ffn=696, vocab=1000, n_heads=8,
                              n_kv_heads=2), 2e-2
        tun.update(grid=64, attn_splits=8)
        kw = dict(n_prompt=50, n_steps=4, expect_batched=False)
    else:  # bf16_stage_drain
        cfg, tol = tiny.with_(n_heads=8, n_kv_heads=2, **bf), 2e-2
        tun.update(stage_drain=1, ring_slots=5, prefetch_depth=3)
        kw = dict(n_prompt=60, n_steps=4)
    errs, agree = run_pair(env, cfg, seed=80, tuning=tun, **kw)
    assert max(errs) <= tol and agree == kw["n_steps"]


def test_llama1b_two_slots_per_step(env):
    cfg = synth.CONFIGS["llama1b"]
    errs, agree = run_pair(env, cfg, seed=81, n_prompt=cfg.context, n_steps=3, gains="random", use_prefill=False,
                           tuning={"slots_per_step": 2})
    assert max(errs) <= 2e-2 and agree == 3


def test_llama1b_full_size_synthetic_context(env):
    cfg = synth.CONFIGS["llama1b"]
    errs, agree = run_pair(env, cfg, seed=5, n_prompt=cfg.context, n_steps=3, gains="ones", use_prefill=False)
    assert max(errs) <= 2e-2 and agree == 3


@pytest.mark.parametrize("depth,drain", [(0, 0), (2, 1)])
def test_llama1b_prefill_short_prompt(env, depth, drain):
    cfg = synth.CONFIGS["llama1b"]
    errs, agree = run_pair(env, cfg, seed=6, n_prompt=5, n_steps=2, gains="random",
                           tuning={"prefetch_depth": depth, "stage_drain": drain})
    assert max(errs) <= 2e-2 and agree == 2


# ---- more shapes: group sizes and head widths the full-size models use ----

def test_tiny_bf16_group8(env):
    # eight query heads per KV head (the 70B shape's grouping): each consumer
    # holds two heads of the group
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=16, n_kv_heads=2, head_dim=64, rope_theta=500000.0)
    errs, agree = run_pair(env, cfg, seed=7, n_prompt=30, n_steps=4)
    assert max(errs) <= 2e-2 and agree == 4


def test_tiny_fp32_mha(env):
    # one query head per KV head: four consumers share each head and the
    # combine merges their records as extra splits
    cfg = synth.CONFIGS["tiny"].with_(n_heads=4, n_kv_heads=4)
    errs, agree = run_pair(env, cfg, seed=8, n_prompt=50, n_steps=4)
    assert max(errs) <= 1e-4 and agree == 4


def test_tiny_bf16_head128(env):
    # head_dim 128 in bfloat16 (the 8B/70B head width): 16 lanes per cache row
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=4, n_kv_heads=1, head_dim=128, rope_theta=500000.0)
    errs, agree = run_pair(env, cfg, seed=9, n_prompt=70, n_steps=4)
    assert max(errs) <= 2e-2 and agree == 4


def test_tiny_bf16_group8_head128_prefill(env):
    # the 70B shape's pairing of eight query heads per KV head with head_dim
    # 128, through both instantiations: the prefill (no LM head) fills the
    # cache, whose rows are compared with the oracle's, then decode steps
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=16, n_kv_heads=2, head_dim=128, rope_theta=500000.0)
    errs, agree = run_pair(env, cfg, seed=13, n_prompt=45, n_steps=4)
    assert max(errs) <= 2e-2 and agree == 4


@pytest.mark.parametrize("n_prompt", [63, 64, 65, 72, 200])
def test_split_remainders(env, n_prompt):
    # splits whose positions end exactly on a KV slot, one past it, a short
    # tail folded from registers, and a long tail through the ring
    cfg = synth.CONFIGS["tiny"]
    errs, agree = run_pair(env, cfg, seed=10, n_prompt=n_prompt, n_steps=2, tuning={"attn_splits": 1})
    assert max(errs) <= 1e-4 and agree == 2


# ---- determinism and the device-token entry point ----

def _make(env, cfg, seed, max_seq, tuning=None):
    torch, oracle, mkp = env
    host = synth.gen_weights(cfg, seed=seed)
    dev_w = mkp.upload_weights(host)
    mk = mkp.MegaKernel(shape_of(cfg), dev_w, max_seq, tuning=tuning)
    return mk, host


def test_bit_identical_reruns_and_device_token(env):
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=8, n_kv_heads=2, rope_theta=500000.0)
    n_prompt, max_seq = 33, 40
    mk, _ = _make(env, cfg, 11, max_seq)
    toks = synth.gen_tokens(11, n_prompt + 1, cfg.vocab)
    kv = mkp.KVCache(shape_of(cfg), max_seq)
    mk.prefill_kv(toks[:n_prompt], 0, kv)
    la = torch.empty(cfg.vocab, device="cuda")
    lb = torch.empty(cfg.vocab, device="cuda")
    mk.decode_step(int(toks[n_prompt]), n_prompt, kv, la)
    # the same step again (it rewrites the same cache row with the same values)
    mk.decode_step(int(toks[n_prompt]), n_prompt, kv, lb)
    torch.cuda.synchronize()
    assert torch.equal(la, lb), "two launches of the same step differ"
    # device-token variant: same logits bit for bit, token = lowest-index argmax
    tin = torch.tensor([int(toks[n_prompt])], dtype=torch.int32, device="cuda")
    tout = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    lc = torch.empty(cfg.vocab, device="cuda")
    mk.decode_step_device_token(tin, n_prompt, kv, lc, tout)
    torch.cuda.synchronize()
    assert mk.device_error() == 0
    assert torch.equal(la, lc)
    host_logits = la.cpu().numpy()
    assert int(tout.item()) == int(np.flatnonzero(host_logits == host_logits.max())[0])
    # and without logits
    tout2 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    mk.decode_step_device_token(tin, n_prompt, kv, None, tout2)
    torch.cuda.synchronize()
    assert int(tout2.item()) == int(tout.item())
    mk.close()


def test_alternating_streams_keep_call_order(env):
    """One handle's calls on two streams, alternating, with no host
    synchronisation between them: the prefill on one stream, then every
    decode step on the other stream than the call before.  Each step reads
    the cache rows the previous calls wrote, so the steps match the oracle
    only if the library orders each call after the handle's last one (it
    records an event after each call and makes a new stream wait on it)."""
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=8, n_kv_heads=2, rope_theta=500000.0)
    n_prompt, n_steps = 150, 12
    max_seq = n_prompt + n_steps
    mk, host = _make(env, cfg, 17, max_seq)
    ref = oracle.Model(shape_of(cfg), host, max_seq)
    toks = synth.gen_tokens(17, n_prompt + 1, cfg.vocab)
    ref.prefill(toks[:n_prompt])
    # the oracle's teacher-forced run first: the GPU calls are then enqueued back to back
    feed, want = [int(toks[n_prompt])], []
    for s in range(n_steps):
        want.append(ref.decode_step(feed[-1], n_prompt + s))
        feed.append(oracle.argmax(want[-1]))
    kv = mkp.KVCache(shape_of(cfg), max_seq, fill=float("nan"))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    logits = torch.full((n_steps, cfg.vocab), float("nan"), device="cuda")
    torch.cuda.synchronize()
    mk.prefill_kv(toks[:n_prompt], 0, kv, stream=streams[0])
    for s in range(n_steps):
        mk.decode_step(feed[s], n_prompt + s, kv, logits[s], stream=streams[(s + 1) % 2])
    torch.cuda.synchronize()
    assert mk.device_error() == 0
    got = logits.cpu().numpy().astype(np.float64)
    for s in range(n_steps):
        assert np.isfinite(got[s]).all(), s
        assert float(np.abs(got[s] - want[s]).max()) <= 2e-2, s
        assert int(np.argmax(got[s])) == feed[s + 1], s
    mk.close()


def test_prefill_equals_decode_loop(env):
    # mk_prefill_kv(n) writes exactly the cache rows that n decode steps write
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", n_heads=8, n_kv_heads=2, rope_theta=500000.0)
    n, max_seq = 20, 24
    mk, _ = _make(env, cfg, 12, max_seq)
    toks = synth.gen_tokens(12, n, cfg.vocab)
    kv1 = mkp.KVCache(shape_of(cfg), max_seq)
    kv2 = mkp.KVCache(shape_of(cfg), max_seq)
    mk.prefill_kv(toks, 0, kv1)
    logits = torch.empty(cfg.vocab, device="cuda")
    for i in range(n):
        mk.decode_step(int(toks[i]), i, kv2, logits)
    torch.cuda.synchronize()
    assert mk.device_error() == 0
    assert torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v)
    mk.close()


def test_device_token_out_of_range_sets_device_error(env):
    # a token id outside [0, vocab) read from device memory cannot be checked
    # on the host: the kernel raises the device error flag (and embeds row 0)
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"]
    mk, _ = _make(env, cfg, 13, 8)
    kv = mkp.KVCache(shape_of(cfg), 8)
    tin = torch.tensor([cfg.vocab + 5], dtype=torch.int32, device="cuda")
    tout = torch.empty(1, dtype=torch.int32, device="cuda")
    mk.decode_step_device_token(tin, 0, kv, None, tout)
    assert mk.device_error() == mkp.mk.MK_ERR_DEVICE
    # the handle is now disabled
    with pytest.raises(mkp.MkError):
        mk.decode_step_device_token(tin, 1, kv, None, tout)
    mk.close()


def test_deferred_weight_loading(env):
    """mk_create_deferred + mk_load_weights, layers loaded in reverse order:
    steps are refused until every part is loaded, then match the oracle like
    a handle made by mk_create."""
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"].with_(n_layers=3)
    shape = shape_of(cfg)
    host = synth.gen_weights(cfg, seed=31, gains="random")
    mk = mkp.MegaKernel(shape, None, 40)
    kv = mkp.KVCache(shape, 40)
    logits = torch.empty(cfg.vocab, device="cuda")
    for l in (2, 0):
        mk.load_weights(mkp.upload_weights({"layers": [host["layers"][l]]}), first_layer=l)
    mk.load_weights(mkp.upload_weights({k: v for k, v in host.items() if k != "layers"}))
    with pytest.raises(mkp.MkError) as ei:  # layer 1 still missing
        mk.decode_step(1, 0, kv, logits)
    assert ei.value.status == mkp.mk.MK_ERR_STATE
    with pytest.raises(mkp.MkError) as ei:
        mk.load_weights(mkp.upload_weights({"layers": [host["layers"][1]]}), first_layer=3)
    assert ei.value.status == mkp.mk.MK_ERR_RANGE
    mk.close()
    errs, agree = run_pair(env, cfg, seed=31, n_prompt=20, n_steps=6, deferred=True)
    assert max(errs) <= 1e-4 and agree == 6


def test_row_groups_hidden4096(env):
    """Rows of 8 KiB (hidden 4096 bf16): the pre-layout interleaves whole
    groups of four rows chunk by chunk.  QKV has 6 units per workgroup (one
    group and two rows after it), O exactly one group, gate/up two rows (no
    group), the LM head 0 or 1 row per workgroup."""
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16", hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=1024,
                                      vocab=1000, tied=True, rope_theta=500000.0)
    errs, agree = run_pair(env, cfg, seed=41, n_prompt=30, n_steps=4)
    assert max(errs) <= 2e-2 and agree == 4


def test_stage_timeline_tool_runs(env, capsys):
    """The stage-timeline diagnostic (mk_read_trace) runs end to end and
    reports every stage kind."""
    from transformer_megakernel_persistent_amd import stage_timeline
    stage_timeline.summarise("tiny", {})
    out = capsys.readouterr().out
    for st in stage_timeline.STAGES:
        assert f"  {st:5s} epilogue" in out
    assert "per layer" in out


# ---- per-length attention mapping: position-major for long splits ----

@pytest.mark.parametrize("n_prompt,splits,dtype", [(130, 2, "f32"), (200, 2, "f32"), (333, 3, "f32"), (260, 2, "bf16")])
def test_position_major_attention(env, n_prompt, splits, dtype):
    """Four query heads per KV head with the position-major mapping forced
    (attn_pm_slots 1): each consumer folds two chunks of every KV slot for all
    four heads, the four partials merged in LDS.  Splits with whole slots plus
    a register tail (130: 65 positions each), a second partial slot (200),
    three splits (333), and the bf16 cache."""
    cfg = synth.CONFIGS["tiny"].with_(n_heads=8, n_kv_heads=2, dtype=dtype,
                                      rope_theta=10000.0 if dtype == "f32" else 500000.0)
    errs, agree = run_pair(env, cfg, seed=81, n_prompt=n_prompt, n_steps=3,
                           tuning={"attn_splits": splits, "attn_pm_slots": 1})
    assert max(errs) <= tol_of(cfg) and agree == 3


def test_position_major_equals_head_major(env):
    """The same steps with the position-major mapping forced and with it off
    agree to fp32 rounding (the mapping only changes the summation order)."""
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"].with_(n_heads=8, n_kv_heads=2)
    n, max_seq = 300, 304
    toks = synth.gen_tokens(82, n + 1, cfg.vocab)
    outs = []
    for pm in (1, -1):
        mk, _ = _make(env, cfg, 82, max_seq, tuning={"attn_splits": 2, "attn_pm_slots": pm})
        kv = mkp.KVCache(shape_of(cfg), max_seq)
        mk.prefill_kv(toks[:n], 0, kv)
        lg = torch.empty(cfg.vocab, device="cuda")
        mk.decode_step(int(toks[n]), n, kv, lg)
        torch.cuda.synchronize()
        assert mk.device_error() == 0
        outs.append(lg.cpu().numpy().astype(np.float64))
        mk.close()
    d = float(np.abs(outs[0] - outs[1]).max())
    print(f"[parity] position-major vs head-major logits max|d| = {d:.3e}", flush=True)
    assert d <= 1e-5
