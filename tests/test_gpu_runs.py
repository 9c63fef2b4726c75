"""GPU parity over whole decode runs at the workloads' full sizes, through the
C ABI, against the CPU oracle.

Each run starts from the GPU's OWN prefill: mk_prefill_kv fills the context,
the oracle's cache is a host copy of that cache (an fp64 oracle prefill of
thousands of positions is too slow for a test), and

  1. sampled cache rows of the prefill are checked against the oracle: for a
     position p, the oracle runs the step at p from the GPU's rows [0, p);
     its K and V rows at p must match the GPU's within 5e-2 in every layer,
     and within one bfloat16 rounding step in layer 0 (whose rows depend on
     nothing but the token and the layer's weights, so both sides round the
     same real value);
  2. the decode steps are teacher-forced (both sides are fed the oracle's
     greedy token): every step's logits within max|dlogit| <= 2e-2 and the
     greedy tokens in agreement on at least 99 % of the steps; a step where
     they differ must be a near tie of the oracle's top two logits.

The device-token chain is the exact path the benchmark times: K launches of
mk_decode_step_device_token back to back, each reading the token the
previous one wrote.  Its tokens and logits are compared with the oracle
stepped along the same token sequence.

Each run prints one "[run]" line with its max|dlogit|, agreement and the
smallest top-2 gap of the oracle's logits (how close the run came to a tie).
"""
import numpy as np
import pytest

import synth

from test_gpu_parity import cache_f64, check_layer0_rounding, env, shape_of, to_host  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

TOL = 2e-2  # bf16 weights


class Run:
    """A model on both sides with the context prefilled by the GPU."""

    def __init__(self, env, cfg, seed, n_steps):
        torch, oracle, mkp = env
        self.torch, self.oracle, self.mkp, self.cfg = torch, oracle, mkp, cfg
        print(f"[run] {cfg.name}: generating weights (seed {seed})", flush=True)
        shape = shape_of(cfg)
        ctx = cfg.context
        self.ctx = ctx
        self.max_seq = ctx + n_steps
        host = synth.gen_weights(cfg, seed=seed, gains="ones")
        self.ref = oracle.Model(shape, host, self.max_seq)
        dev_w = mkp.upload_weights(host)
        self.mk = mkp.MegaKernel(shape, dev_w, self.max_seq)
        del dev_w
        torch.cuda.empty_cache()
        self.kv = mkp.KVCache(shape, self.max_seq, fill=float("nan"))
        self.toks = synth.gen_tokens(seed, ctx + 1, cfg.vocab)
        print(f"[run] {cfg.name}: GPU prefill of {ctx} positions", flush=True)
        self.mk.prefill_kv(self.toks[:ctx], 0, self.kv)
        torch.cuda.synchronize()
        assert self.mk.device_error() == 0
        self.gk = to_host(self.kv.k).copy()
        self.gv = to_host(self.kv.v).copy()
        assert np.isfinite(cache_f64(oracle, cfg, self.gk[:, :, :ctx])).all()
        assert np.isfinite(cache_f64(oracle, cfg, self.gv[:, :, :ctx])).all()
        self.ref.k[:, :, :ctx] = self.gk[:, :, :ctx]
        self.ref.v[:, :, :ctx] = self.gv[:, :, :ctx]

    def check_prefill_rows(self, positions):
        """The oracle's K/V rows at each sampled position, computed from the
        GPU's rows before it, against the GPU's rows (all layers, heads)."""
        worst = np.zeros(self.cfg.n_layers)
        for p in positions:
            self.ref.decode_step(int(self.toks[p]), int(p), want_logits=False)
            for name, g, r in (("K", self.gk, self.ref.k), ("V", self.gv, self.ref.v)):
                got = cache_f64(self.oracle, self.cfg, g[:, :, p])
                want = cache_f64(self.oracle, self.cfg, r[:, :, p])
                d = np.abs(got - want)
                worst = np.maximum(worst, d.reshape(d.shape[0], -1).max(1))
                assert float(d.max()) <= 5e-2, f"{name} row {p}: max|d| {float(d.max()):.3e}"
                check_layer0_rounding(got, want, f"{name} row {p}")
            # back to the GPU's row, so that later positions read the GPU's cache
            self.ref.k[:, :, p] = self.gk[:, :, p]
            self.ref.v[:, :, p] = self.gv[:, :, p]
        print(f"[run] {self.cfg.name}: prefill rows at {list(positions)}: max|d| {worst.max():.3e} "
              f"(per layer {['%.1e' % x for x in worst]}), layer 0 within one bf16 step", flush=True)

    def teacher_forced(self, n_steps):
        torch = self.torch
        logits = torch.empty(self.cfg.vocab, device="cuda")
        tok = int(self.toks[self.ctx])
        errs, gaps, mism = [], [], []
        for s in range(n_steps):
            pos = self.ctx + s
            want = self.ref.decode_step(tok, pos)
            logits.fill_(float("nan"))
            self.mk.decode_step(tok, pos, self.kv, logits)
            torch.cuda.synchronize()
            got = logits.cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all()
            errs.append(float(np.abs(got - want).max()))
            top2 = np.sort(np.partition(want, -2)[-2:])
            gaps.append(float(top2[1] - top2[0]))
            nxt = self.oracle.argmax(want)
            if int(np.argmax(got)) != nxt:
                mism.append((s, gaps[-1]))
            tok = nxt
        assert self.mk.device_error() == 0
        agree = n_steps - len(mism)
        print(f"[run] {self.cfg.name}: {n_steps} teacher-forced steps from position {self.ctx}: "
              f"max|dlogit| {max(errs):.3e} (median step {np.median(errs):.3e}), greedy agreement "
              f"{agree}/{n_steps}, smallest top-2 gap {min(gaps):.3e}, mismatches (step, gap) {mism}", flush=True)
        return errs, agree, mism

    def close(self):
        self.mk.close()


def assert_run(errs, agree, mism, n_steps, tol=TOL):
    assert max(errs) <= tol
    assert agree >= 0.99 * n_steps
    for s, gap in mism:  # only a near tie of the oracle's top two may flip
        assert gap <= 2 * errs[s], (s, gap, errs[s])


def test_llama1b_full_run_from_gpu_prefill(env):
    """Llama-3.2-1B shape, 2048-token context prefilled on the GPU, all 128
    decode steps of the workload."""
    cfg = synth.CONFIGS["llama1b"]
    run = Run(env, cfg, seed=51, n_steps=cfg.decode_steps)
    run.check_prefill_rows([0, 1, 777, cfg.context - 1])
    errs, agree, mism = run.teacher_forced(cfg.decode_steps)
    run.close()
    assert_run(errs, agree, mism, cfg.decode_steps)


def test_llama1b_32k_full_run_from_gpu_prefill(env):
    """The 1B shape with a 32768-token context prefilled on the GPU, all 64
    decode steps of the workload."""
    cfg = synth.CONFIGS["llama1b_32k"]
    run = Run(env, cfg, seed=52, n_steps=cfg.decode_steps)
    run.check_prefill_rows([0, 20000, cfg.context - 1])
    errs, agree, mism = run.teacher_forced(cfg.decode_steps)
    run.close()
    assert_run(errs, agree, mism, cfg.decode_steps)


def test_llama8b_run_from_gpu_prefill(env):
    """Llama-3-8B shape, 2048-token context prefilled on the GPU, the first 16
    of the workload's 128 decode steps (the fp64 oracle needs about 3 s per
    8B step on the test host)."""
    cfg = synth.CONFIGS["llama8b"]
    n = 16
    run = Run(env, cfg, seed=53, n_steps=n)
    run.check_prefill_rows([1, cfg.context - 1])
    errs, agree, mism = run.teacher_forced(n)
    run.close()
    assert_run(errs, agree, mism, n)


def _device_token_chain(env, run, n_steps, tol=TOL):
    """n_steps launches of mk_decode_step_device_token back to back (the loop
    the benchmark times), then the oracle stepped along the GPU's tokens."""
    torch = run.torch
    cfg = run.cfg
    tin = torch.tensor([int(run.toks[run.ctx])], dtype=torch.int32, device="cuda")
    toks = torch.full((n_steps,), -1, dtype=torch.int32, device="cuda")
    logits = torch.full((n_steps, cfg.vocab), float("nan"), device="cuda")
    for i in range(n_steps):
        src = tin if i == 0 else toks[i - 1:i]
        run.mk.decode_step_device_token(src, run.ctx + i, run.kv, logits[i], toks[i:i + 1])
    torch.cuda.synchronize()
    assert run.mk.device_error() == 0
    g_toks = toks.cpu().numpy()
    g_logits = logits.cpu().numpy().astype(np.float64)
    tok = int(run.toks[run.ctx])
    errs, mism, gaps = [], [], []
    for i in range(n_steps):
        want = run.ref.decode_step(tok, run.ctx + i)
        got = g_logits[i]
        assert np.isfinite(got).all()
        errs.append(float(np.abs(got - want).max()))
        # the token the device wrote is the argmax of its own logits, lowest index on ties
        assert int(g_toks[i]) == int(np.flatnonzero(got == got.max())[0]), i
        o = run.oracle.argmax(want)
        top2 = np.sort(np.partition(want, -2)[-2:])
        gaps.append(float(top2[1] - top2[0]))
        if int(g_toks[i]) != o:
            mism.append((i, float(want[o] - want[int(g_toks[i])])))
        tok = int(g_toks[i])  # the oracle follows the chain the device took
    agree = n_steps - len(mism)
    print(f"[run] {cfg.name}: device-token chain of {n_steps} launches: max|dlogit| {max(errs):.3e}, "
          f"greedy agreement {agree}/{n_steps}, smallest top-2 gap {min(gaps):.3e}, mismatches {mism}, "
          f"tokens {[int(t) for t in g_toks[:8]]}...", flush=True)
    assert_run(errs, agree, mism, n_steps, tol)


def test_tiny_device_token_chain(env):
    """The tiny fp32 model: 16 chained device-token launches against the
    oracle at the fp32 bar."""
    torch, oracle, mkp = env
    cfg = synth.CONFIGS["tiny"]
    run = Run.__new__(Run)
    run.torch, run.oracle, run.mkp, run.cfg = torch, oracle, mkp, cfg
    shape = shape_of(cfg)
    run.ctx = cfg.context
    run.max_seq = cfg.max_seq
    host = synth.gen_weights(cfg, seed=54, gains="random")
    run.ref = oracle.Model(shape, host, run.max_seq)
    run.mk = mkp.MegaKernel(shape, mkp.upload_weights(host), run.max_seq)
    run.kv = mkp.KVCache(shape, run.max_seq, fill=float("nan"))
    run.toks = synth.gen_tokens(54, run.ctx + 1, cfg.vocab)
    run.mk.prefill_kv(run.toks[:run.ctx], 0, run.kv)
    run.ref.prefill(run.toks[:run.ctx])  # the tiny model is prefilled independently on both sides
    try:
        _device_token_chain(env, run, cfg.decode_steps, tol=1e-4)
    finally:
        run.close()


def test_llama1b_device_token_chain(env):
    """The benchmark's timed loop on the Llama-3.2-1B shape: 32 chained
    launches from the GPU-prefilled 2048-token context."""
    cfg = synth.CONFIGS["llama1b"]
    run = Run(env, cfg, seed=55, n_steps=32)
    try:
        _device_token_chain(env, run, 32)
    finally:
        run.close()
