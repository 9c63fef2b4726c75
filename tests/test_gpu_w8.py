"""GPU parity of the weight-only INT8 path (dtype "w8": int8 matrices with one
float32 scale per output row, bf16 embedding, gains and KV cache) through the
C ABI, against the oracle's dequantising decode step (or_gemv_q8), on the
same seeded inputs.

Bars: max|dlogit| <= 2e-2 on every step and greedy agreement (the bf16 bar;
the weights the kernel multiplies are exactly the oracle's s * q, only the
order of the fp32 rounding differs); prefilled K/V rows within 5e-2, and
within one bf16 rounding step in layer 0.  An INT8 model's prefill goes
through the matrix-core GEMMs (codes widened to bf16, row scales on the
sums) when its down-stage slices start at multiples of 8, else it runs as
one decode launch per position.

Cases: every query-group size with both head sizes; ragged shapes (an int8
row shorter than one 1 KiB chunk, SwiGLU slices that end inside a 16-element
piece, a vocabulary that ends inside a unit, fewer workgroups so that each
holds larger scale blocks); weights loaded a layer at a time; the full
Llama-3.2-1B and Llama-3-8B shapes from the GPU's own prefill, teacher-forced
and as the device-token chain the benchmark times."""
import numpy as np
import pytest

import synth

from test_gpu_parity import env, run_pair  # noqa: F401  (fixture)
from test_gpu_runs import Run, _device_token_chain, assert_run

pytestmark = pytest.mark.gpu

W8_TINY = synth.CONFIGS["tiny"].with_(name="tiny_w8", dtype="w8", rope_theta=500000.0, tied=False)


@pytest.mark.parametrize("gq,d", [(1, 64), (2, 64), (4, 64), (8, 64), (2, 128), (4, 128)])
def test_tiny_w8_groups_and_head_sizes(env, gq, d):
    cfg = W8_TINY.with_(n_heads=2 * gq, n_kv_heads=2, head_dim=d)
    errs, agree = run_pair(env, cfg, seed=60 + gq + d, n_prompt=37, n_steps=6, expect_batched=False)
    assert max(errs) <= 2e-2
    assert agree == 6


def test_tiny_w8_ragged_shapes_and_small_grid(env):
    # hidden 264: an int8 row of 264 bytes (one partial chunk); ffn 696: 43.5
    # pieces of 16 SwiGLU outputs; vocab 1000; 64 workgroups (larger blocks)
    cfg = W8_TINY.with_(hidden=264, ffn=696, vocab=1000, n_heads=8, n_kv_heads=2)
    errs, agree = run_pair(env, cfg, seed=71, n_prompt=50, n_steps=6, tuning={"grid": 64, "attn_splits": 8},
                           expect_batched=False)
    assert max(errs) <= 2e-2
    assert agree == 6


@pytest.mark.parametrize("d", [64, 128])
def test_tiny_w8_batched_prefill(env, d):
    # 64 workgroups own 8 gate/up units each, so every down slice starts at a
    # multiple of 16 inputs and the batched prefill applies; chunks of 32
    # positions with a ragged last chunk
    cfg = W8_TINY.with_(n_heads=8, n_kv_heads=2, head_dim=d, ffn=1024)
    errs, agree = run_pair(env, cfg, seed=77 + d, n_prompt=70, n_steps=4,
                           tuning={"grid": 64, "attn_splits": 8, "prefill_chunk": 32}, expect_batched=True)
    assert max(errs) <= 2e-2
    assert agree == 4


@pytest.mark.parametrize("case", ["wide_ragged", "input_split"])
def test_tiny_w8_batched_prefill_wide_and_split(env, case):
    # The int8 codes on the GEMM's 128 x 256 tiles: ffn 2112 over 8
    # workgroups (slices on multiples of 8), gate/up of 4224 outputs = 16.5
    # wide tiles, a 2000-token chunk ending inside its 16th token tile.  Or
    # the int8 down projection in two input splits: hidden 2048 (8 x 16 wide
    # tiles), ffn 4096, a ragged 1930-token chunk.
    if case == "wide_ragged":
        cfg = W8_TINY.with_(n_heads=8, n_kv_heads=2, ffn=2112)
        kw = dict(n_prompt=2000, tuning={"grid": 8, "attn_splits": 4})
    else:
        cfg = W8_TINY.with_(hidden=2048, n_heads=16, n_kv_heads=2, head_dim=128, ffn=4096, n_layers=1)
        kw = dict(n_prompt=1930)
    errs, agree = run_pair(env, cfg, seed=79, n_steps=3, expect_batched=True, **kw)
    assert max(errs) <= 2e-2
    assert agree == 3


def test_tiny_w8_deferred_load(env):
    cfg = W8_TINY.with_(n_layers=3, n_heads=8, n_kv_heads=2)
    errs, agree = run_pair(env, cfg, seed=72, n_prompt=20, n_steps=4, deferred=True, expect_batched=False)
    assert max(errs) <= 2e-2
    assert agree == 4


def test_tiny_w8_synthetic_cache_long_split(env):
    # a longer context from a synthetic cache: several KV slots per split
    cfg = W8_TINY.with_(n_heads=8, n_kv_heads=2)
    errs, agree = run_pair(env, cfg, seed=73, n_prompt=900, n_steps=4, use_prefill=False)
    assert max(errs) <= 2e-2
    assert agree == 4


def test_tiny_w8_masked_cache_reads_never_see_weight_bytes(env):
    # Cache positions past a split's end are loaded from a fixed place and
    # multiplied by probability 0, so they must read as finite numbers.  Here
    # the first row of every Wq is int8 codes (-1, 127) alternating: read as
    # bf16 pairs these bytes spell NaN (0x7FFF).  With 32 workgroups every
    # workgroup owns QKV rows, and splits of 25+ positions end inside a ring
    # slot, so masked positions exist on every step.
    torch, oracle, mkp = env
    cfg = W8_TINY.with_(n_heads=8, n_kv_heads=2)
    host = synth.gen_weights(cfg, seed=76, gains="random")
    for lw in host["layers"]:
        lw["wq"][0, 0::2] = -1
        lw["wq"][0, 1::2] = 127
    import test_gpu_parity as tp
    shape = tp.shape_of(cfg)
    n_prompt, n_steps = 100, 4
    ref = oracle.Model(shape, host, n_prompt + n_steps)
    mk = mkp.MegaKernel(shape, mkp.upload_weights(host), n_prompt + n_steps, tuning={"grid": 32, "attn_splits": 4})
    kv = mkp.KVCache(shape, n_prompt + n_steps, fill=float("nan"))
    toks = synth.gen_tokens(76, n_prompt + 1, cfg.vocab)
    ref.prefill(toks[:n_prompt])
    mk.prefill_kv(toks[:n_prompt], 0, kv)
    logits = torch.empty(cfg.vocab, device="cuda")
    tok = int(toks[n_prompt])
    for s in range(n_steps):
        want = ref.decode_step(tok, n_prompt + s)
        mk.decode_step(tok, n_prompt + s, kv, logits)
        torch.cuda.synchronize()
        got = logits.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), s
        assert float(np.abs(got - want).max()) <= 2e-2, s
        assert int(np.argmax(got)) == oracle.argmax(want)
        tok = oracle.argmax(want)
    assert mk.device_error() == 0
    mk.close()


def test_llama1b_w8_run_from_gpu_prefill(env):
    """The Llama-3.2-1B shape with int8 matrices (own int8 LM head): the
    2048-token context prefilled on the GPU, prefill rows sampled, 32
    teacher-forced steps, then 16 device-token launches."""
    cfg = synth.CONFIGS["llama1b_w8"]
    run = Run(env, cfg, seed=74, n_steps=48)
    try:
        run.check_prefill_rows([0, 1, cfg.context - 1])
        errs, agree, mism = run.teacher_forced(32)
        assert_run(errs, agree, mism, 32)
        # the chain continues from the cache the teacher-forced steps left:
        # restart both sides at the context end, the rows past it are rewritten
        _device_token_chain(env, run, 16)
    finally:
        run.close()


def test_llama8b_w8_run_from_gpu_prefill(env):
    """The Llama-3-8B shape with int8 matrices: 2048-token GPU prefill,
    sampled prefill rows, 8 teacher-forced steps (about 3 s per oracle step)."""
    cfg = synth.CONFIGS["llama8b_w8"]
    run = Run(env, cfg, seed=75, n_steps=8)
    try:
        run.check_prefill_rows([1, cfg.context - 1])
        errs, agree, mism = run.teacher_forced(8)
        assert_run(errs, agree, mism, 8)
    finally:
        run.close()
