"""The batched prefill (mk_prefill_kv in chunks: matrix-core GEMMs over the
packed weights, causal attention inside the chunk and over the cache)
against the CPU oracle, through the C ABI.

Bars: the cache rows within 5e-2 of the oracle's own prefill in every layer
and within one bf16 rounding step in layer 0 (see check_layer0_rounding);
the decode steps after it at the usual bar (max|dlogit| <= 2e-2, greedy
agreement).  Chunks are ragged (the last one short) and several per call.
Chunking is invisible in the result: every token's arithmetic (its norm, its
GEMM rows, its attention over positions in order) does not depend on which
other tokens share its chunk, so any chunk size gives the same cache bit for
bit.  The full-size 1B, 8B and 32K runs (test_gpu_runs.py) check rows of the
batched prefill at the workloads' own sizes."""
import numpy as np
import pytest

import synth

from test_gpu_parity import cache_f64, check_layer0_rounding, env, run_pair, shape_of, to_host  # noqa: F401

pytestmark = pytest.mark.gpu


# Shapes whose down-stage workgroups own inputs starting at multiples of 8 at
# 256 workgroups (ffn 2048: 4 units = 8 inputs each), so the batched path is taken.
def tiny_bf16(**kw):
    base = dict(dtype="bf16", hidden=256, n_heads=8, n_kv_heads=2, head_dim=64, ffn=2048, vocab=1024,
                rope_theta=500000.0)
    base.update(kw)
    return synth.CONFIGS["tiny"].with_(**base)


def _handle(env, cfg, seed, max_seq, tuning=None):
    torch, oracle, mkp = env
    host = synth.gen_weights(cfg, seed=seed, gains="random")
    mk = mkp.MegaKernel(shape_of(cfg), mkp.upload_weights(host), max_seq, tuning=tuning)
    return mk, host


@pytest.mark.parametrize("chunk", [64, 0])
def test_batched_prefill_gqa4_then_decode(env, chunk):
    # 200 positions: three full chunks of 64 and a ragged one (or one of 200)
    cfg = tiny_bf16()
    errs, agree = run_pair(env, cfg, seed=71, n_prompt=200, n_steps=4, tuning={"prefill_chunk": chunk},
                           expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 4


def test_batched_prefill_group8_head128(env):
    # the 70B pairing: eight query heads per KV head, head_dim 128
    cfg = tiny_bf16(n_heads=16, n_kv_heads=2, head_dim=128)
    errs, agree = run_pair(env, cfg, seed=72, n_prompt=45, n_steps=4, tuning={"prefill_chunk": 32},
                           expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 4


def test_batched_prefill_mha_tied(env):
    # one query head per KV head, tied embeddings
    cfg = tiny_bf16(n_heads=4, n_kv_heads=4, tied=True)
    errs, agree = run_pair(env, cfg, seed=73, n_prompt=70, n_steps=3, tuning={"prefill_chunk": 16},
                           expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 3


def test_batched_prefill_ragged_gemm_tiles(env):
    # hidden 160: the QKV and gate/up GEMMs end on a half k-tile (64 + 64 +
    # 32 inputs) and the O and down GEMMs on a partial tile of 128 outputs
    # (160 = 128 + 32); one chunk of 150 tokens ends inside the second tile
    # of 128 tokens; two query heads per KV head
    cfg = tiny_bf16(hidden=160, n_heads=4, n_kv_heads=2)
    errs, agree = run_pair(env, cfg, seed=76, n_prompt=150, n_steps=4, expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 4


def test_batched_prefill_wide_tiles_ragged(env):
    # GEMMs with at least 256 tiles of 128 tokens x 256 outputs take the
    # wide tile.  ffn 2112 over 8 workgroups (264 SwiGLU inputs each, slices
    # on multiples of 8): gate/up has 4224 outputs, 16.5 wide tiles, and a
    # 2000-token chunk ends inside its 16th tile of 128 tokens (17 x 16 =
    # 272 tiles); the other GEMMs stay on 128-output tiles
    cfg = tiny_bf16(ffn=2112, n_layers=2)
    errs, agree = run_pair(env, cfg, seed=78, n_prompt=2000, n_steps=3, tuning={"grid": 8, "attn_splits": 4},
                           expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 3


def test_batched_prefill_input_split_ragged(env):
    # hidden 2048 (the 1B width): the down GEMM has 8 x 16 wide tiles, too
    # few for the chip, and 4096 inputs, so it runs as two input splits (the
    # second one's sums added afterwards); a 1930-token chunk ends inside the
    # 16th tile of 128 tokens
    cfg = tiny_bf16(hidden=2048, n_heads=16, n_kv_heads=2, head_dim=128, ffn=4096, n_layers=1)
    errs, agree = run_pair(env, cfg, seed=77, n_prompt=1930, n_steps=3, expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 3


@pytest.mark.parametrize("heads,head_dim,chunk", [(4, 64, 2048), (8, 64, 2048), (8, 128, 2048), (4, 64, 0)])
def test_batched_prefill_long_prompt_two_row_blocks(env, heads, head_dim, chunk):
    # Once a chunk's causal range passes 8192 positions the attention takes
    # two 16-row query blocks per wave for 64-dim heads (128-dim heads keep
    # one).  8300 positions in chunks of 2048 (or the default 4096): the
    # last chunk (pos0 8192, 108 tokens) ends inside a query block of that
    # path, with one KV head (four or eight query heads per KV head)
    cfg = tiny_bf16(n_layers=1, n_heads=heads, n_kv_heads=1, head_dim=head_dim)
    errs, agree = run_pair(env, cfg, seed=79, n_prompt=8300, n_steps=2, tuning={"prefill_chunk": chunk},
                           expect_batched=True)
    assert max(errs) <= 2e-2 and agree == 2


def test_chunking_is_invisible_and_start_pos(env):
    """Chunks of 7, 64 and 256 positions, and the same prompt prefilled in
    two calls (positions 0..99, then 100..149), leave identical caches."""
    torch, oracle, mkp = env
    cfg = tiny_bf16()
    n, max_seq = 150, 160
    toks = synth.gen_tokens(74, n, cfg.vocab)
    caches = []
    for chunk, split in ((7, None), (64, None), (256, None), (64, 100)):
        mk, _ = _handle(env, cfg, 74, max_seq, {"prefill_chunk": chunk})
        assert mk.info()["prefill_chunk"] == chunk
        kv = mkp.KVCache(shape_of(cfg), max_seq, fill=0.0)
        if split is None:
            mk.prefill_kv(toks, 0, kv)
        else:
            mk.prefill_kv(toks[:split], 0, kv)
            mk.prefill_kv(toks[split:], split, kv)
        torch.cuda.synchronize()
        assert mk.device_error() == 0
        caches.append((kv.k.clone(), kv.v.clone()))
        mk.close()
    for k, v in caches[1:]:
        assert torch.equal(k, caches[0][0]) and torch.equal(v, caches[0][1])


def test_batched_prefill_close_to_decode_launches(env):
    """The batched prefill and the one-launch-per-position prefill of the
    same model fill caches that agree within the bf16 bar."""
    torch, oracle, mkp = env
    cfg = tiny_bf16()
    n, max_seq = 90, 96
    toks = synth.gen_tokens(75, n, cfg.vocab)
    out = []
    for chunk in (0, -1):
        mk, _ = _handle(env, cfg, 75, max_seq, {"prefill_chunk": chunk})
        assert (mk.info()["prefill_chunk"] > 0) == (chunk == 0)
        kv = mkp.KVCache(shape_of(cfg), max_seq, fill=0.0)
        mk.prefill_kv(toks, 0, kv)
        torch.cuda.synchronize()
        out.append((cache_f64(oracle, cfg, to_host(kv.k)[:, :, :n]), cache_f64(oracle, cfg, to_host(kv.v)[:, :, :n])))
        mk.close()
    for i, name in ((0, "K"), (1, "V")):
        d = float(np.abs(out[0][i] - out[1][i]).max())
        print(f"[prefill] batched vs decode launches: {name} max|d| {d:.3e}", flush=True)
        assert d <= 5e-2
        check_layer0_rounding(out[0][i], out[1][i], name)


def test_unsupported_geometry_uses_decode_launches(env):
    # ffn 688 at 256 workgroups: down-stage workgroups start at odd multiples
    # of 2, not of 8, so the prefill falls back to decode launches
    cfg = tiny_bf16(ffn=688)
    mk, _ = _handle(env, cfg, 76, 32)
    assert mk.info()["prefill_chunk"] == 0
    mk.close()
