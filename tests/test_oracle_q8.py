"""Pins for the oracle's weight-only INT8 path (dtype "w8"): the dequantising
matrix-vector product W[r][c] = s[r] * q[r][c] and the whole decode step of
an INT8 model.

- or_gemv_q8: a hand-worked example with exact values (signed codes
  including -128, a different scale per row, a non-square matrix: a
  transposed operand, a column-indexed scale or an unsigned code fails it),
  numpy's product with the dequantised matrix, and the unit-scale special
  case, which reduces it to the pinned or_gemv on the codes.
- The decode step: an INT8 model whose scales are powers of two dequantises
  to weights that bfloat16 holds exactly, so its step must equal, bit for
  bit, the pinned bf16 step of the model with those weights (same cache,
  same logits); and transformers' Llama in float64, given the dequantised
  weights, agrees with it at the bf16-cache bound of the bf16 pin.
CPU only, tiny shapes."""
import numpy as np
import pytest

import synth
from test_oracle_model import TINY, hf_logits, make


def test_gemv_q8_hand_example(orc):
    q = np.array([[1, -2, 127, 0], [-127, 0, 3, 4], [-128, 5, 0, -1]], dtype=np.int8)
    s = np.array([0.5, 0.25, 0.125], dtype=np.float32)
    h = np.array([1.0, 2.0, 3.0, -4.0])
    # row 0: 0.5 * (1 - 4 + 381 + 0) = 189
    # row 1: 0.25 * (-127 + 0 + 9 - 16) = -33.5
    # row 2: 0.125 * (-128 + 10 + 0 + 4) = -14.25
    np.testing.assert_array_equal(orc.gemv_q8(q, s, h), [189.0, -33.5, -14.25])


def test_gemv_q8_matches_numpy_dequantised_product(orc):
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(37, 53)).astype(np.int8)
    s = rng.uniform(1e-4, 2e-3, size=37).astype(np.float32)
    h = rng.standard_normal(53)
    ref = (s.astype(np.float64)[:, None] * q.astype(np.float64)) @ h
    np.testing.assert_allclose(orc.gemv_q8(q, s, h), ref, rtol=1e-13, atol=1e-15)


def test_gemv_q8_unit_scales_is_gemv_of_the_codes(orc):
    rng = np.random.default_rng(6)
    q = rng.integers(-128, 128, size=(19, 64)).astype(np.int8)
    h = rng.standard_normal(64)
    got = orc.gemv_q8(q, np.ones(19, dtype=np.float32), h)
    np.testing.assert_array_equal(got, orc.gemv(q.astype(np.float32), h))


def _pow2_w8(cfg, seed):
    """A w8 model whose per-row scales are 2^-k (k varies by row) and the
    bf16 model holding its dequantised weights exactly."""
    w = synth.gen_weights(cfg, seed=seed, gains="random")
    wb = {"embed": w["embed"], "final_norm": w["final_norm"], "layers": []}

    def pow2(key_rows):
        k = 7 + (np.arange(key_rows) % 4)
        return np.ldexp(np.ones(key_rows), -k).astype(np.float32)

    def deq(q, s):
        f = (s[:, None] * q.astype(np.float32)).astype(np.float32)  # exact: 8-bit code times 2^-k
        bits = f.view(np.uint32)
        assert not (bits & 0xFFFF).any()
        return (bits >> 16).astype(np.uint16)

    w["lm_head_scale"] = pow2(cfg.vocab)
    wb["lm_head"] = deq(w["lm_head"], w["lm_head_scale"])
    for lw in w["layers"]:
        lb = {"attn_norm": lw["attn_norm"], "ffn_norm": lw["ffn_norm"]}
        for k in synth.MATRIX_KINDS:
            lw[k + "_scale"] = pow2(lw[k].shape[0])
            lb[k] = deq(lw[k], lw[k + "_scale"])
        wb["layers"].append(lb)
    return w, wb


def test_w8_step_with_power_of_two_scales_equals_bf16_step(orc):
    cfg = TINY.with_(dtype="w8", n_heads=8, n_kv_heads=2, head_dim=32, rope_theta=500000.0, tied=False)
    w, wb = _pow2_w8(cfg, 21)
    a = make(orc, cfg, w)
    b = make(orc, cfg.with_(dtype="bf16"), wb)
    toks = synth.gen_tokens(21, 7, cfg.vocab)
    a.prefill(toks[:-1])
    b.prefill(toks[:-1])
    la, lb = a.decode_step(int(toks[-1]), 6), b.decode_step(int(toks[-1]), 6)
    np.testing.assert_array_equal(la, lb)
    np.testing.assert_array_equal(a.k, b.k)
    np.testing.assert_array_equal(a.v, b.v)
    assert np.abs(la).max() > 0.05


def test_w8_step_matches_transformers_llama_on_dequantised_weights(orc):
    cfg = TINY.with_(dtype="w8", n_heads=8, n_kv_heads=2, head_dim=32, rope_theta=500000.0, tied=False)
    w = synth.gen_weights(cfg, seed=22, gains="random")
    m = make(orc, cfg, w)
    toks = synth.gen_tokens(22, 9, cfg.vocab)
    m.prefill(toks[:-1])
    got = m.decode_step(int(toks[-1]), len(toks) - 1)
    # float64 dequantised weights (s * q is exact in float64), bf16 gains and embedding
    f = {"embed": orc.f64_array_from_bf16(w["embed"]).astype(np.float32),
         "final_norm": orc.f64_array_from_bf16(w["final_norm"]).astype(np.float32),
         "lm_head": w["lm_head_scale"].astype(np.float64)[:, None] * w["lm_head"], "layers": []}
    for lw in w["layers"]:
        lf = {k: orc.f64_array_from_bf16(lw[k]).astype(np.float32) for k in ("attn_norm", "ffn_norm")}
        for k in synth.MATRIX_KINDS:
            lf[k] = lw[k + "_scale"].astype(np.float64)[:, None] * lw[k]
        f["layers"].append(lf)
    ref = hf_logits(orc, cfg.with_(dtype="f32"), f, toks)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-2)
    assert np.corrcoef(got, ref)[0, 1] > 0.9999


def test_w8_model_is_never_tied(orc):
    cfg = TINY.with_(dtype="w8", tied=True)
    w = synth.gen_weights(cfg.with_(tied=False), seed=23)
    with pytest.raises(AssertionError):
        make(orc, cfg, w)


def test_w8_generator_recipe():
    cfg = TINY.with_(dtype="w8", tied=False)
    w = synth.gen_weights(cfg, seed=24)
    q, s = w["layers"][0]["w_up"], w["layers"][0]["w_up_scale"]
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    assert abs(q.std() / synth.CODE_STD - 1) < 0.02
    base = synth.WEIGHT_STD / synth.CODE_STD
    assert s.dtype == np.float32 and s.shape == (cfg.ffn,)
    assert s.min() >= 0.75 * base * (1 - 1e-6) and s.max() < 1.25 * base and np.unique(s).size > cfg.ffn // 2
    assert w["embed"].dtype == np.uint16 and w["layers"][0]["attn_norm"].dtype == np.uint16
