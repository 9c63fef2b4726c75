"""Pins for the oracle's operators, each against something other than the
oracle itself: hand-worked values, closed forms, invariants, or a library
routine for a special case.  CPU only."""
import math

import numpy as np
import pytest
import torch


# ---- bfloat16 storage rounding ------------------------------------------------

@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (3.140625, 0x4049),
    (1.0 + 2.0 ** -8, 0x3F80),              # exact tie -> even (0x3F80)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),          # exact tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 3 * 2.0 ** -9, 0x3F81),          # 0.75 ulp above 1 -> up
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie: no double rounding via binary32
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -133, 0x0001),                  # smallest bfloat16 subnormal
    (2.0 ** -134, 0x0000),                  # half of it: tie -> even (zero)
    (0.75 * 2.0 ** -133, 0x0001),
    (3.3895313892515355e38, 0x7F7F),        # largest finite
    (3.40282346638528859e38, 0x7F80),       # float32 max rounds past it -> inf
    (math.inf, 0x7F80),
    (-math.inf, 0xFF80),
])
def test_bf16_rne_known_cases(orc, value, bits):
    assert orc.bf16_from_f64(value) == bits


def test_bf16_nan_stays_nan(orc):
    b = orc.bf16_from_f64(float("nan"))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0


def test_bf16_matches_torch_for_binary32_inputs(orc):
    # For inputs exactly representable in binary32 there is no double
    # rounding, so torch's float32 -> bfloat16 conversion (RNE) must agree.
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = orc.bf16_array_from_f64(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_widen_is_exact(orc):
    for bits, val in [(0x3F80, 1.0), (0x4049, 3.140625), (0xC000, -2.0), (0x0001, 2.0 ** -133)]:
        assert orc.f64_from_bf16(bits) == val


# ---- RMSNorm ---------------------------------------------------------------------

def test_rmsnorm_unit_rms_before_gain(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1000) * 0.3
    g = (1.0 + 0.1 * rng.standard_normal(1000)).astype(np.float32)
    eps = 1e-5
    y = orc.rmsnorm(x, g, eps)
    ms = np.mean(x * x)
    rms_before_gain = np.sqrt(np.mean((y / g.astype(np.float64)) ** 2))
    assert rms_before_gain == pytest.approx(math.sqrt(ms / (ms + eps)), rel=1e-13)
    # eps = 0: exactly unit RMS
    y0 = orc.rmsnorm(x, np.ones(1000, np.float32), 0.0)
    assert np.sqrt(np.mean(y0 ** 2)) == pytest.approx(1.0, rel=1e-14)


def test_rmsnorm_constant_vector(orc):
    c, eps = 0.37, 1e-5
    g = np.array([1.0, 2.0, -0.5, 0.25], np.float32)
    y = orc.rmsnorm(np.full(4, c), g, eps)
    np.testing.assert_allclose(y, g.astype(np.float64) * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_rmsnorm_applies_bf16_gain(orc):
    g = np.array([0x3F80, 0x4000, 0xBF00], np.uint16)  # 1, 2, -0.5
    y = orc.rmsnorm(np.array([1.0, 1.0, 1.0]), g, 0.0)
    np.testing.assert_allclose(y, [1.0, 2.0, -0.5], rtol=1e-15)


# ---- GEMV --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_matches_numpy_matmul_nonsquare(orc, dtype):
    rng = np.random.default_rng(3)
    rows, cols = 37, 53  # non-square: a transposed operand cannot pass
    Wf = rng.standard_normal((rows, cols)) * 0.02
    if dtype == "f32":
        W = Wf.astype(np.float32)
        W64 = W.astype(np.float64)
    else:
        W = orc.bf16_array_from_f64(Wf)
        W64 = orc.f64_array_from_bf16(W)
    h = rng.standard_normal(cols)
    np.testing.assert_allclose(orc.gemv(W, h), W64 @ h, rtol=1e-12, atol=1e-15)


def test_gemv_brute_force_exact_sum(orc):
    # Tiny brute force: the exactly rounded sum (math.fsum) of the products.
    rng = np.random.default_rng(4)
    W = rng.standard_normal((5, 7)).astype(np.float32)
    h = rng.standard_normal(7)
    y = orc.gemv(W, h)
    for r in range(5):
        ref = math.fsum(float(W[r, c]) * float(h[c]) for c in range(7))
        assert y[r] == pytest.approx(ref, rel=1e-14, abs=1e-15)


def test_gemv_identity_and_one_hot(orc):
    h = np.arange(1, 9, dtype=np.float64) / 7.0
    np.testing.assert_array_equal(orc.gemv(np.eye(8, dtype=np.float32), h), h)
    W = np.arange(24, dtype=np.float32).reshape(3, 8)
    e = np.zeros(8)
    e[5] = 1.0
    np.testing.assert_array_equal(orc.gemv(W, e), W[:, 5].astype(np.float64))


# ---- RoPE ----------------------------------------------------------------------------

def test_rope_hand_example():
    import oracle as orc
    # d = 4, theta = 1e4: pair (0,2) turns by p*1, pair (1,3) by p*1e4^(-1/2) = p*0.01.
    out = orc.rope([1.0, 0.0, 0.0, 0.0], 1, 4, 1, 1e4)
    np.testing.assert_allclose(out, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], atol=1e-15)
    out = orc.rope([0.0, 1.0, 0.0, 0.0], 1, 4, 1, 1e4)
    np.testing.assert_allclose(out, [0.0, math.cos(0.01), 0.0, math.sin(0.01)], atol=1e-15)
    out = orc.rope([0.0, 0.0, 1.0, 0.0], 1, 4, 3, 1e4)  # second element of pair 0
    np.testing.assert_allclose(out, [-math.sin(3.0), 0.0, math.cos(3.0), 0.0], atol=1e-15)


def test_rope_identity_at_zero_and_pair_norms(orc):
    rng = np.random.default_rng(5)
    nh, d = 3, 64
    v = rng.standard_normal(nh * d)
    np.testing.assert_array_equal(orc.rope(v, nh, d, 0, 5e5), v)
    r = orc.rope(v, nh, d, 1234, 5e5)
    a = v.reshape(nh, 2, d // 2)
    b = r.reshape(nh, 2, d // 2)
    np.testing.assert_allclose(np.hypot(b[:, 0], b[:, 1]), np.hypot(a[:, 0], a[:, 1]), rtol=1e-13)


def test_rope_pair_angles(orc):
    # Each pair (i, i+d/2) of a unit vector (1, 0) turns by pos * theta^(-2i/d).
    d, pos, theta = 16, 7, 10000.0
    v = np.zeros(d)
    v[: d // 2] = 1.0
    r = orc.rope(v, 1, d, pos, theta)
    for i in range(d // 2):
        ang = pos * theta ** (-2.0 * i / d)
        assert math.atan2(r[i + d // 2], r[i]) == pytest.approx(math.remainder(ang, 2 * math.pi), abs=1e-12)


def test_rope_relative_position_property(orc):
    rng = np.random.default_rng(6)
    d, theta = 64, 10000.0
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for p, pp in [(5, 2), (100, 37), (40, 40)]:
        lhs = orc.rope(q, 1, d, p, theta) @ orc.rope(k, 1, d, pp, theta)
        rhs = orc.rope(q, 1, d, p - pp, theta) @ k
        assert lhs == pytest.approx(rhs, rel=1e-11, abs=1e-11)


# ---- softmax / attention -------------------------------------------------------------

def test_softmax_sums_to_one_and_shift_invariance(orc):
    rng = np.random.default_rng(7)
    s = rng.standard_normal(300) * 5
    p = orc.softmax(s)
    assert p.sum() == pytest.approx(1.0, abs=1e-14)
    np.testing.assert_allclose(orc.softmax(s + 123.0), p, rtol=1e-12)
    np.testing.assert_allclose(orc.softmax([0.0, math.log(2.0)]), [1 / 3, 2 / 3], rtol=1e-15)
    np.testing.assert_allclose(orc.softmax([1000.0, 1000.0]), [0.5, 0.5])  # overflow protection


def test_attention_single_token_returns_v(orc):
    rng = np.random.default_rng(8)
    d = 64
    K = orc.bf16_array_from_f64(rng.standard_normal((1, d)))
    V = orc.bf16_array_from_f64(rng.standard_normal((1, d)))
    o = orc.attend(rng.standard_normal(d) * 10, K, V)
    np.testing.assert_array_equal(o, orc.f64_array_from_bf16(V[0]))


def test_attention_equal_keys_give_mean_of_v(orc):
    rng = np.random.default_rng(9)
    n, d = 11, 16
    K = np.tile(rng.standard_normal(d).astype(np.float32), (n, 1))
    V = rng.standard_normal((n, d)).astype(np.float32)
    o = orc.attend(rng.standard_normal(d), K, V)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_two_token_hand_example(orc):
    # d = 2, so scores are q.k / sqrt(2).  q = (sqrt(2) ln 3, 0), k0 = 0,
    # k1 = (1, 0): scores 0 and ln 3 -> weights 1/4, 3/4.
    q = [math.sqrt(2.0) * math.log(3.0), 0.0]
    K = np.array([[0.0, 0.0], [1.0, 0.0]], np.float32)
    V = np.array([[4.0, 0.0], [0.0, 8.0]], np.float32)
    np.testing.assert_allclose(orc.attend(q, K, V), [1.0, 6.0], rtol=1e-14)


# ---- SiLU / argmax ---------------------------------------------------------------------

def test_silu_values(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert orc.silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-15)
    for z in (0.3, 2.5, 11.0):  # silu(z) - silu(-z) = z
        assert orc.silu(z) - orc.silu(-z) == pytest.approx(z, rel=1e-14)
    assert orc.silu(60.0) == pytest.approx(60.0, rel=1e-15)


def test_argmax_lowest_index_on_ties(orc):
    assert orc.argmax([0.0, 3.0, 1.0, 3.0]) == 1
    assert orc.argmax([-5.0]) == 0
    assert orc.argmax([2.0, 2.0]) == 0
