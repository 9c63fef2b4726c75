"""The input generator: known-answer vectors of Philox4x32-10 (published
with the algorithm by Salmon et al., SC'11, in the Random123 distribution),
determinism, slice independence and the distribution of the draws."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("ctr,key,out", [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, out):
    assert synth.philox4x32_10(ctr, key) == out


def test_slices_regenerate_identically():
    full = synth.normal(3, 9, (1000,), 0.02, dtype="f32")
    part = synth.normal(3, 9, (333,), 0.02, dtype="f32", offset=501)
    np.testing.assert_array_equal(full[501:834], part)
    np.testing.assert_array_equal(full, synth.normal(3, 9, (1000,), 0.02, dtype="f32"))
    assert not np.array_equal(full, synth.normal(4, 9, (1000,), 0.02, dtype="f32"))


def test_normal_moments_and_bf16_rounding():
    a = synth.normal(0, 5, (1 << 20,), 0.02, dtype="f32").astype(np.float64)
    assert abs(a.mean()) < 1e-4 and a.std() == pytest.approx(0.02, rel=5e-3)
    b = synth.normal(0, 5, (1 << 12,), 0.02, dtype="bf16")
    widened = (b.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_allclose(widened, a[: 1 << 12], rtol=2.0 ** -8)


def test_tokens_in_range():
    t = synth.gen_tokens(0, 5000, 128256)
    assert t.min() >= 0 and t.max() < 128256 and len(np.unique(t)) > 4800


def test_workload_byte_counts():
    c = synth.CONFIGS["llama1b"]
    # 16 layers x 60,821,504 + 128256 x 2048 + 2 x 2048 elements, 2 bytes each
    assert c.weight_bytes_per_step() == 2_471_632_896
    assert c.kv_read_bytes(2048) == 2 * 2 * 16 * 512 * 2049
    assert synth.CONFIGS["llama1b"].max_seq == 2176
