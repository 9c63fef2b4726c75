"""The C ABI without a GPU: the library loads, exports every entry point that
include/mk.h declares, and rejects bad arguments on the host before any
device work (no call here reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")

import torch  # noqa: E402,F401  (one HIP runtime per process: torch loads it first)

import transformer_megakernel_persistent_amd.mk as mkb  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mkb.LIB_PATH):
        from transformer_megakernel_persistent_amd.build import build
        build()
    return mkb.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mk_\w+)\s*\(", text, flags=re.M)))


def header_enum(name_prefix):
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(rf"({name_prefix}\w*)\s*=\s*(\d+)", text)}


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(mkb.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_and_dtype_values_match_binding():
    st = header_enum("MK_ERR_") | header_enum("MK_OK")
    for k, v in st.items():
        assert getattr(mkb, k) == v, k
    dt = header_enum("MK_F32") | header_enum("MK_BF16") | header_enum("MK_W8")
    assert dt == {"MK_F32": mkb.MK_F32, "MK_BF16": mkb.MK_BF16, "MK_W8": mkb.MK_W8}
    assert [f for f, _ in mkb.LayerPtrs._fields_[9:]] == ["s_" + k for k in mkb.MATRIX_KINDS]


def test_status_strings(lib):
    seen = set()
    for s in range(0, 11):
        txt = lib.mk_status_str(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 11
    assert lib.mk_status_str(99).decode() == "unknown status"


def _desc(**over):
    shape = dict(n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=64, ffn=128, vocab=100,
                 rms_eps=1e-5, rope_theta=10000.0, dtype="bf16", tied=True)
    d = mkb.model_desc(shape, 32)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _weights(n_layers, null_field=None):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    layers = (mkb.LayerPtrs * n_layers)()
    for l in range(n_layers):
        layers[l] = mkb.LayerPtrs(*[None if k == null_field else fake.value for k in mkb.LAYER_KINDS])
    w = mkb.WeightPtrs(fake.value, fake.value, None, layers)
    return w, layers


def _create(lib, desc, weights, tuning=None):
    h = ctypes.c_void_p(0xDEAD)
    rc = lib.mk_create(ctypes.byref(desc) if desc is not None else None,
                       ctypes.byref(weights) if weights is not None else None,
                       ctypes.byref(tuning) if tuning is not None else None, ctypes.byref(h))
    return rc, h


def test_create_rejects_null_arguments(lib):
    w, _keep = _weights(2)
    assert lib.mk_create(None, None, None, None) == mkb.MK_ERR_NULL
    rc, h = _create(lib, None, w)
    assert rc == mkb.MK_ERR_NULL and h.value is None  # *out is cleared on failure
    rc, _ = _create(lib, _desc(), None)
    assert rc == mkb.MK_ERR_NULL
    w2, _keep2 = _weights(2, null_field="w_down")
    assert _create(lib, _desc(), w2)[0] == mkb.MK_ERR_NULL
    w3, _keep3 = _weights(2)
    assert _create(lib, _desc(tied_embeddings=0), w3)[0] == mkb.MK_ERR_NULL  # untied needs lm_head


def test_int8_models_need_scales_and_their_own_head(lib):
    fake = ctypes.c_void_p(0x1000).value  # never dereferenced: validation fails first
    layers = (mkb.LayerPtrs * 2)()
    for l in range(2):
        layers[l] = mkb.LayerPtrs(*[fake] * 9, *[fake] * 7)
    w = mkb.WeightPtrs(fake, fake, fake, layers, fake)
    # weight-only INT8 with a tied head: the int8 LM head is its own matrix
    assert _create(lib, _desc(dtype=mkb.MK_W8, tied_embeddings=1), w)[0] == mkb.MK_ERR_SHAPE
    w_nohs = mkb.WeightPtrs(fake, fake, fake, layers, None)
    assert _create(lib, _desc(dtype=mkb.MK_W8, tied_embeddings=0), w_nohs)[0] == mkb.MK_ERR_NULL
    layers[1] = mkb.LayerPtrs(*[fake] * 9, *[fake] * 6, None)  # no w_down scales
    assert _create(lib, _desc(dtype=mkb.MK_W8, tied_embeddings=0), w)[0] == mkb.MK_ERR_NULL


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), mkb.MK_ERR_DTYPE),
    (dict(head_dim=96), mkb.MK_ERR_SHAPE),          # 192 bytes per head row
    (dict(n_heads=6, n_kv_heads=4), mkb.MK_ERR_SHAPE),  # heads not a multiple of kv heads
    (dict(n_heads=6, n_kv_heads=2), mkb.MK_ERR_SHAPE),  # group of 3
    (dict(hidden=60), mkb.MK_ERR_SHAPE),
    (dict(ffn=0), mkb.MK_ERR_SHAPE),
    (dict(n_layers=0), mkb.MK_ERR_SHAPE),
    (dict(vocab=0), mkb.MK_ERR_SHAPE),
    (dict(max_seq=0), mkb.MK_ERR_SHAPE),
    (dict(rope_theta=0.0), mkb.MK_ERR_SHAPE),
    (dict(rms_eps=-1.0), mkb.MK_ERR_SHAPE),
])
def test_create_rejects_bad_shapes(lib, over, status):
    n_layers = over.get("n_layers", 2) or 1
    w, _keep = _weights(n_layers)
    assert _create(lib, _desc(**over), w)[0] == status


@pytest.mark.parametrize("over", [dict(grid=-1), dict(grid=1025), dict(ring_slots=2), dict(ring_slots=10),
                                  dict(attn_splits=-3), dict(attn_splits=65), dict(timeout_ms=-1), dict(cooperative=3),
                                  dict(trace=2), dict(prefetch_depth=-1), dict(stage_drain=2),
                                  dict(prefill_chunk=-2), dict(prefill_chunk=4097), dict(attn_pm_slots=-2),
                                  dict(slots_per_step=-1), dict(slots_per_step=3)])
def test_create_rejects_bad_tuning(lib, over):
    w, _keep = _weights(2)
    assert _create(lib, _desc(), w, mkb.Tuning(**over))[0] == mkb.MK_ERR_TUNING


def test_calls_on_a_null_handle(lib):
    kv = mkb.KVDesc(None, None, 32)
    buf = (ctypes.c_int32 * 4)()
    assert lib.mk_decode_step(None, 0, 0, ctypes.byref(kv), buf, None) == mkb.MK_ERR_NULL
    assert lib.mk_decode_step_device_token(None, buf, 0, ctypes.byref(kv), None, buf, None) == mkb.MK_ERR_NULL
    assert lib.mk_decode_step_device_token_noalloc(None, buf, 0, ctypes.byref(kv), None, buf, None) == mkb.MK_ERR_NULL
    assert lib.mk_prefill_kv(None, buf, 1, 0, ctypes.byref(kv), None) == mkb.MK_ERR_NULL
    assert lib.mk_get_device_error(None) == mkb.MK_ERR_NULL
    assert lib.mk_get_info(None, ctypes.byref(mkb.Info())) == mkb.MK_ERR_NULL
    assert lib.mk_read_trace(None, buf, 4) == mkb.MK_ERR_NULL
    lib.mk_destroy(None)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(mkb, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        mkb.load_library(str(tmp_path / "libmk.so"))


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "transformer_megakernel_persistent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "or_decode_step" not in text and "liboracle" not in text, f


def test_deferred_create_and_load_reject_bad_arguments(lib):
    h = ctypes.c_void_p(0xDEAD)
    assert lib.mk_create_deferred(None, None, ctypes.byref(h)) == mkb.MK_ERR_NULL and h.value is None
    assert lib.mk_create_deferred(ctypes.byref(_desc()), None, None) == mkb.MK_ERR_NULL
    assert lib.mk_create_deferred(ctypes.byref(_desc(head_dim=96)), None, ctypes.byref(h)) == mkb.MK_ERR_SHAPE
    assert lib.mk_create_deferred(ctypes.byref(_desc()), ctypes.byref(mkb.Tuning(ring_slots=2)),
                                  ctypes.byref(h)) == mkb.MK_ERR_TUNING
    w, _keep = _weights(1)
    assert lib.mk_load_weights(None, ctypes.byref(w), 0, 1) == mkb.MK_ERR_NULL
