"""ctypes binding of libmk.so (include/mk.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
converts torch tensors to device pointers and torch streams to hipStream_t.
torch must be imported before the library is loaded so that both share one
HIP runtime in the process.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK, MK_ERR_NULL, MK_ERR_SHAPE, MK_ERR_DTYPE, MK_ERR_RANGE = 0, 1, 2, 3, 4
MK_ERR_NOMEM, MK_ERR_HIP, MK_ERR_DEVICE, MK_ERR_STATE, MK_ERR_TUNING, MK_ERR_SCRATCH = 5, 6, 7, 8, 9, 10
MK_STATIC_SCRATCH_BYTES = 64 * 1024 * 1024
MK_F32, MK_BF16, MK_W8 = 0, 1, 2
DTYPES = {"f32": MK_F32, "bf16": MK_BF16, "w8": MK_W8}

EXPORTED = ("mk_create", "mk_create_deferred", "mk_load_weights", "mk_decode_step", "mk_decode_step_device_token",
            "mk_decode_step_device_token_noalloc", "mk_prefill_kv", "mk_get_device_error", "mk_get_info",
            "mk_read_trace", "mk_status_str", "mk_destroy")


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("rms_eps", ctypes.c_double),
                ("rope_theta", ctypes.c_double), ("dtype", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32)]


MATRIX_KINDS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class LayerPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up",
                                               "w_down")] + [("s_" + n, ctypes.c_void_p) for n in MATRIX_KINDS]


class WeightPtrs(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerPtrs)), ("lm_head_scale", ctypes.c_void_p)]


class KVDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("max_seq", ctypes.c_int32)]


class Tuning(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("ring_slots", ctypes.c_int32), ("attn_splits", ctypes.c_int32),
                ("timeout_ms", ctypes.c_int32), ("cooperative", ctypes.c_int32), ("trace", ctypes.c_int32),
                ("prefetch_depth", ctypes.c_int32), ("stage_drain", ctypes.c_int32),
                ("prefill_chunk", ctypes.c_int32), ("attn_pm_slots", ctypes.c_int32),
                ("slots_per_step", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("ring_slots", ctypes.c_int32), ("attn_splits", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("cu_count", ctypes.c_int32),
                ("prefetch_slots", ctypes.c_int32), ("packed_bytes", ctypes.c_int64), ("weight_bytes", ctypes.c_int64),
                ("record_bytes", ctypes.c_int64), ("prefill_chunk", ctypes.c_int32),
                ("slots_per_step", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmk.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with transformer_megakernel_persistent_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
    sig = {
        "mk_create": ([p(ModelDesc), p(WeightPtrs), p(Tuning), p(vp)], ctypes.c_int),
        "mk_create_deferred": ([p(ModelDesc), p(Tuning), p(vp)], ctypes.c_int),
        "mk_load_weights": ([vp, p(WeightPtrs), i32, i32], ctypes.c_int),
        "mk_decode_step": ([vp, i32, i32, p(KVDesc), vp, vp], ctypes.c_int),
        "mk_decode_step_device_token": ([vp, vp, i32, p(KVDesc), vp, vp, vp], ctypes.c_int),
        "mk_decode_step_device_token_noalloc": ([vp, vp, i32, p(KVDesc), vp, vp, vp], ctypes.c_int),
        "mk_prefill_kv": ([vp, vp, i32, i32, p(KVDesc), vp], ctypes.c_int),
        "mk_get_device_error": ([vp], ctypes.c_int),
        "mk_get_info": ([vp, p(Info)], ctypes.c_int),
        "mk_read_trace": ([vp, vp, ctypes.c_int64], ctypes.c_int),
        "mk_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "mk_destroy": ([vp], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    _lib = lib
    return lib


class MkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {load_library().mk_status_str(status).decode()} (status {status})")


def _check(status: int, what: str):
    if status != MK_OK:
        raise MkError(status, what)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def model_desc(shape: dict, max_seq: int) -> ModelDesc:
    return ModelDesc(shape["n_layers"], shape["hidden"], shape["n_heads"], shape["n_kv_heads"], shape["head_dim"],
                     shape["ffn"], shape["vocab"], int(max_seq), float(shape["rms_eps"]), float(shape["rope_theta"]),
                     DTYPES[shape["dtype"]], int(bool(shape["tied"])))


class KVCache:
    """Caller-owned contiguous cache: K and V each [n_layers][n_kv_heads][max_seq][head_dim]."""

    def __init__(self, shape: dict, max_seq: int, device="cuda", fill: float | None = 0.0):
        dt = torch.float32 if shape["dtype"] == "f32" else torch.bfloat16  # "w8" keeps a bf16 cache
        size = (shape["n_layers"], shape["n_kv_heads"], int(max_seq), shape["head_dim"])
        self.k = torch.empty(size, dtype=dt, device=device)
        self.v = torch.empty(size, dtype=dt, device=device)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)
        self.max_seq = int(max_seq)

    def desc(self) -> KVDesc:
        return KVDesc(self.k.data_ptr(), self.v.data_ptr(), self.max_seq)


LAYER_KINDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class MegaKernel:
    """A created handle.  `weights` holds device tensors (row-major [out][in])
    in the model dtype: 'embed', 'final_norm', optional 'lm_head' and
    'layers' (a list of dicts keyed by LAYER_KINDS).  A "w8" model's
    matrices are int8 tensors with float32 per-row scales under
    '<kind>_scale' (and 'lm_head_scale')."""

    def __init__(self, shape: dict, weights: dict | None, max_seq: int, tuning: dict | None = None):
        """weights=None creates the handle with mk_create_deferred; the
        weights then come through load_weights."""
        lib = load_library()
        self.shape = dict(shape)
        self.max_seq = int(max_seq)
        self._desc = model_desc(shape, max_seq)
        tun = Tuning(**(tuning or {}))
        h = ctypes.c_void_p()
        if weights is None:
            _check(lib.mk_create_deferred(ctypes.byref(self._desc), ctypes.byref(tun), ctypes.byref(h)),
                   "mk_create_deferred")
        else:
            wp, _layers = _weight_ptrs(weights)
            _check(lib.mk_create(ctypes.byref(self._desc), ctypes.byref(wp), ctypes.byref(tun), ctypes.byref(h)),
                   "mk_create")
        self._h = h

    def load_weights(self, weights: dict, first_layer: int = 0):
        """Pre-lay out weights['layers'] as layers first_layer.. and, if
        weights has 'embed', the head tensors (mk_load_weights)."""
        wp, _layers = _weight_ptrs(weights)
        n = len(weights.get("layers", []))
        _check(load_library().mk_load_weights(self._h, ctypes.byref(wp), int(first_layer), n), "mk_load_weights")

    # -- the four calls of the boundary --
    def decode_step(self, token: int, pos: int, kv: KVCache, logits: torch.Tensor, stream=None):
        d = kv.desc()
        _check(load_library().mk_decode_step(self._h, int(token), int(pos), ctypes.byref(d), _ptr(logits),
                                             _stream(stream)), "mk_decode_step")

    def decode_step_device_token(self, token_in: torch.Tensor, pos: int, kv: KVCache, logits, token_out, stream=None):
        d = kv.desc()
        _check(load_library().mk_decode_step_device_token(self._h, _ptr(token_in), int(pos), ctypes.byref(d),
                                                          _ptr(logits), _ptr(token_out), _stream(stream)),
               "mk_decode_step_device_token")

    def decode_step_device_token_noalloc(self, token_in: torch.Tensor, pos: int, kv: KVCache, logits, token_out,
                                         stream=None):
        d = kv.desc()
        _check(load_library().mk_decode_step_device_token_noalloc(self._h, _ptr(token_in), int(pos), ctypes.byref(d),
                                                                  _ptr(logits), _ptr(token_out), _stream(stream)),
               "mk_decode_step_device_token_noalloc")

    def prefill_kv(self, tokens, start_pos: int, kv: KVCache, stream=None):
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        d = kv.desc()
        _check(load_library().mk_prefill_kv(self._h, arr, len(tokens), int(start_pos), ctypes.byref(d),
                                            _stream(stream)), "mk_prefill_kv")

    def device_error(self) -> int:
        return load_library().mk_get_device_error(self._h)

    def info(self) -> dict:
        inf = Info()
        _check(load_library().mk_get_info(self._h, ctypes.byref(inf)), "mk_get_info")
        return {f: getattr(inf, f) for f, _ in Info._fields_}

    def read_trace(self):
        """Stage timeline of the last step as a numpy array [grid][5L+2][4]
        of wall-clock ticks (handle created with tuning trace=1)."""
        import numpy as np
        n_b = 5 * self.shape["n_layers"] + 2
        grid = self.info()["grid"]
        n_stage, n_steps = grid * n_b * 4, grid * 64 * 2
        raw = np.zeros(n_stage + n_steps + grid * 96 * 2, dtype=np.uint64)
        _check(load_library().mk_read_trace(self._h, raw.ctypes.data_as(ctypes.c_void_p), raw.size), "mk_read_trace")
        # consumer 0's layer-1 data steps (barrier exit, compute done) and
        # loader 0's layer-1 barriers (arrival, exit)
        self.last_steps = raw[n_stage:n_stage + n_steps].reshape(grid, 64, 2)
        self.last_loader = raw[n_stage + n_steps:].reshape(grid, 96, 2)
        return raw[:grid * n_b * 4].reshape(grid, n_b, 4)

    def close(self):
        if getattr(self, "_h", None):
            load_library().mk_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _weight_ptrs(weights: dict):
    layers_in = weights.get("layers", [])
    layers = (LayerPtrs * max(len(layers_in), 1))()
    for l, lw in enumerate(layers_in):
        layers[l] = LayerPtrs(*[_ptr(lw[k]) for k in LAYER_KINDS], *[_ptr(lw.get(k + "_scale")) for k in MATRIX_KINDS])
    wp = WeightPtrs(_ptr(weights.get("embed")), _ptr(weights.get("final_norm")), _ptr(weights.get("lm_head")),
                    layers if layers_in else None, _ptr(weights.get("lm_head_scale")))
    return wp, layers


def upload_weights(host: dict, device="cuda") -> dict:
    """Host numpy weights (float32, uint16 bfloat16 bits, int8 codes) -> device tensors."""
    import numpy as np

    def up(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(np.ascontiguousarray(a))
        return t.to(device)

    out = {k: up(v) for k, v in host.items() if k != "layers"}
    out["layers"] = [{k: up(v) for k, v in lw.items()} for lw in host.get("layers", [])]
    return out
