"""CPU oracle for the batch-1 decode step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
shares no code with the GPU library.  The arithmetic lives in ``oracle.c``
(plain float64 C); this module only marshals numpy arrays.

Parity status of each function (how it is pinned, see tests/test_oracle_*.py):
  bf16 rounding, rmsnorm, gemv, gemv_q8, rope, softmax, attend, silu, argmax,
  decode_step (all three dtypes), prefill: pinned by closed forms, hand-worked examples, library
  special cases and invariants.  Full-model logits beyond those pins have no
  printed values on the pages to compare against.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


class _Model(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("rms_eps", ctypes.c_double),
                ("rope_theta", ctypes.c_double), ("dtype", ctypes.c_int32), ("tied", ctypes.c_int32),
                ("scales", ctypes.c_void_p)]


def build(force: bool = True) -> str:
    """Compile liboracle.so (gcc, -O2, no FP contraction, OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        v, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        sig = {
            "or_f64_from_bf16": ([ctypes.c_uint16], dbl),
            "or_bf16_from_f64": ([dbl], ctypes.c_uint16),
            "or_rmsnorm": ([v, i32, v, i32, dbl, v], None),
            "or_gemv": ([v, i32, i32, i32, v, v], None),
            "or_gemv_q8": ([v, v, i32, i32, v, v], None),
            "or_rope": ([v, i32, i32, i32, dbl], None),
            "or_softmax": ([v, i32, v], None),
            "or_attend": ([v, v, v, i32, i32, i32, v], None),
            "or_silu": ([dbl], dbl),
            "or_argmax": ([v, i32], i32),
            "or_decode_step": ([ctypes.POINTER(_Model), v, v, v, i32, i32, v], i32),
            "or_prefill": ([ctypes.POINTER(_Model), v, v, v, v, i32, i32], i32),
            "or_num_threads": ([], i32),
            "or_set_num_threads": ([i32], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, res
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"weights must be float32 or uint16 (bfloat16 bits), got {a.dtype}")


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---- storage conversions -----------------------------------------------------

def bf16_from_f64(x: float) -> int:
    return int(_load().or_bf16_from_f64(float(x)))


def f64_from_bf16(b: int) -> float:
    return float(_load().or_f64_from_bf16(int(b)))


def bf16_array_from_f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    f = _load().or_bf16_from_f64
    return np.array([f(float(x)) for x in a.ravel()], dtype=np.uint16).reshape(a.shape)


def f64_array_from_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # exact widening


# ---- operators -----------------------------------------------------------------

def rmsnorm(x, g: np.ndarray, eps: float) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _load().or_rmsnorm(_p(x), x.size, _p(g), _dt(g), float(eps), _p(y))
    return y


def gemv(W: np.ndarray, h) -> np.ndarray:
    h = _f64(h)
    rows, cols = W.shape
    assert h.size == cols
    y = np.empty(rows, dtype=np.float64)
    _load().or_gemv(_p(W), _dt(W), rows, cols, _p(h), _p(y))
    return y


def gemv_q8(q: np.ndarray, s: np.ndarray, h) -> np.ndarray:
    """Weight-only INT8 product: int8 codes q [rows][cols], float32 scales
    s [rows]; returns (s[:, None] * q) @ h in float64."""
    q = np.ascontiguousarray(q)
    s = np.ascontiguousarray(s)
    assert q.dtype == np.int8 and s.dtype == np.float32
    h = _f64(h)
    rows, cols = q.shape
    assert h.size == cols and s.shape == (rows,)
    y = np.empty(rows, dtype=np.float64)
    _load().or_gemv_q8(_p(q), _p(s), rows, cols, _p(h), _p(y))
    return y


def rope(v, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    v = _f64(v).copy()
    assert v.size == n_heads * head_dim
    _load().or_rope(_p(v), n_heads, head_dim, pos, float(theta))
    return v


def softmax(s) -> np.ndarray:
    s = _f64(s)
    p = np.empty_like(s)
    _load().or_softmax(_p(s), s.size, _p(p))
    return p


def attend(q, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """q [d]; K, V [n_pos][d] float32 or bf16 bits."""
    q = _f64(q)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    n_pos, d = K.shape
    o = np.empty(d, dtype=np.float64)
    _load().or_attend(_p(q), _p(K), _p(V), _dt(K), d, n_pos, _p(o))
    return o


def silu(z: float) -> float:
    return float(_load().or_silu(float(z)))


def num_threads() -> int:
    """OpenMP threads the oracle's row loops use."""
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's row loops from now on (timing only)."""
    _load().or_set_num_threads(int(n))


def argmax(v) -> int:
    v = _f64(v)
    return int(_load().or_argmax(_p(v), v.size))


# ---- whole model -----------------------------------------------------------------

LAYER_KINDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class Model:
    """Shapes plus host weights (numpy, row-major [out][in]) and the oracle's
    own KV cache arrays [n_layers][n_kv_heads][max_seq][head_dim].

    shape["dtype"] is "f32", "bf16" or "w8".  A "w8" model (weight-only
    INT8) holds each matrix as int8 codes under its usual key and its
    float32 per-row scales under "<key>_scale" (the LM head as "lm_head" and
    "lm_head_scale"; such a model is never tied); the embedding and the gains
    are bf16 bits, and so is the cache."""

    def __init__(self, shape: dict, weights: dict, max_seq: int):
        self.shape = dict(shape)
        self.max_seq = int(max_seq)
        dt = {"f32": 0, "bf16": 1, "w8": 2}[shape["dtype"]]
        q8 = dt == 2
        assert not (q8 and shape["tied"]), "a weight-only INT8 model has its own LM head"
        self._keep = []
        ptrs, sptrs = [], []

        def add(a, matrix=False, scale=None):
            if a is None:
                ptrs.append(None)
                sptrs.append(None)
                return
            a = np.ascontiguousarray(a)
            if q8 and matrix:
                assert a.dtype == np.int8, "INT8 model matrices are int8 codes"
                sc = np.ascontiguousarray(scale, dtype=np.float32)
                assert sc.shape == (a.shape[0],), "one scale per output row"
                self._keep.append(sc)
                sptrs.append(sc.ctypes.data)
            else:
                assert _dt(a) == min(dt, 1), "weight dtype must match the model dtype"
                sptrs.append(None)
            self._keep.append(a)
            ptrs.append(a.ctypes.data)

        add(weights["embed"])
        add(weights["final_norm"])
        if shape["tied"]:
            add(None)
        else:
            add(weights["lm_head"], True, weights.get("lm_head_scale"))
        assert len(weights["layers"]) == shape["n_layers"]
        for lw in weights["layers"]:
            for k in LAYER_KINDS:
                mat = k not in ("attn_norm", "ffn_norm")
                add(lw[k], mat, lw.get(k + "_scale") if mat else None)
        self._ptrs = (ctypes.c_void_p * len(ptrs))(*ptrs)
        self._sptrs = (ctypes.c_void_p * len(sptrs))(*sptrs)
        self._m = _Model(shape["n_layers"], shape["hidden"], shape["n_heads"], shape["n_kv_heads"],
                         shape["head_dim"], shape["ffn"], shape["vocab"], self.max_seq,
                         float(shape["rms_eps"]), float(shape["rope_theta"]), dt, int(bool(shape["tied"])),
                         ctypes.cast(self._sptrs, ctypes.c_void_p) if q8 else None)
        npdt = np.uint16 if dt else np.float32
        cache_shape = (shape["n_layers"], shape["n_kv_heads"], self.max_seq, shape["head_dim"])
        self.k = np.zeros(cache_shape, dtype=npdt)
        self.v = np.zeros(cache_shape, dtype=npdt)

    def decode_step(self, token: int, pos: int, want_logits: bool = True):
        logits = np.empty(self.shape["vocab"], dtype=np.float64) if want_logits else None
        rc = _load().or_decode_step(ctypes.byref(self._m), self._ptrs, _p(self.k), _p(self.v), int(token),
                                    int(pos), _p(logits) if want_logits else None)
        if rc != 0:
            raise ValueError(f"or_decode_step failed with code {rc}")
        return logits

    def prefill(self, tokens, start_pos: int = 0) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        rc = _load().or_prefill(ctypes.byref(self._m), self._ptrs, _p(self.k), _p(self.v), _p(t), t.size,
                                int(start_pos))
        if rc != 0:
            raise ValueError(f"or_prefill failed with code {rc}")
