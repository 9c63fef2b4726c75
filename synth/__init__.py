"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

This module only *produces inputs*: model shapes for the five workloads, random
weights, norm gains, prompt token ids and (optionally) synthetic KV-cache
contents.  It holds none of the decode-step arithmetic.  Values come from the
counter-based Philox4x32-10 generator in ``synth.c`` keyed by a seed and a
per-tensor stream id, so every tensor (or slice of one) can be regenerated
independently.

Weights follow the recipe of the workloads: i.i.d. N(0, 0.02^2) (0.02 read as
the standard deviation), stored as float32 for the tiny model and as bfloat16
(round-to-nearest-even) otherwise.  Norm gains are 1.0 unless ``gains="random"``
(1 + 0.1 * N(0,1), used by tests so a dropped gain cannot hide).  Prompt tokens
are uniform over [0, vocab).

Weight-only INT8 workloads (dtype "w8") keep the embedding, the gains and the
KV cache in bfloat16 and give every matrix (the LM head included; such a
model is never tied) as int8 codes with one float32 scale per output row.
The codes are N(0, 32^2) draws rounded to integers and clamped to
[-127, 127] -- the shape of the codes that max-abs quantisation of a Gaussian
row leaves -- and the scales are uniform in [0.75, 1.25) * 0.02 / 32, so the
dequantised weights have about the 0.02 standard deviation of the other
workloads while every row has its own scale.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP-parallel, -O2)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.synth_normal.restype = None
        lib.synth_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_uniform_int.restype = None
        lib.synth_uniform_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.synth_uniform_f32.restype = None
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox4x32_10.restype = None
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------
# Model shapes and workloads
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    dtype: str            # "f32" or "bf16": weights and KV cache; "w8": int8 matrices, bf16 rest
    tied: bool            # LM head shares the token-embedding matrix
    context: int          # prompt tokens prefilled into the KV cache
    decode_steps: int     # greedy decode steps after the prompt
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def max_seq(self) -> int:
        # A C-token context is a prompt of C+1 tokens: positions 0..C-1 are
        # prefilled and decode step k feeds position C+k.
        return self.context + self.decode_steps

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def wbytes(self) -> int:
        """Bytes per element of the embedding, the gains and the KV cache."""
        return 4 if self.dtype == "f32" else 2

    @property
    def mbytes(self) -> int:
        """Bytes per element of the layer matrices and the LM head."""
        return 1 if self.dtype == "w8" else self.wbytes

    def weight_bytes_per_step(self) -> int:
        """Every weight read once per step: all layer matrices (with their
        per-row scales for INT8) and gains, the final gain, the LM head and
        one embedding row."""
        H, F = self.hidden, self.ffn
        mat = (self.q_dim + 2 * self.kv_dim) * H + H * self.q_dim + 3 * H * F
        rows = (self.q_dim + 2 * self.kv_dim) + H + 2 * F + H  # output rows of the seven matrices
        per_layer = mat * self.mbytes + 2 * H * self.wbytes + (4 * rows if self.dtype == "w8" else 0)
        head = self.vocab * H * self.mbytes + (4 * self.vocab if self.dtype == "w8" else 0)
        return self.n_layers * per_layer + head + 2 * H * self.wbytes

    def kv_read_bytes(self, pos: int) -> int:
        """K and V bytes read by attention at decode position pos (0..pos)."""
        return self.wbytes * 2 * self.n_layers * self.kv_dim * (pos + 1)

    def step_bytes(self, pos: int) -> int:
        return self.weight_bytes_per_step() + self.kv_read_bytes(pos)

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": ModelConfig("tiny", 2, 256, 4, 2, 64, 688, 1024, 1e-5, 10000.0, "f32", False, 64, 16),
    "llama1b": ModelConfig("llama1b", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 500000.0, "bf16", True, 2048, 128),
    "llama8b": ModelConfig("llama8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "bf16", False, 2048, 128),
    "llama1b_32k": ModelConfig("llama1b_32k", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 500000.0, "bf16", True, 32768, 64),
    "llama70b": ModelConfig("llama70b", 80, 8192, 64, 8, 128, 28672, 128256, 1e-5, 500000.0, "bf16", False, 4096, 32),
    # weight-only INT8 versions of the 1B and 8B shapes (own int8 LM head)
    "llama1b_w8": ModelConfig("llama1b_w8", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 500000.0, "w8", False, 2048, 128),
    "llama8b_w8": ModelConfig("llama8b_w8", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "w8", False, 2048, 128),
}

WEIGHT_STD = 0.02
CODE_STD = 32.0  # int8 codes of the "w8" workloads

# Stream ids: one per tensor so each can be regenerated on its own.
LAYER_KINDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
_STREAM_EMBED, _STREAM_FINAL_NORM, _STREAM_LM_HEAD = 1, 2, 3
_STREAM_TOKENS = 0x70000000
_STREAM_KV = 0x60000000
_STREAM_SCALE = 0x50000000  # + the matrix's stream: its per-row INT8 scales


def layer_stream(layer: int, kind: str) -> int:
    return 16 + 16 * layer + LAYER_KINDS.index(kind)


def layer_shapes(cfg: ModelConfig) -> dict:
    H, F = cfg.hidden, cfg.ffn
    return {
        "attn_norm": (H,), "wq": (cfg.q_dim, H), "wk": (cfg.kv_dim, H), "wv": (cfg.kv_dim, H),
        "wo": (H, cfg.q_dim), "ffn_norm": (H,), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }


def _np_dtype(cfg: ModelConfig):
    return np.float32 if cfg.dtype == "f32" else np.uint16  # bf16 stored as raw bits


def _code(cfg: ModelConfig) -> int:
    return 0 if cfg.dtype == "f32" else 1


_STORE = {"f32": (np.float32, 0), "bf16": (np.uint16, 1), "i8": (np.int8, 2)}


def normal(seed: int, stream: int, shape, std: float, mean: float = 0.0, dtype: str = "bf16",
           out: np.ndarray | None = None, offset: int = 0) -> np.ndarray:
    """mean + std*N(0,1) for elements [offset, offset+size) of a stream,
    stored as dtype "f32", "bf16" (bits) or "i8" (rounded, clamped codes)."""
    n = int(np.prod(shape))
    npdt, code = _STORE[dtype]
    if out is None:
        out = np.empty(shape, dtype=npdt)
    assert out.dtype == npdt and out.size == n and out.flags["C_CONTIGUOUS"]
    _load().synth_normal(seed, stream, offset, n, mean, std, code, out.ctypes.data_as(ctypes.c_void_p))
    return out


def uniform_f32(seed: int, stream: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_uniform_f32(seed, stream, 0, n, lo, hi, out.ctypes.data_as(ctypes.c_void_p))
    return out


def gen_tensor(cfg: ModelConfig, seed: int, name: str, layer: int | None = None,
               gains: str = "ones", out: np.ndarray | None = None) -> np.ndarray:
    """One weight tensor of the model, row-major [out][in]."""
    H = cfg.hidden
    if layer is not None:
        shape = layer_shapes(cfg)[name]
        stream = layer_stream(layer, name)
        is_gain = name in ("attn_norm", "ffn_norm")
    elif name == "embed":
        shape, stream, is_gain = (cfg.vocab, H), _STREAM_EMBED, False
    elif name == "lm_head":
        shape, stream, is_gain = (cfg.vocab, H), _STREAM_LM_HEAD, False
    elif name == "final_norm":
        shape, stream, is_gain = (H,), _STREAM_FINAL_NORM, True
    else:
        raise KeyError(name)
    store = "f32" if cfg.dtype == "f32" else "bf16"  # embedding, gains
    if is_gain and gains == "ones":
        arr = np.empty(shape, dtype=_np_dtype(cfg)) if out is None else out
        arr[...] = 1.0 if cfg.dtype == "f32" else 0x3F80  # bf16 bits of 1.0
        return arr
    if is_gain:
        return normal(seed, stream, shape, 0.1, 1.0, store, out)
    if cfg.dtype == "w8" and name != "embed":  # a matrix: int8 codes
        return normal(seed, stream, shape, CODE_STD, 0.0, "i8", out)
    return normal(seed, stream, shape, WEIGHT_STD, 0.0, store, out)


def gen_scale(cfg: ModelConfig, seed: int, name: str, layer: int | None = None) -> np.ndarray:
    """Per-row float32 scales of an INT8 matrix ("w8" workloads)."""
    assert cfg.dtype == "w8"
    if layer is not None:
        rows, stream = layer_shapes(cfg)[name][0], layer_stream(layer, name)
    elif name == "lm_head":
        rows, stream = cfg.vocab, _STREAM_LM_HEAD
    else:
        raise KeyError(name)
    base = WEIGHT_STD / CODE_STD
    return uniform_f32(seed, _STREAM_SCALE + stream, rows, 0.75 * base, 1.25 * base)


MATRIX_KINDS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def gen_layer(cfg: ModelConfig, seed: int, layer: int, gains: str = "ones") -> dict:
    """One layer's tensors (and, for "w8", the matrices' "<kind>_scale")."""
    lw = {k: gen_tensor(cfg, seed, k, layer=layer, gains=gains) for k in LAYER_KINDS}
    if cfg.dtype == "w8":
        for k in MATRIX_KINDS:
            lw[k + "_scale"] = gen_scale(cfg, seed, k, layer)
    return lw


def gen_weights(cfg: ModelConfig, seed: int = 0, gains: str = "ones") -> dict:
    """All weights as host numpy arrays: {'embed', 'final_norm', 'lm_head'
    (absent when tied), 'layers': [ {kind: array} ]}."""
    w = {"embed": gen_tensor(cfg, seed, "embed"), "final_norm": gen_tensor(cfg, seed, "final_norm", gains=gains)}
    if not cfg.tied:
        w["lm_head"] = gen_tensor(cfg, seed, "lm_head")
        if cfg.dtype == "w8":
            w["lm_head_scale"] = gen_scale(cfg, seed, "lm_head")
    w["layers"] = [gen_layer(cfg, seed, l, gains) for l in range(cfg.n_layers)]
    return w


def gen_tokens(seed: int, n: int, vocab: int, sub: int = 0) -> np.ndarray:
    """n prompt token ids, uniform over [0, vocab)."""
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_int(seed, _STREAM_TOKENS + sub, 0, n, vocab, out.ctypes.data_as(ctypes.c_void_p))
    return out


def kv_std(cfg: ModelConfig) -> float:
    """Scale of K/V entries of a random-init model: a unit-RMS normed input
    times N(0, 0.02^2) rows gives N(0, 0.02^2 * hidden)."""
    return WEIGHT_STD * float(np.sqrt(cfg.hidden))


def gen_kv_prefix(cfg: ModelConfig, seed: int, n_pos: int, which: str, layer: int,
                  out: np.ndarray | None = None) -> np.ndarray:
    """Synthetic cache contents for positions [0, n_pos) of one layer,
    shape [n_kv_heads][n_pos][head_dim], stream (layer, K or V)."""
    stream = _STREAM_KV + 2 * layer + (0 if which == "k" else 1)
    return normal(seed, stream, (cfg.n_kv_heads, n_pos, cfg.head_dim), kv_std(cfg), 0.0,
                  "f32" if cfg.dtype == "f32" else "bf16", out)


def philox4x32_10(ctr, key) -> list:
    """Raw generator block (for its known-answer test)."""
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _load().synth_philox4x32_10(c, k, o)
    return list(o)
