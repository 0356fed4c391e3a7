"""Python wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU path. It imports nothing
from the GPU package; weights, caches and tokens are passed in as numpy
arrays (bf16 as uint16 bit patterns, or float32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, W4 = 0, 1, 2


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("qk_norm", ctypes.c_int), ("wtype", ctypes.c_int),
                ("mtype", ctypes.c_int), ("kvtype", ctypes.c_int), ("eps", ctypes.c_double),
                ("rope_base", ctypes.c_double)]


_LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]


class _Layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_rmsnorm.argtypes = [vp, i, vp, i, d, vp]
        lib.orc_matvec.argtypes = [vp, i, i, i, vp, vp]
        lib.orc_rope.argtypes = [vp, i, i, d]
        lib.orc_swiglu.argtypes = [vp, vp, i, vp]
        lib.orc_attention_head.argtypes = [vp, vp, vp, i, i, i, vp, vp]
        lib.orc_layer_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Layer), vp, vp, i, i, vp]
        lib.orc_model_forward.argtypes = [ctypes.POINTER(_Cfg), vp, ctypes.POINTER(_Layer), vp, vp, vp, vp, i, i, i,
                                          vp]
        lib.orc_model_forward.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [i]
        lib.orc_get_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _tcode(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("oracle arrays must be uint16 (bf16 bits) or float32, got %s" % a.dtype)


def _c(a: np.ndarray) -> np.ndarray:
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return a


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ---------------------------------------------------------------- primitives

def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = _c(np.ascontiguousarray(x, dtype=np.float32))
    y = np.empty_like(x)
    _load().orc_rmsnorm(x.ctypes.data, x.size, _c(gain).ctypes.data, _tcode(gain), eps, y.ctypes.data)
    return y


def matvec(W: np.ndarray, x: np.ndarray, w4_shape=None) -> np.ndarray:
    """y = W x. W: [rows, cols] float32 / bf16 bits, or a W4 buffer (uint8,
    one dimension) with w4_shape = (rows, cols)."""
    W = _c(W)
    x = _c(np.ascontiguousarray(x, dtype=np.float32))
    if w4_shape is not None:
        rows, cols = w4_shape
        t = W4
    else:
        rows, cols = W.shape
        t = _tcode(W)
    assert x.size == cols
    y = np.empty(rows, dtype=np.float32)
    _load().orc_matvec(W.ctypes.data, t, rows, cols, x.ctypes.data, y.ctypes.data)
    return y


def rope(v: np.ndarray, pos: int, base: float = 10000.0) -> np.ndarray:
    v = np.array(v, dtype=np.float32, copy=True)
    _load().orc_rope(v.ctypes.data, v.size, int(pos), base)
    return v


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    out = np.empty_like(g)
    _load().orc_swiglu(g.ctypes.data, u.ctypes.data, g.size, out.ctypes.data)
    return out


def attention_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, return_probs: bool = False):
    q = np.ascontiguousarray(q, dtype=np.float32)
    K, V = _c(K), _c(V)
    n, D = K.shape
    assert V.shape == (n, D) and q.size == D and K.dtype == V.dtype
    out = np.empty(D, dtype=np.float32)
    probs = np.empty(max(n, 1), dtype=np.float64)
    _load().orc_attention_head(q.ctypes.data, K.ctypes.data, V.ctypes.data, _tcode(K), n, D, out.ctypes.data,
                               probs.ctypes.data)
    return (out, probs[:n]) if return_probs else out


# ---------------------------------------------------------------- model

class Oracle:
    """Sequential decoder forward for one sequence at a time.

    ``shape`` provides n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn,
    vocab, eps, rope_base, qk_norm; ``weights`` is the dict produced by the
    synthetic-input module (``layers`` list + embed / lm_head / final_norm).
    Caches are per sequence: dict(k=[n_layers, Hkv, cap, D], v=...).
    """

    _MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

    def __init__(self, shape, weights: Dict):
        self.shape = shape
        self.w = weights
        layers = weights["layers"]
        self._keep = []
        self._layers = (_Layer * len(layers))()
        wt = None
        w4 = getattr(shape, "wdtype", "") == "w4"
        for li, lw in enumerate(layers):
            for name in _LAYER_FIELDS:
                a = lw.get(name)
                if a is None:
                    setattr(self._layers[li], name, None)
                    continue
                a = _c(a)
                self._keep.append(a)
                if w4 and name in self._MATS:
                    if a.dtype != np.uint8 or a.ndim != 1:
                        raise TypeError("W4 matrices are one-dimensional uint8 buffers")
                else:
                    t = _tcode(a)
                    wt = t if wt is None else wt
                    if t != wt:
                        raise TypeError("mixed weight types")
                setattr(self._layers[li], name, a.ctypes.data)
        self.wtype = wt
        self.cfg = _Cfg(shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                        shape.vocab, int(bool(shape.qk_norm)), wt, W4 if w4 else wt,
                        BF16 if shape.kv_dtype == "bf16" else F32, float(shape.eps), float(shape.rope_base))

    def _check_cache(self, cache):
        k, v = _c(cache["k"]), _c(cache["v"])
        want = np.uint16 if self.shape.kv_dtype == "bf16" else np.float32
        assert k.dtype == want and v.dtype == want and k.shape == v.shape
        return k, v, k.shape[2]

    def layer_forward(self, layer: int, cache, pos: int, x: np.ndarray) -> np.ndarray:
        """One layer; cache holds all layers; returns the new hidden state."""
        k, v, cap = self._check_cache(cache)
        assert 0 <= pos < cap
        x = np.array(x, dtype=np.float32, copy=True)
        kc = k[layer]
        vc = v[layer]
        _load().orc_layer_forward(ctypes.byref(self.cfg), ctypes.byref(self._layers[layer]), kc.ctypes.data,
                                  vc.ctypes.data, cap, int(pos), x.ctypes.data)
        return x

    def model_forward(self, cache, token: int, pos: int) -> np.ndarray:
        """Full step (embedding .. logits) for one sequence; appends to cache."""
        k, v, cap = self._check_cache(cache)
        assert 0 <= pos < cap
        logits = np.empty(self.shape.vocab, dtype=np.float32)
        rc = _load().orc_model_forward(ctypes.byref(self.cfg), _c(self.w["embed"]).ctypes.data, self._layers,
                                       _c(self.w["final_norm"]).ctypes.data, _c(self.w["lm_head"]).ctypes.data,
                                       k.ctypes.data, v.ctypes.data, cap, int(token), int(pos), logits.ctypes.data)
        if rc != 0:
            raise ValueError("token out of range: %d" % token)
        return logits

    def hidden_forward(self, cache, pos: int, x: np.ndarray) -> np.ndarray:
        """All layers on a hidden state (no embedding / LM head)."""
        for l in range(self.shape.n_layers):
            x = self.layer_forward(l, cache, pos, x)
        return x
