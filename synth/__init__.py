"""Seeded synthetic inputs for the decode-step workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It holds no arithmetic of the decode step: it only produces
weights, KV-cache contents, token ids, sequence lengths and block tables
from fixed seeds, with the shapes and value distributions of the workloads
(8B-class decoder shapes with random N(0, 0.02) weights, N(0, 1) KV).

Random numbers come from the counter-based generator in ``synth.c``
(SplitMix64 words, Box-Muller normals), so results do not depend on the
thread count. Norm gains are 1.0 for the workloads (the N(0, 0.02) draw
applies to matrices); tests that must tell one gain vector from another ask
for ``gains="random"``: every gain vector (attention, MLP, final, per-head q
and k) then holds its own seeded draw from 1 + N(0, 0.25).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# fixed seeds per input family
SEED_WEIGHTS = 0
SEED_KV = 1
SEED_TOKENS = 2
SEED_LENGTHS = 3
SEED_BLOCKS = 4
SEED_HIDDEN = 5

BF16_ONE = 0x3F80


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, dbl, dbl, i64, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, dbl, dbl, i64, vp]
        lib.synth_uniform_int.argtypes = [u64, u64, i64, i64, i64, vp]
        lib.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
        lib.synth_codes_u4.argtypes = [u64, u64, dbl, i64, vp]
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------
# raw generators


def normal(seed: int, stream: int, shape, std: float = 1.0, dtype: str = "bf16", mean: float = 0.0) -> np.ndarray:
    """N(mean, std) array; dtype 'bf16' returns uint16 bit patterns, 'f32' float32."""
    n = int(np.prod(shape)) if len(shape) else 1
    lib = _load()
    if dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(seed, stream, mean, std, n, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(seed, stream, mean, std, n, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform_int(seed: int, stream: int, lo: int, hi: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    _load().synth_uniform_int(seed, stream, lo, hi, n, out.ctypes.data)
    return out


def uniform01(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(seed, stream, n, out.ctypes.data)
    return out


# ----------------------------------------------------------------------------
# 4-bit weight matrices (W4A16)
#
# One buffer per [rows, cols] matrix: the 4-bit codes in row order, two per
# byte (low nibble first), rows * cols / 2 bytes; then, from that size
# rounded up to 256 bytes, one bf16 scale per group of W4_GROUP inputs of a
# row, [rows][cols / W4_GROUP]. The weight is (code - 8) * scale.
W4_GROUP = 128
# codes of N(0, 2.5^2) values rounded and clamped to [-8, 7] (offset 8):
# (code - 8) then has mean -0.0013 and rms 2.5096 (exact sums over the
# normal distribution), so scales of std / 2.5096 give the weights about the
# standard deviation of the bf16 matrices
W4_CODE_SIGMA = 2.5
W4_SCALE_PER_STD = 1.0 / 2.5096


def w4_scale_offset(rows: int, cols: int) -> int:
    return (rows * cols // 2 + 255) // 256 * 256


def w4_matrix(seed: int, stream: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """Seeded W4 matrix buffer: codes of N(0, W4_CODE_SIGMA^2) values under
    symmetric 4-bit quantization (offset 8, clamped to [0, 15]); group scales
    |N(1, 0.25)| * std * W4_SCALE_PER_STD in bf16, so that the dequantized
    matrix has rms about std and mean about zero."""
    assert cols % W4_GROUP == 0 and cols % 2 == 0
    off = w4_scale_offset(rows, cols)
    buf = np.zeros(off + rows * (cols // W4_GROUP) * 2, dtype=np.uint8)
    _load().synth_codes_u4(seed, stream, W4_CODE_SIGMA, rows * cols // 2, buf.ctypes.data)
    sc = normal(seed, stream + (1 << 40), (rows * (cols // W4_GROUP),), 0.25, "f32", mean=1.0)
    sc = np.abs(sc) * np.float32(std * W4_SCALE_PER_STD)
    buf[off:] = f32_to_bf16(sc).view(np.uint8)
    return buf


def w4_dequant(buf: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """float64 [rows, cols] weights of a W4 buffer (for tests)."""
    q = buf[: rows * cols // 2]
    codes = np.empty(rows * cols, dtype=np.int64)
    codes[0::2] = q & 15
    codes[1::2] = q >> 4
    off = w4_scale_offset(rows, cols)
    sc = bf16_to_f32(buf[off: off + rows * (cols // W4_GROUP) * 2].view(np.uint16)).astype(np.float64)
    w = (codes.reshape(rows, cols) - 8).astype(np.float64)
    return w * np.repeat(sc.reshape(rows, cols // W4_GROUP), W4_GROUP, axis=1)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even narrowing of float32 to bf16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (b & 0x7F800000) == 0x7F800000
    nan &= (b & 0x007FFFFF) != 0
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return r


# ----------------------------------------------------------------------------
# model shapes and workloads


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    eps: float = 1e-6
    rope_base: float = 10000.0
    qk_norm: bool = True
    wdtype: str = "bf16"  # 'bf16', 'f32', or 'w4' (4-bit layer matrices; gains, embedding, LM head bf16)
    kv_dtype: str = "bf16"
    embed_head: bool = True  # False: hidden-state in/out (one layer, no embedding / LM head)

    @property
    def qdim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kvdim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def kv_bytes_per_token_layer(self) -> int:
        es = 2 if self.kv_dtype == "bf16" else 4
        return 2 * self.kvdim * es

    def layer_weight_bytes(self) -> int:
        es = 4 if self.wdtype == "f32" else 2
        H, F = self.hidden, self.ffn
        norms = 2 * H + (2 * self.head_dim if self.qk_norm else 0)
        if self.wdtype == "w4":
            dims = [(self.qdim, H), (self.kvdim, H), (self.kvdim, H), (H, self.qdim), (F, H), (F, H), (H, F)]
            # codes and scales (the 256-byte alignment pad is not read)
            return sum(r * c // 2 + r * (c // W4_GROUP) * 2 for r, c in dims) + norms * 2
        mats = (self.qdim + 2 * self.kvdim) * H + H * self.qdim + 3 * F * H
        return (mats + norms) * es

    def step_weight_bytes(self) -> int:
        """Weight bytes one decode step streams (embedding rows not included)."""
        es = 4 if self.wdtype == "f32" else 2
        b = self.n_layers * self.layer_weight_bytes()
        if self.embed_head:
            b += self.vocab * self.hidden * es + self.hidden * es
        return b


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int
    steps: int
    kv_len: str  # 'fixed:N', 'loguniform:lo:hi', 'uniform:lo:hi'
    prompt: int = 0  # >0: prefill this many teacher-forced tokens instead of random KV
    paged: bool = False
    kv_block: int = 16

    def capacity(self) -> int:
        """KV capacity per sequence needed for the whole run."""
        kind, *a = self.kv_len.split(":")
        hi = int(a[-1])
        return max(hi, self.prompt) + self.steps + 1


TINY = ModelShape(n_layers=2, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=1024, vocab=1024,
                  qk_norm=False, wdtype="f32", kv_dtype="f32")
Q8B = ModelShape(n_layers=36, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288, vocab=151936)
Q8B_LAYER = replace(Q8B, n_layers=1, embed_head=False)
Q8B_W4 = replace(Q8B, wdtype="w4")

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, batch=1, steps=16, kv_len="fixed:32"),
    "layer8b": Workload("layer8b", Q8B_LAYER, batch=1, steps=64, kv_len="fixed:512"),
    "q8b_b1": Workload("q8b_b1", Q8B, batch=1, steps=128, kv_len="fixed:1024", prompt=1024),
    "q8b_b16": Workload("q8b_b16", Q8B, batch=16, steps=64, kv_len="loguniform:32:4096"),
    "q8b_b8_paged": Workload("q8b_b8_paged", Q8B, batch=8, steps=32, kv_len="uniform:4096:16384", paged=True),
    "q8b_w4_b1": Workload("q8b_w4_b1", Q8B_W4, batch=1, steps=128, kv_len="fixed:1024"),
}


# ----------------------------------------------------------------------------
# generators for the workloads

# matrix ids inside one layer (stream = layer * 32 + id)
_MATS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]
_STREAM_EMBED = 1_000_001
_STREAM_LM = 1_000_002
_STREAM_FINAL_GAIN = 1_000_003
# gain vector ids inside one layer (stream = layer * 32 + 16 + id)
_GAINS = ["attn_norm", "mlp_norm", "q_norm", "k_norm"]
GAIN_STD = 0.25


def _gain(n: int, wdtype: str, gains: str = "unit", seed: int = SEED_WEIGHTS, stream: int = 0) -> np.ndarray:
    """Norm gain vector: all ones ('unit') or a seeded 1 + N(0, GAIN_STD) draw ('random')."""
    if gains == "random":
        return normal(seed, stream, (n,), GAIN_STD, wdtype, mean=1.0)
    if gains != "unit":
        raise ValueError(gains)
    if wdtype == "bf16":
        return np.full(n, BF16_ONE, dtype=np.uint16)
    return np.ones(n, dtype=np.float32)


def layer_weights(shape: ModelShape, layer: int, seed: int = SEED_WEIGHTS, std: float = 0.02,
                  gains: str = "unit") -> Dict[str, np.ndarray]:
    H, F, D = shape.hidden, shape.ffn, shape.head_dim
    dims = {"wq": (shape.qdim, H), "wk": (shape.kvdim, H), "wv": (shape.kvdim, H), "wo": (H, shape.qdim),
            "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F)}
    out = {}
    for i, name in enumerate(_MATS):
        if shape.wdtype == "w4":
            out[name] = w4_matrix(seed, layer * 32 + i, dims[name][0], dims[name][1], std)
        else:
            out[name] = normal(seed, layer * 32 + i, dims[name], std, shape.wdtype)
    gt = "bf16" if shape.wdtype == "w4" else shape.wdtype
    names = ["attn_norm", "mlp_norm"] + (["q_norm", "k_norm"] if shape.qk_norm else [])
    for name in names:
        n = D if name in ("q_norm", "k_norm") else H
        out[name] = _gain(n, gt, gains, seed, layer * 32 + 16 + _GAINS.index(name))
    return out


def model_weights(shape: ModelShape, seed: int = SEED_WEIGHTS, std: float = 0.02, gains: str = "unit") -> Dict[str, object]:
    """Weights of a model: matrices N(0, std); norm gains per `gains` ('unit' or 'random')."""
    w: Dict[str, object] = {"layers": [layer_weights(shape, l, seed, std, gains) for l in range(shape.n_layers)]}
    if shape.embed_head:
        et = "bf16" if shape.wdtype == "w4" else shape.wdtype
        w["embed"] = normal(seed, _STREAM_EMBED, (shape.vocab, shape.hidden), std, et)
        w["lm_head"] = normal(seed, _STREAM_LM, (shape.vocab, shape.hidden), std, et)
        w["final_norm"] = _gain(shape.hidden, et, gains, seed, _STREAM_FINAL_GAIN)
    return w


def with_gains(shape: ModelShape, weights: Dict[str, object], gains: str = "random",
               seed: int = SEED_WEIGHTS) -> Dict[str, object]:
    """Shallow copy of `weights` whose norm gains are replaced by the `gains`
    draw (the same vectors model_weights(shape, seed, gains=gains) makes);
    the matrices are shared, not copied."""
    H, D = shape.hidden, shape.head_dim
    out: Dict[str, object] = {k: v for k, v in weights.items() if k != "layers"}
    layers = []
    for l, lw in enumerate(weights["layers"]):
        nl = dict(lw)
        gt = "bf16" if shape.wdtype == "w4" else shape.wdtype
        for name in ["attn_norm", "mlp_norm"] + (["q_norm", "k_norm"] if shape.qk_norm else []):
            n = D if name in ("q_norm", "k_norm") else H
            nl[name] = _gain(n, gt, gains, seed, l * 32 + 16 + _GAINS.index(name))
        layers.append(nl)
    out["layers"] = layers
    if shape.embed_head:
        out["final_norm"] = _gain(H, "bf16" if shape.wdtype == "w4" else shape.wdtype, gains, seed, _STREAM_FINAL_GAIN)
    return out


def seq_lengths(wl: Workload, seed: int = SEED_LENGTHS) -> np.ndarray:
    """Initial KV length per sequence."""
    kind, *a = wl.kv_len.split(":")
    B = wl.batch
    if kind == "fixed":
        return np.full(B, int(a[0]), dtype=np.int64)
    lo, hi = int(a[0]), int(a[1])
    if kind == "uniform":
        return uniform_int(seed, 0, lo, hi, B)
    if kind == "loguniform":
        u = uniform01(seed, 1, B)
        v = np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return np.clip(np.rint(v).astype(np.int64), lo, hi)
    raise ValueError(kind)


def kv_sequence(shape: ModelShape, b: int, n: int, capacity: int, seed: int = SEED_KV) -> Dict[str, np.ndarray]:
    """KV cache of sequence b of a workload: k, v arrays [n_layers, n_kv_heads,
    capacity, head_dim] (cache dtype); positions < n hold N(0, 1) values, the
    rest are zero. The random stream depends on (b, layer, head, k/v) only, so
    one sequence can be generated without the others."""
    L, Hkv, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    dt = np.uint16 if shape.kv_dtype == "bf16" else np.float32
    n = int(n)
    seq = {}
    for kind, kid in (("k", 0), ("v", 1)):
        arr = np.zeros((L, Hkv, capacity, D), dtype=dt)
        for l in range(L):
            for h in range(Hkv):
                stream = ((b * 4096 + l) * 256 + h) * 2 + kid
                arr[l, h, :n] = normal(seed, stream, (n, D), 1.0, shape.kv_dtype)
        seq[kind] = arr
    return seq


def kv_contents(shape: ModelShape, lengths: np.ndarray, capacity: int, seed: int = SEED_KV) -> List[Dict[str, np.ndarray]]:
    """Per sequence b: kv_sequence(shape, b, lengths[b], capacity)."""
    return [kv_sequence(shape, b, int(n), capacity, seed) for b, n in enumerate(lengths)]


def tokens(wl: Workload, n: Optional[int] = None, seed: int = SEED_TOKENS, stream: int = 0) -> np.ndarray:
    n = wl.batch if n is None else n
    return uniform_int(seed, stream, 0, wl.shape.vocab - 1, n).astype(np.int32)


def hidden_inputs(shape: ModelShape, batch: int, step: int, seed: int = SEED_HIDDEN) -> np.ndarray:
    """N(0, 1) hidden-state input for hidden-I/O workloads, per step."""
    return normal(seed, step, (batch, shape.hidden), 1.0, "f32")


def block_table(lengths_cap: List[int], block: int, seed: int = SEED_BLOCKS) -> np.ndarray:
    """Random permutation of a pool of ceil(cap_b / block) blocks per sequence.

    Returns [B, max_blocks] int32 (unused entries = -1).
    """
    nblk = [(int(c) + block - 1) // block for c in lengths_cap]
    pool = sum(nblk)
    # Fisher-Yates with the counter generator
    perm = np.arange(pool, dtype=np.int64)
    if pool > 1:
        r = uniform_int(seed, 0, 0, (1 << 62), pool)
        for i in range(pool - 1, 0, -1):
            j = int(r[i] % (i + 1))
            perm[i], perm[j] = perm[j], perm[i]
    mb = max(nblk)
    tab = np.full((len(nblk), mb), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        tab[b, :n] = perm[o:o + n]
        o += n
    return tab
