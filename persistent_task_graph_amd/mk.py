"""ctypes binding of the C ABI in include/mk.h (argument marshalling only).

Every computation happens in libmk.so; this module only fills the C
structs and forwards pointers. It raises if the library was not built:
there is no CPU fallback.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_F32, MK_BF16, MK_W4 = 0, 1, 2
MK_KV_CONTIGUOUS, MK_KV_PAGED = 0, 1
MK_PERSISTENT, MK_KERNEL_PER_OP = 0, 1
MK_OK, MK_ERR_ARG, MK_ERR_HIP, MK_ERR_UNSUPPORTED, MK_ERR_STATE = 0, -1, -2, -3, -4
MK_ERR_TOKEN, MK_ERR_KV_OVERFLOW, MK_ERR_TIMEOUT, MK_ERR_BLOCK_TABLE = 1, 2, 4, 8

# operator ids (mk_plan_info.tasks_per_op index)
OP_QKV, OP_O, OP_GATEUP, OP_DOWN, OP_LM, OP_ATTN, OP_EMBED, OP_APPEND = 1, 2, 3, 4, 5, 6, 7, 8

EXPORTS = ["mk_build_graph", "mk_destroy_plan", "mk_last_error", "mk_plan_query", "mk_decode_step",
           "mk_decode_step_greedy", "mk_decode_step_hidden", "mk_get_device_error", "mk_argmax", "mk_plan_verify", "mk_plan_dry_run",
           "mk_plan_trace", "mk_argmax_noalloc", "mk_decode_steps_greedy", "mk_prefill", "mk_pack_tiled"]
MK_WEIGHTS_ROWS, MK_WEIGHTS_TILED = 0, 1


class ExecOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("mode", "workers", "sched_wgs", "jit", "kv_chunk", "watchdog_ms",
                                               "host_only", "device_cus", "debug_event", "debug_extra_required",
                                               "trace", "prefetch_kb", "lds_stream", "kv_chunk_max", "lds_preload",
                                               "schedule", "prefill", "down_ksplit", "o_ksplit")]


class ModelDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab")] + \
               [("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float)] + \
               [(n, ctypes.c_int32) for n in ("qk_norm", "weight_dtype", "kv_dtype", "batch", "max_seq_len", "kv_layout",
                                               "kv_block", "max_blocks_per_seq", "hidden_io")] + \
               [("opts", ExecOpts), ("weight_layout", ctypes.c_int32)]


LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)), ("n_layers", ctypes.c_int32)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("layer_stride", ctypes.c_int64),
                ("block_table", ctypes.c_void_p)]


class TraceRec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "id", "worker", "op")] + \
               [(n, ctypes.c_uint64) for n in ("t_wait", "t_ready", "t_done", "t_a", "t_b", "t_c", "t_d")]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("workers", "sched_waves", "n_aot_tasks", "n_events", "n_levels",
                                               "max_jit_tasks", "kv_chunk", "max_splits")] + \
               [("tasks_per_op", ctypes.c_int32 * 12)] + \
               [(n, ctypes.c_int64) for n in ("weight_bytes_per_step", "kv_bytes_per_token", "device_bytes")] + \
               [(n, ctypes.c_int32) for n in ("jit", "mode", "host_only", "schedule")] + \
               [("predicted_layer_us", ctypes.c_double)]


_lib = None


class MKError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libmk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MKError("libmk.so not built: run __graft_entry__.build() (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER
        L.mk_build_graph.argtypes = [P(ModelDesc)]
        L.mk_build_graph.restype = vp
        L.mk_destroy_plan.argtypes = [vp]
        L.mk_destroy_plan.restype = None
        L.mk_last_error.argtypes = []
        L.mk_last_error.restype = ctypes.c_char_p
        L.mk_plan_query.argtypes = [vp, P(PlanInfo)]
        L.mk_decode_step.argtypes = [vp, P(Weights), P(KVCache), vp, vp, vp, vp]
        L.mk_decode_step_greedy.argtypes = [vp, P(Weights), P(KVCache), vp, vp, vp, vp]
        L.mk_decode_step_hidden.argtypes = [vp, P(Weights), P(KVCache), vp, vp, vp, vp]
        L.mk_get_device_error.argtypes = [vp, vp]
        L.mk_argmax.argtypes = [vp, vp, vp, vp]
        L.mk_plan_verify.argtypes = [vp]
        L.mk_plan_dry_run.argtypes = [vp, i32, ctypes.c_uint64, i32, i32, vp]
        L.mk_plan_trace.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.mk_argmax_noalloc.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.mk_decode_steps_greedy.argtypes = [vp, P(Weights), P(KVCache), vp, vp, vp, ctypes.c_int32, vp, vp]
        L.mk_prefill.argtypes = [vp, P(Weights), P(KVCache), vp, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.mk_pack_tiled.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
        for f in ("mk_pack_tiled", "mk_argmax_noalloc", "mk_decode_steps_greedy", "mk_prefill", "mk_plan_query", "mk_decode_step", "mk_decode_step_greedy", "mk_decode_step_hidden",
                  "mk_get_device_error", "mk_argmax", "mk_plan_verify", "mk_plan_dry_run", "mk_plan_trace"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mk_last_error().decode(errors="replace")


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise MKError("%s failed (%d): %s" % (what, rc, last_error()))
    return rc


def make_desc(shape, batch: int, max_seq_len: int, *, paged: bool = False, kv_block: int = 16,
              max_blocks_per_seq: int = 0, tiled: bool = False, **opts) -> ModelDesc:
    """Fill mk_model_desc from a model shape (attributes as in synth.ModelShape).
    tiled: the layer matrices and LM head are in the tiled layout (mk_pack_tiled)."""
    d = ModelDesc()
    d.weight_layout = MK_WEIGHTS_TILED if tiled else MK_WEIGHTS_ROWS
    d.n_layers, d.hidden, d.n_heads, d.n_kv_heads = shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads
    d.head_dim, d.ffn, d.vocab = shape.head_dim, shape.ffn, shape.vocab
    d.rms_eps, d.rope_base = shape.eps, shape.rope_base
    d.qk_norm = int(bool(shape.qk_norm))
    d.weight_dtype = {"bf16": MK_BF16, "f32": MK_F32, "w4": MK_W4}[shape.wdtype]
    d.kv_dtype = MK_BF16 if shape.kv_dtype == "bf16" else MK_F32
    d.batch = batch
    d.max_seq_len = max_seq_len
    d.kv_layout = MK_KV_PAGED if paged else MK_KV_CONTIGUOUS
    d.kv_block = kv_block
    d.max_blocks_per_seq = max_blocks_per_seq or ((max_seq_len + kv_block - 1) // kv_block)
    d.hidden_io = 0 if shape.embed_head else 1
    for k, v in opts.items():
        if not hasattr(d.opts, k):
            raise TypeError("unknown exec option %r" % k)
        setattr(d.opts, k, int(v))
    return d


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor (or pass an int / None through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_live_plans: "weakref.WeakSet[Plan]" = weakref.WeakSet()


@atexit.register
def _close_live_plans() -> None:
    # free every plan while the HIP runtime is still up: atexit handlers run
    # before the interpreter tears modules down, and before the C runtime's
    # exit handlers (a profiler's among them) run
    for pl in list(_live_plans):
        pl.close()


class Plan:
    """Owns one mk_plan (task graph + device tables)."""

    def __init__(self, desc: ModelDesc):
        self.desc = desc
        h = lib().mk_build_graph(ctypes.byref(desc))
        if not h:
            raise MKError("mk_build_graph failed: " + last_error())
        self._h = h
        _live_plans.add(self)

    @property
    def handle(self) -> int:
        return self._h

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().mk_destroy_plan(self._h)
            self._h = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # no HIP call once the interpreter is finalizing: the plan was freed
        # by the atexit hook, or the process is ending and the driver takes
        # the memory back (the check is bound at definition: module globals
        # may already be gone)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> PlanInfo:
        inf = PlanInfo()
        _check(lib().mk_plan_query(self._h, ctypes.byref(inf)), "mk_plan_query")
        return inf

    def verify(self) -> None:
        _check(lib().mk_plan_verify(self._h), "mk_plan_verify")

    def dry_run(self, n_threads: int = 8, seed: int = 0, drop_task: int = -1, timeout_ms: int = 5000,
                seq_lens: Optional[Sequence[int]] = None) -> int:
        arr = None
        if seq_lens is not None:
            arr = (ctypes.c_int32 * len(seq_lens))(*[int(v) for v in seq_lens])
        rc = lib().mk_plan_dry_run(self._h, n_threads, seed, drop_task, timeout_ms,
                                   ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None)
        return rc

    def step(self, weights: "Weights", kv: "KVCache", tokens, seq_lens, logits, stream=None) -> None:
        _check(lib().mk_decode_step(self._h, ctypes.byref(weights), ctypes.byref(kv), _ptr(tokens), _ptr(seq_lens),
                                    _ptr(logits), _stream(stream)), "mk_decode_step")

    def step_greedy(self, weights: "Weights", kv: "KVCache", tokens, seq_lens, logits, stream=None) -> None:
        """One step; tokens become the greedy next tokens and seq_lens advance by one, in the same launch."""
        _check(lib().mk_decode_step_greedy(self._h, ctypes.byref(weights), ctypes.byref(kv), _ptr(tokens),
                                           _ptr(seq_lens), _ptr(logits), _stream(stream)), "mk_decode_step_greedy")

    def steps_greedy(self, weights: "Weights", kv: "KVCache", tokens, seq_lens, logits, n_steps: int,
                     out_tokens=None, stream=None) -> None:
        """n_steps greedy steps in one launch; out_tokens [n_steps, batch] receives each step's tokens."""
        _check(lib().mk_decode_steps_greedy(self._h, ctypes.byref(weights), ctypes.byref(kv), _ptr(tokens),
                                            _ptr(seq_lens), _ptr(logits), int(n_steps), _ptr(out_tokens),
                                            _stream(stream)), "mk_decode_steps_greedy")

    def prefill(self, weights: "Weights", kv: "KVCache", tokens, pos0: int, T: int, logits, stream=None) -> None:
        """T prompt tokens of one sequence, a chunk of `batch` positions per launch (plan built with prefill=1)."""
        _check(lib().mk_prefill(self._h, ctypes.byref(weights), ctypes.byref(kv), _ptr(tokens), int(pos0), int(T),
                                _ptr(logits), _stream(stream)), "mk_prefill")

    def step_hidden(self, weights: "Weights", kv: "KVCache", x_in, seq_lens, x_out, stream=None) -> None:
        _check(lib().mk_decode_step_hidden(self._h, ctypes.byref(weights), ctypes.byref(kv), _ptr(x_in),
                                           _ptr(seq_lens), _ptr(x_out), _stream(stream)), "mk_decode_step_hidden")

    def device_error(self, stream=None) -> int:
        return _check(lib().mk_get_device_error(self._h, _stream(stream)), "mk_get_device_error")

    def trace(self, max_records: int = 1 << 20, stream=None):
        """Task trace of the last persistent step as a numpy structured array."""
        import numpy as np

        buf = (TraceRec * max_records)()
        n = _check(lib().mk_plan_trace(self._h, ctypes.cast(buf, ctypes.c_void_p), max_records, _stream(stream)),
                   "mk_plan_trace")
        dt = np.dtype([("kind", "<i4"), ("id", "<i4"), ("worker", "<i4"), ("op", "<i4"), ("t_wait", "<u8"),
                       ("t_ready", "<u8"), ("t_done", "<u8"), ("t_a", "<u8"), ("t_b", "<u8"),
                       ("t_c", "<u8"), ("t_d", "<u8")])
        return np.frombuffer(bytes(buf)[: n * ctypes.sizeof(TraceRec)], dtype=dt).copy()

    def argmax(self, logits, out_tokens, stream=None) -> None:
        _check(lib().mk_argmax(self._h, _ptr(logits), _ptr(out_tokens), _stream(stream)), "mk_argmax")


def argmax_noalloc(logits, out_tokens, batch: int, vocab: int, stream=None) -> None:
    """mk_argmax_noalloc: greedy tokens of `batch` rows of `vocab` logits, no plan, no allocation."""
    _check(lib().mk_argmax_noalloc(_ptr(logits), int(batch), int(vocab), _ptr(out_tokens), _stream(stream)),
           "mk_argmax_noalloc")


def pack_tiled(src, dst, rows: int, cols: int, stream=None) -> None:
    """mk_pack_tiled: tiled copy of a row-major bf16 [rows, cols] matrix into dst (device)."""
    _check(lib().mk_pack_tiled(_ptr(src), _ptr(dst), int(rows), int(cols), _stream(stream)), "mk_pack_tiled")


def make_weights(layer_ptrs, embed=None, final_norm=None, lm_head=None) -> Weights:
    """layer_ptrs: list of dicts name -> device pointer (int) or tensor."""
    n = len(layer_ptrs)
    arr = (LayerWeights * n)()
    for i, lp in enumerate(layer_ptrs):
        for name in LAYER_FIELDS:
            setattr(arr[i], name, _ptr(lp.get(name)))
    w = Weights()
    w.embed, w.final_norm, w.lm_head = _ptr(embed), _ptr(final_norm), _ptr(lm_head)
    w.layers = arr
    w.n_layers = n
    w._keep = arr  # keep the array alive with the struct
    return w


def make_kv(k, v, layer_stride: int, block_table=None) -> KVCache:
    kv = KVCache()
    kv.k, kv.v = _ptr(k), _ptr(v)
    kv.layer_stride = int(layer_stride)
    kv.block_table = _ptr(block_table)
    return kv
