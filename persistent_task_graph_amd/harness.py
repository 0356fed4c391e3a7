"""Device-side setup for tests and benchmarks: torch tensors holding the
weights and KV cache, and the C-ABI structs pointing at them.

torch provides device memory and streams only; every step of the decode
path runs in libmk.so.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import mk


def _torch():
    import torch

    return torch


def to_device(a: np.ndarray, device="cuda"):
    """numpy array (uint16 bf16 bits or float32) -> device tensor with the same bits."""
    torch = _torch()
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def from_device(t) -> np.ndarray:
    torch = _torch()
    a = t.detach().cpu().numpy()
    if t.dtype == torch.int16:
        return a.view(np.uint16)
    return a


TILED_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class DeviceModel:
    """Weights of one model on the device plus the mk_weights struct.

    tiled=True also makes tiled copies (mk_pack_tiled) of the layer matrices
    and the LM head, with their own struct `struct_tiled` for plans built
    with tiled=True (the embedding and the gains are shared)."""

    def __init__(self, shape, weights: Dict, device="cuda", tiled: bool = False):
        self.shape = shape
        self.layers: List[Dict[str, object]] = []
        for lw in weights["layers"]:
            self.layers.append({k: to_device(v, device) for k, v in lw.items()})
        self.embed = to_device(weights["embed"], device) if "embed" in weights else None
        self.lm_head = to_device(weights["lm_head"], device) if "lm_head" in weights else None
        self.final_norm = to_device(weights["final_norm"], device) if "final_norm" in weights else None
        self.struct = mk.make_weights(self.layers, self.embed, self.final_norm, self.lm_head)
        self.struct_tiled = None
        if tiled:
            self.add_tiled()

    def add_tiled(self) -> None:
        """Tiled copies of the seven layer matrices and the LM head."""
        torch = _torch()

        def pack(t):
            out = torch.empty_like(t)
            mk.pack_tiled(t, out, t.shape[0], t.shape[1])
            return out

        self.layers_tiled = []
        for lw in self.layers:
            d = dict(lw)
            for k in TILED_MATRICES:
                d[k] = pack(lw[k])
            self.layers_tiled.append(d)
        self.lm_head_tiled = pack(self.lm_head) if self.lm_head is not None else None
        self.struct_tiled = mk.make_weights(self.layers_tiled, self.embed, self.final_norm, self.lm_head_tiled)


class DeviceKV:
    """KV cache on the device in the library's contiguous or paged layout.

    Contiguous: k, v [L, B, Hkv, cap, D]. Paged: k, v [L, n_blocks, Hkv, block, D]
    with block_table [B, max_blocks] (physical block of each logical block).
    """

    def __init__(self, shape, batch: int, cap: int, paged: bool = False, block: int = 16,
                 block_table: Optional[np.ndarray] = None, device="cuda"):
        torch = _torch()
        self.shape, self.B, self.cap, self.paged, self.block = shape, batch, cap, paged, block
        L, Hkv, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
        dt = torch.int16 if shape.kv_dtype == "bf16" else torch.float32
        if paged:
            assert block_table is not None
            self.table_np = np.ascontiguousarray(block_table, dtype=np.int32)
            self.n_blocks = int(self.table_np.max()) + 1
            self.k = torch.zeros((L, self.n_blocks, Hkv, block, D), dtype=dt, device=device)
            self.v = torch.zeros_like(self.k)
            self.table = torch.from_numpy(self.table_np).to(device)
            self.layer_stride = self.n_blocks * Hkv * block * D
            self.max_blocks = self.table_np.shape[1]
        else:
            self.k = torch.zeros((L, batch, Hkv, cap, D), dtype=dt, device=device)
            self.v = torch.zeros_like(self.k)
            self.table = None
            self.layer_stride = batch * Hkv * cap * D
            self.max_blocks = 0
        self.struct = mk.make_kv(self.k, self.v, self.layer_stride, self.table)

    def _view(self, t, b: int, n: int):
        """[L, Hkv, n, D] view/copy of the first n positions of sequence b."""
        torch = _torch()
        if not self.paged:
            return t[:, b, :, :n, :]
        nb = (n + self.block - 1) // self.block
        blocks = torch.from_numpy(self.table_np[b, :nb].astype(np.int64)).to(t.device)
        g = t.index_select(1, blocks)  # [L, nb, Hkv, block, D]
        g = g.permute(0, 2, 1, 3, 4).reshape(t.shape[0], t.shape[2], nb * self.block, t.shape[4])
        return g[:, :, :n, :]

    def load_sequence(self, b: int, k: np.ndarray, v: np.ndarray, n: int) -> None:
        """Write positions [0, n) of sequence b from host arrays [L, Hkv, >=n, D]."""
        torch = _torch()
        if n == 0:
            return
        for src, dst in ((k, self.k), (v, self.v)):
            h = to_device(np.ascontiguousarray(src[:, :, :n, :]), dst.device)
            if not self.paged:
                dst[:, b, :, :n, :].copy_(h)
            else:
                for j0 in range(0, n, self.block):
                    j1 = min(n, j0 + self.block)
                    blk = int(self.table_np[b, j0 // self.block])
                    dst[:, blk, :, : j1 - j0, :].copy_(h[:, :, j0:j1, :])

    def read_sequence(self, b: int, n: int):
        """Host copies (k, v) [L, Hkv, n, D] of sequence b."""
        return from_device(self._view(self.k, b, n).contiguous()), from_device(self._view(self.v, b, n).contiguous())


def build_plan(shape, batch: int, cap: int, paged: bool = False, block: int = 16, max_blocks: int = 0,
               **opts) -> mk.Plan:
    desc = mk.make_desc(shape, batch, cap, paged=paged, kv_block=block, max_blocks_per_seq=max_blocks, **opts)
    return mk.Plan(desc)


def step_bytes(shape, seq_lens: Sequence[int], batch: int) -> int:
    """Algorithmic HBM bytes of one decode step: every weight byte once, the
    KV of positions 0..L_b (L_b + 1 keys, the new one included) read, the new
    K/V row written, embedding rows read, logits written."""
    es = 2 if shape.kv_dtype == "bf16" else 4
    kvtok = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * es
    b = shape.step_weight_bytes()
    b += kvtok * sum(int(l) + 1 for l in seq_lens)  # reads
    b += kvtok * batch  # appends
    if shape.embed_head:
        wes = 4 if shape.wdtype == "f32" else 2
        b += batch * shape.hidden * wes + batch * shape.vocab * 4
    else:
        b += 2 * batch * shape.hidden * 4
    return b
