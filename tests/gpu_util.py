"""Shared helpers for the GPU tests: set up a workload on the device and on
the oracle from the same seeded inputs, run teacher-forced decode steps and
compare."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth
from persistent_task_graph_amd import harness, mk


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class Setup:
    shape: object
    B: int
    cap: int
    weights: Dict
    lens: np.ndarray
    caches: List[Dict[str, np.ndarray]]
    dm: object = None
    paged: bool = False
    block: int = 16
    table: Optional[np.ndarray] = None


def make_setup(shape, B, lens, cap, seed_w=synth.SEED_WEIGHTS, paged=False, block=16, table=None, std=0.02,
               weights=None, device=True):
    weights = weights if weights is not None else synth.model_weights(shape, seed=seed_w, std=std)
    lens = np.asarray(lens, dtype=np.int64)
    caches = synth.kv_contents(shape, lens, cap)
    s = Setup(shape, B, cap, weights, lens, caches, paged=paged, block=block, table=table)
    if device:
        s.dm = harness.DeviceModel(shape, weights)
    return s


def device_kv(s: Setup):
    kv = harness.DeviceKV(s.shape, s.B, s.cap, paged=s.paged, block=s.block, block_table=s.table)
    for b in range(s.B):
        kv.load_sequence(b, s.caches[b]["k"], s.caches[b]["v"], int(s.lens[b]))
    return kv


def plan_for(s: Setup, **opts):
    mb = s.table.shape[1] if s.table is not None else 0
    return harness.build_plan(s.shape, s.B, s.cap, paged=s.paged, block=s.block, max_blocks=mb, **opts)


def run_gpu(s: Setup, plan, kv, tokens0: np.ndarray, steps: int, x_inputs=None):
    """Greedy decode on the GPU; returns per-step (tokens fed, logits or hidden out)."""
    import torch

    B, V = s.B, s.shape.vocab
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    out = []
    if s.shape.embed_head:
        tok = torch.from_numpy(tokens0.astype(np.int32)).cuda()
        logits = torch.empty((B, V), dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        for t in range(steps):
            plan.step(s.dm.struct, kv.struct, tok, d_len, logits)
            plan.argmax(logits, nxt)
            out.append((tok.cpu().numpy().copy(), logits.cpu().numpy().copy(), nxt.cpu().numpy().copy()))
            tok = nxt.clone()
            d_len += 1
    else:
        xo = torch.empty((B, s.shape.hidden), dtype=torch.float32, device="cuda")
        for t in range(steps):
            xi = torch.from_numpy(x_inputs[t]).cuda()
            plan.step_hidden(s.dm.struct, kv.struct, xi, d_len, xo)
            out.append((None, xo.cpu().numpy().copy(), None))
            d_len += 1
    torch.cuda.synchronize()
    err = plan.device_error()
    return out, err


def run_oracle(s: Setup, gpu_out, rows=None, x_inputs=None):
    """Oracle on the GPU's tokens (teacher forcing). rows: batch rows to compute."""
    orc = oracle.Oracle(s.shape, s.weights)
    rows = list(range(s.B)) if rows is None else rows
    caches = {b: {k: s.caches[b][k].copy() for k in ("k", "v")} for b in rows}
    res = []
    for t, (tok, _, _) in enumerate(gpu_out):
        step = {}
        for b in rows:
            pos = int(s.lens[b]) + t
            if s.shape.embed_head:
                step[b] = orc.model_forward(caches[b], int(tok[b]), pos)
            else:
                step[b] = orc.hidden_forward(caches[b], pos, x_inputs[t][b])
        res.append(step)
    return res, caches


def compare(gpu_out, orc_out, rows=None, tol_rel=2e-2):
    """max|d| / std per step over the compared rows, and top-1 agreement."""
    worst = 0.0
    agree = total = 0
    for t, (tok, got, nxt) in enumerate(gpu_out):
        rws = sorted(orc_out[t]) if rows is None else rows
        ref = np.stack([orc_out[t][b] for b in rws])
        g = got[rws]
        d = float(np.abs(g - ref).max())
        sd = float(ref.std())
        worst = max(worst, d / sd)
        if nxt is not None:
            agree += int(np.sum(np.argmax(ref, axis=1) == nxt[rws]))
            total += len(rws)
    return worst, (agree / total if total else 1.0)


def rows_vs_oracle_from_prefix(orc, cap, k_all, v_all, prompt, pos0, positions):
    """For each position p: the oracle, given the GPU's K/V of positions < p,
    computes position p; returns the worst (|gpu - oracle| - 2^-7 max(|gpu|,
    |oracle|)) / rms(oracle row) over p's keys and values."""
    worst = 0.0
    L, Hkv, _, D = k_all.shape
    for p in positions:
        cache = {"k": np.zeros((L, Hkv, cap, D), np.uint16), "v": np.zeros((L, Hkv, cap, D), np.uint16)}
        cache["k"][:, :, :p] = k_all[:, :, :p]
        cache["v"][:, :, :p] = v_all[:, :, :p]
        orc.model_forward(cache, int(prompt[p - pos0]), p)
        for got, want in ((k_all[:, :, p], cache["k"][:, :, p]), (v_all[:, :, p], cache["v"][:, :, p])):
            g = synth.bf16_to_f32(np.ascontiguousarray(got)).astype(np.float64)
            r = synth.bf16_to_f32(np.ascontiguousarray(want)).astype(np.float64)
            rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
            excess = np.abs(g - r) - 2 ** -7 * np.maximum(np.abs(g), np.abs(r))
            worst = max(worst, float((excess / rms).max()))
    return worst
