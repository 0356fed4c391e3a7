"""Host-side tests of the C ABI (no GPU): the library loads and exports every
symbol of include/mk.h, and the binding raises when it is missing; task
graphs for every workload verify; the host dry run of the persistent
protocol matches a sequential evaluation under random delays and thread
counts; fault injection times out instead of hanging; invalid descriptions
are rejected with a message."""
import ctypes
import os
import re
from dataclasses import replace

import numpy as np
import pytest

import synth
from persistent_task_graph_amd import mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mk.LIB_PATH):
        pytest.skip("libmk.so not built (run __graft_entry__.build())")
    return mk.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "mk.h")).read()
    declared = set(re.findall(r"^(?:int|void|const char\*|mk_plan\*)\s+(mk_[a-z_]+)\s*\(", hdr, re.M))
    assert set(mk.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_missing_library_raises(monkeypatch, tmp_path):
    # no CPU fallback: without the built library the binding refuses to run
    monkeypatch.setattr(mk, "LIB_PATH", str(tmp_path / "libmk.so"))
    monkeypatch.setattr(mk, "_lib", None)
    with pytest.raises(mk.MKError, match="not built"):
        mk.lib()


def _plan(shape, batch, cap, **kw):
    kw.setdefault("host_only", 1)
    paged = kw.pop("paged", False)
    return mk.Plan(mk.make_desc(shape, batch, cap, paged=paged, **kw))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_plans_verify(lib, name):
    wl = synth.WORKLOADS[name]
    p = _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged)
    p.verify()
    inf = p.info()
    assert inf.workers == 256 and inf.sched_waves == 0  # AOT attention: no scheduler CUs
    assert inf.weight_bytes_per_step == wl.shape.step_weight_bytes()
    L = wl.shape.n_layers
    assert inf.n_levels == 5 * L + (2 if wl.shape.embed_head else 0)
    # one GEMV task per worker per operator (rows >= workers)
    for op in (mk.OP_QKV, mk.OP_O, mk.OP_GATEUP, mk.OP_DOWN):
        assert inf.tasks_per_op[op] == L * 256
    assert inf.tasks_per_op[mk.OP_ATTN] > 0  # AOT attention slots by default
    j = _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged, jit=1)
    j.verify()
    ji = j.info()
    assert ji.workers == 252 and ji.sched_waves == 16
    assert ji.tasks_per_op[mk.OP_ATTN] == 0  # JIT: created on the device


def test_eight_b_step_bytes_match_definition(lib):
    # 36 x 385,892,864 + LM head 1,244,659,712 + final norm 8,192
    assert synth.Q8B.step_weight_bytes() == 36 * 385_892_864 + 1_244_659_712 + 8_192
    p = _plan(synth.Q8B, 1, 2048)
    assert p.info().kv_bytes_per_token == 147_456


@pytest.mark.parametrize("threads", [1, 3, 8, 64])
@pytest.mark.parametrize("jit", [1, 2])
def test_dry_run_matches_sequential(lib, threads, jit):
    shape = replace(synth.Q8B, n_layers=3)
    rng = np.random.default_rng(threads * 10 + jit)
    seq = rng.integers(0, 900, size=4).tolist()
    p = _plan(shape, 4, 1024, jit=jit, workers=16, kv_chunk=128)
    rc = p.dry_run(n_threads=threads, seed=threads, timeout_ms=20000, seq_lens=seq)
    assert rc == 0, mk.last_error()


def test_dry_run_full_model_default_workers(lib):
    p = _plan(synth.Q8B, 16, 4200)
    seq = synth.seq_lengths(synth.WORKLOADS["q8b_b16"]).tolist()
    assert p.dry_run(n_threads=8, seed=3, timeout_ms=60000, seq_lens=seq) == 0, mk.last_error()


def test_dry_run_dropped_producer_times_out(lib):
    shape = replace(synth.Q8B, n_layers=2)
    p = _plan(shape, 1, 256, workers=8, jit=1)  # task 20 is then a GEMV task
    rc = p.dry_run(n_threads=4, seed=1, drop_task=20, timeout_ms=500, seq_lens=[10])
    assert rc == mk.MK_ERR_STATE and "timeout" in mk.last_error()


def test_debug_extra_required_breaks_verification_count_only(lib):
    # the fault-injection knob adds to one event's required count; the
    # verifier accounts for it, the dry run then times out
    shape = replace(synth.Q8B, n_layers=2)
    p = _plan(shape, 1, 256, workers=8, debug_event=2, debug_extra_required=1)
    p.verify()
    assert p.dry_run(n_threads=4, seed=1, timeout_ms=500, seq_lens=[5]) == mk.MK_ERR_STATE


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 96, "head_dim"),
    ("n_kv_heads", 5, "multiple"),
    ("batch", 17, "batch"),
    ("hidden", 4100, "multiple of 8"),
    ("max_seq_len", 0, "max_seq_len"),
])
def test_bad_desc_rejected(lib, field, value, msg):
    d = mk.make_desc(synth.Q8B, 1, 1024, host_only=1)
    setattr(d, field, value)
    h = lib.mk_build_graph(ctypes.byref(d))
    assert not h
    assert msg in mk.last_error()


def test_step_on_host_only_plan_is_state_error(lib):
    p = _plan(synth.TINY, 1, 64)
    w = mk.make_weights([{}] * 2, 1, 1, 1)
    kv = mk.make_kv(1, 1, 0)
    rc = lib.mk_decode_step(p.handle, ctypes.byref(w), ctypes.byref(kv), 1, 1, 1, None)
    assert rc == mk.MK_ERR_STATE


def test_aot_attention_slots(lib):
    # one slot per split task a step can have: at most 240 while the chunk can
    # still grow, else every split at kv_chunk_max
    p = _plan(synth.TINY, 1, 48, jit=2, kv_chunk=16)
    inf = p.info()
    assert inf.max_splits == 3
    assert inf.tasks_per_op[mk.OP_ATTN] == 2 * 4 * 3
    p.verify()
    p = _plan(replace(synth.Q8B, n_layers=2), 16, 4200, jit=2, kv_chunk=128)
    inf = p.info()
    assert inf.max_splits == 33
    assert inf.tasks_per_op[mk.OP_ATTN] == 2 * 16 * 8 * 2  # 4200 keys need 2 splits of 4096
    p.verify()
    p = _plan(replace(synth.Q8B, n_layers=2), 4, 1024, jit=2, kv_chunk=128)
    assert p.info().tasks_per_op[mk.OP_ATTN] == 2 * 240
    p.verify()


def test_aot_slots_dry_run_capped_chunk(lib):
    # the chunk capped at kv_chunk_max: more than 240 split tasks, one slot each
    shape = replace(synth.Q8B, n_layers=2)
    p = _plan(shape, 16, 4200, jit=2, workers=24, kv_chunk=64, kv_chunk_max=64)
    seq = [4000] * 16  # 16 * 8 * 63 split tasks per layer
    assert p.dry_run(n_threads=6, seed=5, timeout_ms=60000, seq_lens=seq) == 0, mk.last_error()
