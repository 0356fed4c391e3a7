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
    # JIT expanded by the completing QKV arrival (batch >= 5): every CU is a worker
    if wl.batch >= 5:
        k = _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged, jit=3)
        k.verify()
        ki = k.info()
        assert ki.workers == 256 and ki.sched_waves == 0 and ki.jit == 3
        assert ki.tasks_per_op[mk.OP_ATTN] == 0
    else:
        with pytest.raises(mk.MKError, match="batch >= 5"):
            _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged, jit=3)


def test_eight_b_step_bytes_match_definition(lib):
    # 36 x 385,892,864 + LM head 1,244,659,712 + final norm 8,192
    assert synth.Q8B.step_weight_bytes() == 36 * 385_892_864 + 1_244_659_712 + 8_192
    p = _plan(synth.Q8B, 1, 2048)
    assert p.info().kv_bytes_per_token == 147_456


@pytest.mark.parametrize("threads", [1, 3, 8, 64])
@pytest.mark.parametrize("jit", [1, 2, 3])
def test_dry_run_matches_sequential(lib, threads, jit):
    shape = replace(synth.Q8B, n_layers=3)
    rng = np.random.default_rng(threads * 10 + jit)
    B = 8 if jit == 3 else 4
    seq = rng.integers(0, 900, size=B).tolist()
    p = _plan(shape, B, 1024, jit=jit, workers=16, kv_chunk=128)
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
    # arguments are checked first (null weight pointers: MK_ERR_ARG), then the
    # plan's state (host-only: MK_ERR_STATE)
    p = _plan(synth.TINY, 1, 64)
    w = mk.make_weights([{}] * 2, 1, 1, 1)
    kv = mk.make_kv(1, 1, 1 * 4 * 64 * 64)
    rc = lib.mk_decode_step(p.handle, ctypes.byref(w), ctypes.byref(kv), 1, 1, 1, None)
    assert rc == mk.MK_ERR_ARG
    assert _fake_step(p, synth.TINY, 1 * 4 * 64 * 64, False) == mk.MK_ERR_STATE


def test_aot_attention_slots(lib):
    # one slot per split task a step can have: at most 256 while the chunk can
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
    assert p.info().tasks_per_op[mk.OP_ATTN] == 2 * 256
    p.verify()


def test_aot_slots_dry_run_capped_chunk(lib):
    # the chunk capped at kv_chunk_max: more than 256 split tasks, one slot each
    shape = replace(synth.Q8B, n_layers=2)
    p = _plan(shape, 16, 4200, jit=2, workers=24, kv_chunk=64, kv_chunk_max=64)
    seq = [4000] * 16  # 16 * 8 * 63 split tasks per layer
    assert p.dry_run(n_threads=6, seed=5, timeout_ms=60000, seq_lens=seq) == 0, mk.last_error()


# ---------------------------------------------------------------- 32-bit K/V offsets
# Attention addresses K/V with 32-bit byte offsets inside buffer resources,
# and uses 2^31 as the out-of-range offset: a contiguous sequence span and a
# paged layer must both stay below 2 GiB. Larger layouts are refused.

def _fake_step(plan, shape, layer_stride, paged):
    """mk_decode_step on a host-only plan with fake (never dereferenced) device pointers."""
    fake = 0x1000
    lw = [{n: fake for n in mk.LAYER_FIELDS} for _ in range(shape.n_layers)]
    w = mk.make_weights(lw, fake, fake, fake)
    kv = mk.make_kv(fake, fake, layer_stride, fake if paged else None)
    return mk.lib().mk_decode_step(plan.handle, ctypes.byref(w), ctypes.byref(kv), fake, fake, fake, None)


def test_contiguous_span_of_2gib_rejected_at_build(lib):
    shape = synth.ModelShape(n_layers=1, hidden=1024, n_heads=8, n_kv_heads=8, head_dim=128, ffn=2048, vocab=100,
                             wdtype="f32", kv_dtype="f32")
    # fp32, head_dim 128: 4M positions span exactly 2 GiB
    with pytest.raises(mk.MKError, match="2 GiB"):
        _plan(shape, 1, 1 << 22)
    _plan(shape, 1, (1 << 22) - 1).verify()
    _plan(synth.Q8B, 1, 1 << 22).verify()  # bf16: 1 GiB


def test_paged_layer_of_2gib_rejected_at_step(lib):
    shape = replace(synth.Q8B, n_layers=2)
    blk = shape.n_kv_heads * 16 * shape.head_dim  # elements per physical block and layer
    p = _plan(shape, 16, 1 << 22, paged=True)
    max_blocks = ((1 << 31) - 1) // (2 * blk)  # largest pool under 2 GiB per layer
    assert _fake_step(p, shape, max_blocks * blk, True) == mk.MK_ERR_STATE  # arguments fine, plan host-only
    assert _fake_step(p, shape, (max_blocks + 1) * blk, True) == mk.MK_ERR_ARG
    assert "2 GiB" in mk.last_error()
    assert _fake_step(p, shape, blk + 1, True) == mk.MK_ERR_ARG  # not a whole number of blocks
    assert "multiple" in mk.last_error()


def test_contiguous_layer_stride_too_small_rejected(lib):
    shape = replace(synth.Q8B, n_layers=2)
    p = _plan(shape, 4, 1000)
    need = 4 * shape.n_kv_heads * 1000 * shape.head_dim
    assert _fake_step(p, shape, need, False) == mk.MK_ERR_STATE
    assert _fake_step(p, shape, need - 1, False) == mk.MK_ERR_ARG


# ---------------------------------------------------------------- static schedule
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_static_schedule_plans_verify_and_dry_run(lib, name):
    # the searched plan covers every row once, fixes every attention split of
    # the capacity, replays correctly on host threads, and is deterministic
    wl = synth.WORKLOADS[name]
    p = _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged, schedule=1)
    p.verify()
    inf = p.info()
    assert inf.schedule == 1 and inf.jit == 0 and inf.predicted_layer_us > 0
    assert inf.tasks_per_op[mk.OP_ATTN] == wl.shape.n_layers * wl.batch * wl.shape.n_kv_heads * inf.max_splits
    assert inf.max_splits == -(-wl.capacity() // inf.kv_chunk)
    lens = [int(v) for v in synth.seq_lengths(wl)]
    assert p.dry_run(n_threads=6, seed=11, seq_lens=lens) == 0
    q = _plan(wl.shape, wl.batch, wl.capacity(), paged=wl.paged, schedule=1).info()
    assert list(q.tasks_per_op) == list(inf.tasks_per_op) and q.kv_chunk == inf.kv_chunk


@pytest.mark.parametrize("jit", [1, 3])
def test_static_schedule_rejects_jit(lib, jit):
    with pytest.raises(mk.MKError, match="static schedule"):
        _plan(replace(synth.Q8B, n_layers=2), 8, 64, schedule=1, jit=jit)


# ---------------------------------------------------------------- prefill plans
@pytest.mark.parametrize("schedule", [0, 1])
def test_prefill_plan_has_append_level(lib, schedule):
    # one append task per (row, KV head) and layer, between QKV and attention;
    # attention waits for the layer's appends
    shape = replace(synth.Q8B, n_layers=3)
    p = _plan(shape, 16, 2048, prefill=1, schedule=schedule)
    p.verify()
    inf = p.info()
    assert inf.tasks_per_op[mk.OP_APPEND] == 3 * 16 * shape.n_kv_heads
    assert inf.n_levels == 6 * 3 + 2
    assert p.dry_run(n_threads=6, seed=2, seq_lens=list(range(100, 116))) == 0, mk.last_error()


@pytest.mark.parametrize("jit", [1, 3])
def test_prefill_plan_rejects_jit(lib, jit):
    with pytest.raises(mk.MKError, match="prefill"):
        _plan(replace(synth.Q8B, n_layers=2), 8, 64, prefill=1, jit=jit)


def test_prefill_entry_point_checks(lib):
    p = _plan(synth.TINY, 4, 64, prefill=1)
    fake = 0x1000
    lw = [{n: fake for n in mk.LAYER_FIELDS} for _ in range(synth.TINY.n_layers)]
    w = mk.make_weights(lw, fake, fake, fake)
    stride = synth.TINY.n_kv_heads * 64 * synth.TINY.head_dim  # one sequence suffices
    kv = mk.make_kv(fake, fake, stride)
    call = lambda pos0, T: lib.mk_prefill(p.handle, ctypes.byref(w), ctypes.byref(kv), fake, pos0, T, fake, None)
    assert call(0, 64) == mk.MK_ERR_STATE  # arguments fine, plan host-only
    assert call(1, 64) == mk.MK_ERR_ARG and "max_seq_len" in mk.last_error()
    assert call(0, 0) == mk.MK_ERR_ARG
    assert call(-1, 4) == mk.MK_ERR_ARG
    d = _plan(synth.TINY, 4, 64)  # a decode plan refuses prefill
    kv4 = mk.make_kv(fake, fake, 4 * stride)
    assert lib.mk_prefill(d.handle, ctypes.byref(w), ctypes.byref(kv4), fake, 0, 8, fake, None) == mk.MK_ERR_STATE


@pytest.mark.parametrize("B", [1, 4, 16])
def test_w4_plans_any_batch(lib, B):
    # 4-bit layer matrices: the VALU GEMV at batch <= 2, the matrix cores above
    p = _plan(synth.Q8B_W4, B, 2048)
    p.verify()
    assert p.info().weight_bytes_per_step == synth.Q8B_W4.step_weight_bytes()
    assert p.dry_run(n_threads=4, seed=B, seq_lens=[100 + 7 * b for b in range(B)]) == 0, mk.last_error()


@pytest.mark.parametrize("opts", [dict(), dict(schedule=1), dict(prefill=1), dict(jit=3), dict(mode=1)])
def test_tiled_plans_verify_on_8_row_units(lib, opts):
    # tiled weights: the verifier also checks that every matrix task starts
    # and ends on an 8-row unit of the tiled layout
    for B in (3, 16):
        if opts.get("jit") == 3 and B < 5:
            continue
        p = _plan(synth.Q8B, B, 4096, tiled=True, **opts)
        p.verify()
        assert p.dry_run(n_threads=4, seed=B, seq_lens=[100 + 37 * b for b in range(B)]) == 0, mk.last_error()


@pytest.mark.parametrize("case, msg", [
    (dict(batch=2), "batch >= 3"),
    (dict(batch=1), "batch >= 3"),
    (dict(shape=synth.TINY, batch=4), "bf16"),
    (dict(shape=synth.Q8B_W4, batch=16), "bf16"),
    (dict(shape=replace(synth.Q8B, vocab=151937), batch=16), "multiple of 8"),
    (dict(shape=replace(synth.Q8B, ffn=12320), batch=16), "multiples of 64"),
])
def test_tiled_plans_rejected(lib, case, msg):
    shape = case.get("shape", synth.Q8B)
    d = mk.make_desc(shape, case["batch"], 1024, host_only=1, tiled=True)
    h = lib.mk_build_graph(ctypes.byref(d))
    assert not h
    assert msg in mk.last_error()


@pytest.mark.parametrize("rows, cols", [(12, 64), (0, 64), (16, 32), (16, 96)])
def test_pack_tiled_rejects_bad_sizes(lib, rows, cols):
    # checked before anything is launched
    assert lib.mk_pack_tiled(ctypes.c_void_p(4096), ctypes.c_void_p(1 << 30), rows, cols, None) == mk.MK_ERR_ARG
    assert "mk_pack_tiled" in mk.last_error()


def test_pack_tiled_rejects_null_and_overlap(lib):
    assert lib.mk_pack_tiled(None, ctypes.c_void_p(4096), 8, 64, None) == mk.MK_ERR_ARG
    # [4096, 4096 + 1024) and [4608, ...) overlap
    assert lib.mk_pack_tiled(ctypes.c_void_p(4096), ctypes.c_void_p(4608), 8, 64, None) == mk.MK_ERR_ARG
    assert "overlap" in mk.last_error()


@pytest.mark.parametrize("ks", [0, 1, 2, 4])
@pytest.mark.parametrize("opts", [dict(), dict(tiled=True), dict(prefill=1), dict(jit=3)])
def test_down_ksplit_plans_verify_and_dry_run(lib, ks, opts):
    # K-split down projection: every part covers the same row groups, the
    # event counts one arrival per group (its merging part), and the host dry
    # run's merge equals the sequential evaluation
    B = 16
    p = _plan(synth.Q8B, B, 4096, down_ksplit=ks, o_ksplit=ks, **opts)
    p.verify()
    assert p.dry_run(n_threads=8, seed=3 + ks, seq_lens=[50 + 211 * b for b in range(B)]) == 0, mk.last_error()
    for op in (mk.OP_DOWN, mk.OP_O):
        assert p.info().tasks_per_op[op] == 256 * synth.Q8B.n_layers  # per layer: groups x parts = workers


@pytest.mark.parametrize("case, msg", [
    (dict(batch=2, down_ksplit=4), "matrix-core path"),
    (dict(batch=16, down_ksplit=3), "down_ksplit must be"),
    (dict(batch=16, down_ksplit=4, schedule=1), "static schedule"),
    (dict(batch=16, down_ksplit=4, shape=replace(synth.Q8B, ffn=12352)), "multiple of 64 * parts"),
    (dict(batch=2, o_ksplit=2), "matrix-core path"),
    (dict(batch=16, o_ksplit=4, schedule=1), "static schedule"),
])
def test_down_ksplit_rejected(lib, case, msg):
    shape = case.pop("shape", synth.Q8B)
    B = case.pop("batch")
    d = mk.make_desc(shape, B, 1024, host_only=1, **case)
    h = lib.mk_build_graph(ctypes.byref(d))
    assert not h
    assert msg in mk.last_error()


def test_down_ksplit_default(lib):
    # default: 4 parts on the matrix-core path of the event runtime, else none
    # (checked through the dry run's task counts: the plan reports tasks only)
    for B, sched in ((16, 0), (4, 0), (16, 1), (1, 0)):
        p = _plan(synth.Q8B, B, 2048, schedule=sched)
        p.verify()
        assert p.dry_run(n_threads=4, seed=B, seq_lens=[100] * B) == 0, mk.last_error()
