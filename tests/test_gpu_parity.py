"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs, and bit-for-bit identity across execution modes
(persistent task graph vs kernel-per-operator), worker counts, JIT vs AOT
attention and KV layouts.

Tolerance: max|gpu - oracle| <= 2e-2 * std(oracle logits) per step for bf16
weights (fp32 weights: 1e-3 * std); teacher-forced greedy top-1 agreement
>= 99%.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (compare, device_kv, log, make_setup, plan_for, rows_vs_oracle_from_prefix, run_gpu,
                            run_oracle)

pytestmark = pytest.mark.gpu

MID = synth.ModelShape(n_layers=2, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288, vocab=8000)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny"]
    return make_setup(wl.shape, wl.batch, synth.seq_lengths(wl), wl.capacity())


def _tokens(shape, B, stream=0):
    return synth.uniform_int(synth.SEED_TOKENS, stream, 0, shape.vocab - 1, B).astype(np.int32)


def test_tiny_persistent_matches_oracle(tiny):
    s = tiny
    log("tiny: persistent, 16 greedy steps")
    plan = plan_for(s)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(s.shape, s.B), 16)
    assert err == 0
    orc, _ = run_oracle(s, out)
    worst, agree = compare(out, orc)
    log("tiny max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 1e-3
    assert agree >= 0.99


def _logits_seq(s, steps, tokens=None, **opts):
    plan = plan_for(s, **opts)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, tokens if tokens is not None else _tokens(s.shape, s.B), steps)
    assert err == 0, "device error %d (%s)" % (err, opts)
    plan.close()
    return out, kv


def _bitwise(a, b):
    for (ta, la, na), (tb, lb, nb) in zip(a, b):
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))


def test_tiny_kernel_per_op_bitwise(tiny):
    log("tiny: persistent vs kernel-per-op")
    a, _ = _logits_seq(tiny, 8)
    b, _ = _logits_seq(tiny, 8, mode=1)
    _bitwise(a, b)


@pytest.mark.parametrize("workers", [1, 7, 64])
def test_tiny_worker_count_invariance(tiny, workers):
    log("tiny: workers=%d" % workers)
    a, _ = _logits_seq(tiny, 4)
    b, _ = _logits_seq(tiny, 4, workers=workers)
    _bitwise(a, b)


def test_tiny_jit_vs_aot_and_repeat(tiny):
    log("tiny: AOT (default) vs JIT attention, repeat run")
    a, _ = _logits_seq(tiny, 6, kv_chunk=16)
    b, _ = _logits_seq(tiny, 6, kv_chunk=16, jit=1)
    c, _ = _logits_seq(tiny, 6, kv_chunk=16)
    _bitwise(a, b)
    _bitwise(a, c)


@pytest.fixture(scope="module")
def mid_weights():
    return synth.model_weights(MID)


@pytest.mark.parametrize("B,lens,chunk", [
    (1, [0], 64),            # first token: a single key
    (1, [300], 64),          # several splits with a ragged tail
    (3, [5, 129, 700], 128),  # mixed lengths, B < 4 path
    (8, [1, 63, 64, 65, 200, 511, 512, 777], 64),
    (16, list(range(3, 16 * 37, 37)), 256),
])
def test_mid_bf16_matches_oracle(mid_weights, B, lens, chunk):
    log("mid bf16: B=%d lens=%s chunk=%d" % (B, lens, chunk))
    cap = max(lens) + 8
    s = make_setup(MID, B, lens, cap, weights=mid_weights)
    plan = plan_for(s, kv_chunk=chunk)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID, B, 7), 2)
    assert err == 0
    rows = list(range(B)) if B <= 8 else [0, 5, 15]
    orc, caches = run_oracle(s, out, rows=rows)
    worst, agree = compare(out, orc, rows=rows)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2
    assert agree >= 0.99
    _check_appended(s, kv, caches, rows, 2)
    plan.close()


def _check_appended(s, kv, caches, rows, steps):
    """Cached positions are untouched (bit-identical); the appended rows agree
    with the oracle's to one bf16 ulp plus the fp32-vs-fp64 error of the
    projection, which is relative to the head vector's scale (RoPE can cancel
    an element down to near zero)."""
    for b in rows:
        L0 = int(s.lens[b])
        n = L0 + steps
        k, v = kv.read_sequence(b, n)
        for got, ref in ((k, caches[b]["k"][:, :, :n]), (v, caches[b]["v"][:, :, :n])):
            assert np.array_equal(got[:, :, :L0], ref[:, :, :L0])
            g = synth.bf16_to_f32(np.ascontiguousarray(got[:, :, L0:])).astype(np.float64)
            r = synth.bf16_to_f32(np.ascontiguousarray(ref[:, :, L0:])).astype(np.float64)
            rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
            assert np.all(np.abs(g - r) <= 2 ** -7 * np.maximum(np.abs(g), np.abs(r)) + 1e-4 * rms)


# Seeded non-unit gains, different for every gain vector (attention, MLP,
# final, per-head q and k): a kernel that read the wrong gain vector, no
# gain, or applied QK-norm after RoPE fails these (with unit gains it would
# not: RoPE keeps a head's RMS).
@pytest.fixture(scope="module")
def mid_weights_g(mid_weights):
    return synth.with_gains(MID, mid_weights, "random")


def test_tiny_random_gains_matches_oracle():
    wl = synth.WORKLOADS["tiny"]
    log("tiny: random gains, 8 greedy steps")
    w = synth.model_weights(wl.shape, gains="random")
    s = make_setup(wl.shape, wl.batch, synth.seq_lengths(wl), wl.capacity(), weights=w)
    plan = plan_for(s)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(s.shape, s.B), 8)
    assert err == 0
    orc, _ = run_oracle(s, out)
    worst, agree = compare(out, orc)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 1e-3 and agree >= 0.99
    plan.close()


@pytest.mark.parametrize("B,lens,paged", [
    (1, [300], False),
    (3, [5, 129, 700], False),
    (16, list(range(3, 16 * 37, 37)), False),
    (4, [17, 250, 64, 129], True),
])
def test_mid_random_gains_match_oracle(mid_weights_g, B, lens, paged):
    log("mid bf16, random gains: B=%d lens=%s paged=%s" % (B, lens, paged))
    cap = max(lens) + 8
    table = synth.block_table([cap] * B, 16) if paged else None
    s = make_setup(MID, B, lens, cap, weights=mid_weights_g, paged=paged, table=table)
    plan = plan_for(s, kv_chunk=64)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID, B, 9), 2)
    assert err == 0
    rows = list(range(B)) if B <= 8 else [0, 7, 15]
    orc, caches = run_oracle(s, out, rows=rows)
    worst, agree = compare(out, orc, rows=rows)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2
    assert agree >= 0.99
    _check_appended(s, kv, caches, rows, 2)
    plan.close()


def test_mid_modes_bitwise(mid_weights):
    log("mid bf16: persistent vs kernel-per-op vs JIT vs workers=37, B=2")
    s = make_setup(MID, 2, [100, 333], 400, weights=mid_weights)
    a, _ = _logits_seq(s, 3, kv_chunk=64)
    b, _ = _logits_seq(s, 3, kv_chunk=64, mode=1)
    c, _ = _logits_seq(s, 3, kv_chunk=64, jit=1)
    d, _ = _logits_seq(s, 3, kv_chunk=64, workers=37)
    for o in (b, c, d):
        _bitwise(a, o)


@pytest.mark.parametrize("B,paged", [(8, False), (16, False), (8, True)])
def test_mid_modes_bitwise_large_batch(mid_weights, B, paged):
    # the batch-8 and batch-16 kernel instances spread event arrivals over
    # eight count planes; the persistent step (AOT slots, JIT through the
    # scheduler waves, and JIT expanded by the completing QKV arrival) must
    # still give the kernel-per-op bits exactly
    lens = [int(v) for v in np.linspace(0, 900, B)]
    log("mid bf16: persistent vs kernel-per-op vs JIT, B=%d paged=%s lens=%s" % (B, paged, lens))
    cap = max(lens) + 8
    table = synth.block_table([cap] * B, 16) if paged else None
    s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=paged, table=table)
    t0 = _tokens(MID, B, 3)
    a, _ = _logits_seq(s, 3, tokens=t0)
    b, _ = _logits_seq(s, 3, tokens=t0, mode=1)
    c, _ = _logits_seq(s, 3, tokens=t0, jit=1)
    d, _ = _logits_seq(s, 3, tokens=t0, jit=3)
    for o in (b, c, d):
        _bitwise(a, o)
        for (ta, la, na), (to, lo, no) in zip(a, o):
            assert np.array_equal(na, no)


def test_mid_adaptive_chunk_matches_oracle_and_modes(mid_weights):
    # the step's chunk is the smallest multiple of 16 giving at most 256 split
    # tasks: these 4 sequences (8 KV heads) need 2864 splits at a base chunk
    # of 16, 272 at 176 and 256 at 192, so the chunk becomes 192 whatever the
    # worker count
    log("mid bf16: per-step chunk growth (chunk 16 -> 192), B=4")
    s = make_setup(MID, 4, [1000, 1500, 1999, 1200], 2010, weights=mid_weights)
    opts = dict(kv_chunk=16, workers=64)
    plan = plan_for(s, **opts)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID, 4, 11), 2)
    assert err == 0
    plan.close()
    orc, _ = run_oracle(s, out)
    worst, agree = compare(out, orc)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2 and agree >= 0.99
    b, _ = _logits_seq(s, 2, tokens=_tokens(MID, 4, 11), mode=1, **opts)
    c, _ = _logits_seq(s, 2, tokens=_tokens(MID, 4, 11), jit=1, **opts)
    e, _ = _logits_seq(s, 2, tokens=_tokens(MID, 4, 11), kv_chunk=16)  # default worker count: same chunk
    d, _ = _logits_seq(s, 2, tokens=_tokens(MID, 4, 11), kv_chunk=16, kv_chunk_max=16, workers=64)
    _bitwise(out, b)
    _bitwise(out, c)
    _bitwise(out, e)
    # a fixed chunk splits the keys differently: same values within tolerance, other bits
    worst_d = max(float(np.abs(x[1] - y[1]).max()) / float(y[1].std()) for x, y in zip(out, d))
    assert worst_d <= 2e-2


@pytest.mark.parametrize("B", [1, 2])
def test_mid_b1_variants_bitwise(mid_weights, B):
    log("mid bf16 B=%d: register GEMV vs LDS preload vs LDS-ring streaming vs kernel-per-op vs no prefetch" % B)
    s = make_setup(MID, B, [517, 300][:B], 540, weights=mid_weights)
    a, _ = _logits_seq(s, 3)
    variants = [dict(lds_preload=1), dict(mode=1), dict(prefetch_kb=-1), dict(lds_preload=1, prefetch_kb=-1)]
    if B == 1:
        variants.append(dict(lds_stream=1))
    for v in variants:
        o, _ = _logits_seq(s, 3, **v)
        _bitwise(a, o)


def test_mid_paged_equals_contiguous(mid_weights):
    log("mid bf16: paged (identity and permuted tables) vs contiguous, B=4")
    B, lens, cap = 4, [17, 250, 64, 129], 300
    cont = make_setup(MID, B, lens, cap, weights=mid_weights)
    a, _ = _logits_seq(cont, 2, kv_chunk=64)
    nblk = (cap + 15) // 16
    ident = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
    perm = synth.block_table([cap] * B, 16)
    for table in (ident, perm):
        pg = make_setup(MID, B, lens, cap, weights=mid_weights, paged=True, table=table)
        b, kv = _logits_seq(pg, 2, kv_chunk=64)
        _bitwise(a, b)


def _greedy_seq(s, steps, tokens0, **opts):
    """Decode with the fused greedy entry point; per step (tokens fed, logits, next tokens) and final lengths."""
    import torch

    plan = plan_for(s, **opts)
    kv = device_kv(s)
    tok = torch.from_numpy(tokens0.astype(np.int32)).cuda()
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    logits = torch.empty((s.B, s.shape.vocab), dtype=torch.float32, device="cuda")
    out = []
    for _ in range(steps):
        fed = tok.cpu().numpy().copy()
        plan.step_greedy(s.dm.struct, kv.struct, tok, d_len, logits)
        out.append((fed, logits.cpu().numpy().copy(), tok.cpu().numpy().copy()))
    torch.cuda.synchronize()
    assert plan.device_error() == 0
    plan.close()
    return out, d_len.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "mid3", "mid3_per_op", "mid16_jit", "mid16_jit3"])
def test_greedy_step_equals_step_argmax_increment(tiny, mid_weights, case):
    # the fused step gives the logits, tokens and lengths of step + argmax + increment
    if case == "tiny":
        s, opts, steps = tiny, {}, 6
    else:
        B = 16 if case.startswith("mid16") else 3
        lens = [0, 300, 77] if B == 3 else [int(x) for x in np.linspace(1, 500, B)]
        s = make_setup(MID, B, lens, 520, weights=mid_weights)
        opts = {"mid3_per_op": {"mode": 1}, "mid16_jit": {"jit": 1}, "mid16_jit3": {"jit": 3}}.get(case, {})
        steps = 3
    log("greedy step vs step + argmax + increment: %s" % case)
    t0 = _tokens(s.shape, s.B, 5)
    a, _ = _logits_seq(s, steps, tokens=t0, **opts)
    g, lens = _greedy_seq(s, steps, t0, **opts)
    for (ta, la, na), (tg, lg, ng) in zip(a, g):
        assert np.array_equal(ta, tg)
        assert np.array_equal(la.view(np.uint32), lg.view(np.uint32))
        assert np.array_equal(na, ng)
    assert np.array_equal(lens, s.lens + steps)


def test_device_errors_token_and_overflow(tiny):
    import torch

    s = tiny
    plan = plan_for(s)
    kv = device_kv(s)
    logits = torch.empty((s.B, s.shape.vocab), dtype=torch.float32, device="cuda")
    bad_tok = torch.full((s.B,), s.shape.vocab + 5, dtype=torch.int32, device="cuda")
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    plan.step(s.dm.struct, kv.struct, bad_tok, d_len, logits)
    assert plan.device_error() & 1  # MK_ERR_TOKEN
    full = torch.full((s.B,), s.cap, dtype=torch.int32, device="cuda")  # seq_len + 1 > capacity
    tok = torch.zeros((s.B,), dtype=torch.int32, device="cuda")
    plan.step(s.dm.struct, kv.struct, tok, full, logits)
    assert plan.device_error() & 2  # MK_ERR_KV_OVERFLOW
    # the error word was cleared: a good step reports nothing
    plan.step(s.dm.struct, kv.struct, tok, d_len, logits)
    assert plan.device_error() == 0


def test_watchdog_times_out_instead_of_hanging(tiny):
    # one event can never complete (its required count is one too high):
    # waiters give up after the watchdog and the step reports MK_ERR_TIMEOUT
    import torch

    s = tiny
    plan = plan_for(s, debug_event=2, debug_extra_required=1, watchdog_ms=50)
    kv = device_kv(s)
    logits = torch.empty((s.B, s.shape.vocab), dtype=torch.float32, device="cuda")
    tok = torch.zeros((s.B,), dtype=torch.int32, device="cuda")
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    plan.step(s.dm.struct, kv.struct, tok, d_len, logits)
    assert plan.device_error() & 4


def test_block_table_entry_outside_pool_is_reported(mid_weights):
    # a paged block-table entry past the pool or negative: the kernel's range
    # checks read zeros for those positions, store nothing for the new row and
    # raise MK_ERR_BLOCK_TABLE; with the table restored the next step is clean
    import torch

    from persistent_task_graph_amd import mk

    B, lens, cap = 2, [40, 70], 100
    table = synth.block_table([cap] * B, 16)
    s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=True, table=table)
    plan = plan_for(s)
    kv = device_kv(s)
    pool = kv.n_blocks
    good = kv.table.clone()
    kv.table[0, 40 // 16] = pool + 100  # the block holding sequence 0's new row
    kv.table[1, 1] = -7                 # a cached block of sequence 1
    log("paged block table with entries outside the pool (pool %d)" % pool)
    logits = torch.empty((B, MID.vocab), dtype=torch.float32, device="cuda")
    tok = torch.from_numpy(_tokens(MID, B, 1)).cuda()
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    plan.step(s.dm.struct, kv.struct, tok, d_len, logits)
    err = plan.device_error()
    assert err & mk.MK_ERR_BLOCK_TABLE and not err & ~mk.MK_ERR_BLOCK_TABLE
    assert torch.isfinite(logits).all()
    kv.table.copy_(good)
    plan.step(s.dm.struct, kv.struct, tok, d_len, logits)
    assert plan.device_error() == 0
    plan.close()


@pytest.mark.parametrize("case", ["tiny", "mid3", "mid16", "mid4_paged", "mid3_per_op"])
def test_multi_step_launch_equals_repeated_greedy_steps(tiny, mid_weights, case):
    # n greedy steps in one launch give, bit for bit, the tokens of each step,
    # the final lengths and the last step's logits of n separate greedy steps
    import torch

    opts = {}
    if case == "tiny":
        s, n = tiny, 6
    else:
        B = int("".join(ch for ch in case[3:] if ch.isdigit()))
        paged = case.endswith("paged")
        lens = [int(v) for v in np.linspace(3, 700, B)]
        cap = max(lens) + 16
        table = synth.block_table([cap] * B, 16) if paged else None
        s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=paged, table=table)
        n = 4 if B < 16 else 3
        if case.endswith("per_op"):
            opts = {"mode": 1}
    log("multi-step launch vs %d greedy steps: %s" % (n, case))
    t0 = _tokens(s.shape, s.B, 6)
    ref, ref_lens = _greedy_seq(s, n, t0, **opts)
    plan = plan_for(s, **opts)
    kv = device_kv(s)
    tok = torch.from_numpy(t0.astype(np.int32)).cuda()
    d_len = torch.from_numpy(s.lens.astype(np.int32)).cuda()
    logits = torch.empty((s.B, s.shape.vocab), dtype=torch.float32, device="cuda")
    out = torch.full((n, s.B), -1, dtype=torch.int32, device="cuda")
    plan.steps_greedy(s.dm.struct, kv.struct, tok, d_len, logits, n, out)
    torch.cuda.synchronize()
    assert plan.device_error() == 0
    got = out.cpu().numpy()
    for i, (fed, lg, nxt) in enumerate(ref):
        assert np.array_equal(got[i], nxt), (i, got[i], nxt)
    assert np.array_equal(tok.cpu().numpy(), ref[-1][2])
    assert np.array_equal(d_len.cpu().numpy(), ref_lens)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), ref[-1][1].view(np.uint32))
    plan.close()


@pytest.mark.parametrize("B,paged", [(1, False), (4, False), (16, False), (4, True)])
def test_static_schedule_equals_event_runtime(mid_weights, B, paged):
    # the static (searched) schedule runs the event runtime's task bodies: at
    # the same attention split length, and with whole-K down-projection tasks
    # as the static schedule has them, the logits are the same bits
    from persistent_task_graph_amd import harness

    lens = [int(v) for v in np.linspace(5, 900, B)]
    cap = max(lens) + 8
    table = synth.block_table([cap] * B, 16) if paged else None
    s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=paged, table=table)
    info = plan_for(s, schedule=1).info()
    C = int(info.kv_chunk)
    log("static schedule vs event runtime: B=%d paged=%s, split length %d, GEMV tasks %s"
        % (B, paged, C, list(info.tasks_per_op)))
    t0 = _tokens(MID, B, 8)
    a, _ = _logits_seq(s, 3, tokens=t0, schedule=1)
    b, _ = _logits_seq(s, 3, tokens=t0, kv_chunk=C, kv_chunk_max=C, down_ksplit=1)
    _bitwise(a, b)
    if B == 16:
        rows = [0, 15]
        orc, _ = run_oracle(s, a, rows=rows)
        worst, agree = compare(a, orc, rows=rows)
        log("  static schedule vs oracle: max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
        assert worst <= 2e-2 and agree >= 0.99


# ---------------------------------------------------------------- 4-bit weights (W4A16, batch <= 2)
MID_W4 = replace(MID, wdtype="w4")


@pytest.fixture(scope="module")
def mid_w4_weights():
    return synth.model_weights(MID_W4)


@pytest.mark.parametrize("B,lens,gains", [(1, [300], "unit"), (2, [5, 700], "unit"), (1, [77], "random")])
def test_mid_w4_matches_oracle(mid_w4_weights, B, lens, gains):
    log("mid W4: B=%d lens=%s gains=%s" % (B, lens, gains))
    w = mid_w4_weights if gains == "unit" else synth.with_gains(MID_W4, mid_w4_weights, "random")
    cap = max(lens) + 8
    s = make_setup(MID_W4, B, lens, cap, weights=w)
    plan = plan_for(s)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID_W4, B, 12), 2)
    assert err == 0
    orc, caches = run_oracle(s, out)
    worst, agree = compare(out, orc)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2 and agree >= 0.99
    _check_appended(s, kv, caches, list(range(B)), 2)
    plan.close()


@pytest.mark.parametrize("B,gains", [(4, "unit"), (16, "unit"), (8, "random")])
def test_mid_w4_matrix_cores_match_oracle(mid_w4_weights, B, gains):
    # batch >= 3: the matrix-core GEMV with the codes dequantized in registers
    lens = [int(v) for v in np.linspace(3, 700, B)]
    log("mid W4 (matrix cores): B=%d lens=%s gains=%s" % (B, lens, gains))
    w = mid_w4_weights if gains == "unit" else synth.with_gains(MID_W4, mid_w4_weights, "random")
    s = make_setup(MID_W4, B, lens, max(lens) + 8, weights=w)
    plan = plan_for(s)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID_W4, B, 14), 2)
    assert err == 0
    rows = list(range(B)) if B <= 8 else [0, 7, 15]
    orc, caches = run_oracle(s, out, rows=rows)
    worst, agree = compare(out, orc, rows=rows)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2 and agree >= 0.99
    _check_appended(s, kv, caches, rows, 2)
    plan.close()


def test_mid_w4_matrix_cores_modes_bitwise(mid_w4_weights):
    # persistent = kernel-per-op = static schedule = JIT at batch 16 with W4
    log("mid W4 B=16: persistent vs kernel-per-op vs static schedule vs JIT")
    lens = [int(v) for v in np.linspace(1, 500, 16)]
    s = make_setup(MID_W4, 16, lens, 520, weights=mid_w4_weights)
    t0 = _tokens(MID_W4, 16, 15)
    a, _ = _logits_seq(s, 3, tokens=t0, kv_chunk=128, kv_chunk_max=128)
    for o in (dict(mode=1), dict(schedule=1), dict(jit=3), dict(jit=1)):
        b, _ = _logits_seq(s, 3, tokens=t0, kv_chunk=128, kv_chunk_max=128, **o)
        _bitwise(a, b)


def test_mid_w4_modes_bitwise(mid_w4_weights):
    # persistent = kernel-per-op = no prefetch = static schedule; several steps per launch
    log("mid W4 B=2: persistent vs kernel-per-op vs no prefetch vs static schedule")
    s = make_setup(MID_W4, 2, [100, 333], 400, weights=mid_w4_weights)
    t0 = _tokens(MID_W4, 2, 13)
    a, _ = _logits_seq(s, 3, tokens=t0, kv_chunk=128, kv_chunk_max=128)
    for o in (dict(mode=1), dict(prefetch_kb=-1), dict(schedule=1)):
        b, _ = _logits_seq(s, 3, tokens=t0, kv_chunk=128, kv_chunk_max=128, **o)
        _bitwise(a, b)


# ---------------------------------------------------------------- prefill (prompt chunks through the runtime)
# A prefill chunk of more than two positions runs its GEMVs on the matrix
# cores with each fp32 activation split into two bf16 halves, x = hi + lo +
# e with |e| <= 2^-17 |x|: a dot product over K = 4096 then errs by at most
# 2^-17 sum|w x|, about 2^-17 (2/pi) sqrt(K) times its rms for random signs.
HILO_TOL = 2.0 ** -17 * (2 / np.pi) * np.sqrt(4096)  # 3.1e-4
def _prefill_case(mid_weights, B, pos0, T, paged=False, tiled=False, **opts):
    """Prefill T prompt tokens after pos0 cached positions with a batch-B
    prefill plan; returns (the setup, the device KV, the last logits, the
    prompt). tiled: the weights in the tiled layout."""
    import torch
    from persistent_task_graph_amd import harness

    cap = pos0 + T + 8
    table = synth.block_table([cap], 16) if paged else None
    s = make_setup(MID, 1, [pos0], cap, weights=mid_weights, paged=paged, table=table)
    kv = device_kv(s)
    mb = table.shape[1] if paged else 0
    plan = harness.build_plan(MID, B, cap, paged=paged, max_blocks=mb, prefill=1, tiled=tiled, **opts)
    prompt = synth.uniform_int(synth.SEED_TOKENS, 40 + pos0, 0, MID.vocab - 1, T).astype(np.int32)
    d_tok = torch.from_numpy(prompt).cuda()
    logits = torch.empty(MID.vocab, dtype=torch.float32, device="cuda")
    if tiled:
        s.dm.add_tiled()
    plan.prefill(s.dm.struct_tiled if tiled else s.dm.struct, kv.struct, d_tok, pos0, T, logits)
    torch.cuda.synchronize()
    assert plan.device_error() == 0
    plan.close()
    return s, kv, logits.cpu().numpy(), prompt


@pytest.mark.parametrize("B,pos0,T,paged,opts", [
    (16, 0, 37, False, {}),                 # chunks of 16, 16 and a ragged 5
    (16, 100, 20, False, {}),               # after a cached prefix
    (16, 50, 19, True, {}),                 # paged: block-table row 0
    (4, 7, 10, False, {"mode": 1}),         # kernel-per-op, chunks of 4
    (16, 3, 21, False, {"schedule": 1}),    # static schedule
])
def test_prefill_matches_token_by_token_oracle(mid_weights, B, pos0, T, paged, opts):
    # the prompt's keys and values and the logits after its last token agree
    # with T single-token oracle steps (teacher forcing on the prompt)
    log("prefill: chunk %d, pos0 %d, T %d, paged %s, %s" % (B, pos0, T, paged, opts))
    s, kv, got, prompt = _prefill_case(mid_weights, B, pos0, T, paged, **opts)
    orc = oracle.Oracle(MID, s.weights)
    cache = {k: s.caches[0][k].copy() for k in ("k", "v")}
    for i, tok in enumerate(prompt):
        ref = orc.model_forward(cache, int(tok), pos0 + i)
    d = float(np.abs(got - ref).max()) / float(ref.std())
    log("  last logits max|d|/std = %.3g, top-1 %d vs %d" % (d, int(np.argmax(got)), int(np.argmax(ref))))
    assert d <= 2e-2
    assert int(np.argmax(got)) == int(np.argmax(ref))
    # each prompt position's keys and values, recomputed by the oracle from
    # the GPU's cache of the positions before it (so that one position's
    # rounding does not carry into the next), agree to one bf16 ulp plus
    # HILO_TOL * rms
    k_all, v_all = kv.read_sequence(0, pos0 + T)
    assert np.array_equal(k_all[:, :, :pos0], s.caches[0]["k"][:, :, :pos0])
    assert np.array_equal(v_all[:, :, :pos0], s.caches[0]["v"][:, :, :pos0])
    worst = rows_vs_oracle_from_prefix(orc, s.cap, k_all, v_all, prompt, pos0, range(pos0, pos0 + T))
    log("  K/V rows: worst (|d| - 1 ulp) / rms = %.3g" % worst)
    assert worst <= HILO_TOL



def test_prefill_modes_bitwise(mid_weights):
    # persistent and kernel-per-op run the same tasks: the same bits
    log("prefill: persistent vs kernel-per-op, bitwise")
    _, kv_a, a, _ = _prefill_case(mid_weights, 16, 30, 35)
    _, kv_b, b, _ = _prefill_case(mid_weights, 16, 30, 35, mode=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for x, y in zip(kv_a.read_sequence(0, 65), kv_b.read_sequence(0, 65)):
        assert np.array_equal(x, y)


def test_prefill_then_decode_continues(mid_weights):
    # a decode plan picks up the prefilled cache: its first greedy steps agree
    # with the oracle run over the whole prompt and the same tokens
    import torch
    from persistent_task_graph_amd import harness

    log("prefill 24 tokens, then 3 batch-1 decode steps on the same cache")
    s, kv, last, prompt = _prefill_case(mid_weights, 16, 0, 24)
    orc = oracle.Oracle(MID, s.weights)
    cache = {k: s.caches[0][k].copy() for k in ("k", "v")}
    for i, tok in enumerate(prompt):
        orc.model_forward(cache, int(tok), i)
    plan = harness.build_plan(MID, 1, s.cap)
    tok = torch.tensor([int(np.argmax(last))], dtype=torch.int32, device="cuda")
    d_len = torch.tensor([len(prompt)], dtype=torch.int32, device="cuda")
    logits = torch.empty((1, MID.vocab), dtype=torch.float32, device="cuda")
    for t in range(3):
        fed = int(tok.item())
        plan.step_greedy(s.dm.struct, kv.struct, tok, d_len, logits)
        ref = orc.model_forward(cache, fed, len(prompt) + t)
        got = logits.cpu().numpy()[0]
        assert float(np.abs(got - ref).max()) <= 2e-2 * float(ref.std())
        assert int(tok.item()) == int(np.argmax(ref))
    assert plan.device_error() == 0
    plan.close()


# ---------------------------------------------------------------- tiled weights

def _tiled(s):
    """The same setup with the layer matrices and the LM head in the tiled
    layout (mk_pack_tiled); the embedding and gains are shared."""
    import copy
    import types

    if s.dm.struct_tiled is None:
        s.dm.add_tiled()
    t = copy.copy(s)
    # the struct holds bare pointers: keep the DeviceModel (and so the
    # tensors they point into) alive with the view
    t.dm = types.SimpleNamespace(struct=s.dm.struct_tiled, owner=s.dm)
    return t


def test_pack_tiled_matches_layout():
    # the layout as mk.h defines it: row 8u + i, column 32 s + 8 j + e of the
    # row-major matrix at u * 8 * cols + s * 256 + (8 j + i) * 8 + e
    import torch
    from persistent_task_graph_amd import harness, mk

    rng = np.random.default_rng(5)
    for R, C in ((8, 64), (40, 192), (24, 4096)):
        w = rng.integers(0, 65536, size=(R, C), dtype=np.uint16)
        src = harness.to_device(w)
        dst = torch.empty_like(src)
        mk.pack_tiled(src, dst, R, C)
        torch.cuda.synchronize()
        got = harness.from_device(dst).reshape(-1)
        want = np.empty(R * C, np.uint16)
        for u in range(R // 8):
            for i in range(8):
                for c in range(C):
                    sidx, j, e = c // 32, (c % 32) // 8, c % 8
                    want[u * 8 * C + sidx * 256 + (8 * j + i) * 8 + e] = w[8 * u + i, c]
        assert np.array_equal(got, want), (R, C)


@pytest.mark.parametrize("B,paged,opts", [
    (3, False, {}),                 # the batch-4 instance with one empty column
    (16, False, {}),
    (8, True, {}),                  # paged cache
    (16, False, {"mode": 1}),       # kernel-per-op
    (16, False, {"jit": 3}),        # JIT expanded by the completing QKV arrival
    (4, False, {"schedule": 1}),    # static schedule (16-row task cuts)
])
def test_mid_tiled_weights_bitwise(mid_weights, B, paged, opts):
    # the matrix-core GEMV reads the same operands from the tiled copies: the
    # logits and the greedy tokens are the row-major layout's, bit for bit
    lens = [int(v) for v in np.linspace(5, 700, B)]
    log("mid bf16: tiled vs row-major weights, B=%d paged=%s %s" % (B, paged, opts))
    cap = max(lens) + 8
    table = synth.block_table([cap] * B, 16) if paged else None
    s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=paged, table=table)
    t0 = _tokens(MID, B, 21)
    a, _ = _logits_seq(s, 3, tokens=t0, **opts)
    b, _ = _logits_seq(_tiled(s), 3, tokens=t0, tiled=True, **opts)
    _bitwise(a, b)
    for (ta, la, na), (tb, lb, nb) in zip(a, b):
        assert np.array_equal(na, nb)


def test_mid_tiled_weights_match_oracle(mid_weights):
    # and against the oracle directly (batch 16, ragged lengths)
    B = 16
    lens = [int(v) for v in np.linspace(0, 530, B)]
    s = _tiled(make_setup(MID, B, lens, 540, weights=mid_weights))
    plan = plan_for(s, tiled=True)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID, B, 23), 2)
    assert err == 0
    orc, _ = run_oracle(s, out)
    worst, agree = compare(out, orc)
    log("mid tiled B=16: max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2
    assert agree >= 0.99
    plan.close()


def test_prefill_tiled_weights_bitwise(mid_weights):
    log("prefill: tiled vs row-major weights, bitwise")
    _, kv_a, a, _ = _prefill_case(mid_weights, 16, 30, 35)
    _, kv_b, b, _ = _prefill_case(mid_weights, 16, 30, 35, tiled=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for x, y in zip(kv_a.read_sequence(0, 65), kv_b.read_sequence(0, 65)):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- K-split down projection

@pytest.mark.parametrize("ks,oks", [(1, 1), (2, 2), (4, 4), (4, 1), (1, 4)])
def test_mid_down_ksplit_matches_oracle(mid_weights_g, ks, oks):
    # the down and O projections with their K cut into 1, 2 or 4 parts merged
    # by the last arrival, against the oracle (seeded gains), batch 16, ragged
    # lengths; a part that merged the wrong partials, or too few, fails here
    B = 16
    lens = [int(v) for v in np.linspace(2, 610, B)]
    log("mid bf16: down K split %d, O K split %d, B=16" % (ks, oks))
    s = make_setup(MID, B, lens, 620, weights=mid_weights_g)
    plan = plan_for(s, down_ksplit=ks, o_ksplit=oks)
    kv = device_kv(s)
    out, err = run_gpu(s, plan, kv, _tokens(MID, B, 31), 2)
    assert err == 0
    rows = [0, 6, 15]
    orc, _ = run_oracle(s, out, rows=rows)
    worst, agree = compare(out, orc, rows=rows)
    log("  max|d|/std = %.3g, top-1 = %.3f" % (worst, agree))
    assert worst <= 2e-2
    assert agree >= 0.99
    plan.close()


@pytest.mark.parametrize("ks,B,paged", [(2, 16, False), (4, 3, False), (4, 8, True)])
def test_mid_down_ksplit_modes_bitwise(mid_weights, ks, B, paged):
    # one plan's K split gives the same bits in every execution mode
    lens = [int(v) for v in np.linspace(7, 640, B)]
    log("mid bf16: down K split %d, B=%d paged=%s: persistent vs kernel-per-op vs JIT" % (ks, B, paged))
    cap = max(lens) + 8
    table = synth.block_table([cap] * B, 16) if paged else None
    s = make_setup(MID, B, lens, cap, weights=mid_weights, paged=paged, table=table)
    t0 = _tokens(MID, B, 33)
    a, _ = _logits_seq(s, 3, tokens=t0, down_ksplit=ks, o_ksplit=ks)
    b, _ = _logits_seq(s, 3, tokens=t0, down_ksplit=ks, o_ksplit=ks, mode=1)
    c, _ = _logits_seq(s, 3, tokens=t0, down_ksplit=ks, o_ksplit=ks, jit=1)
    others = [b, c]
    if B >= 5:
        others.append(_logits_seq(s, 3, tokens=t0, down_ksplit=ks, o_ksplit=ks, jit=3)[0])
    for o in others:
        _bitwise(a, o)
