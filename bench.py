"""Decode throughput of the persistent task-graph megakernel on one MI355X.

Workload (the headline): the 36-layer Qwen3-8B-shaped decoder (hidden 4096,
32 query / 8 KV heads of 128, SwiGLU 12288, vocab 151936, bf16 weights
~N(0, 0.02) from a fixed seed), batch 1, a prompt of 1024 random token ids
prefilled by a prefill plan, 16 positions per launch (timed on its own, outside
the decode's timed region), then greedy decode. One timed step = one mk_decode_step_greedy launch: the
whole step, the greedy argmax and the seq_lens increment in one persistent
launch.
Further numbers, reported inside the same JSON object: the same model at
batch 16 with KV lengths log-uniform in [32, 4096] (`batch16`), at batch 8
with a paged cache and KV lengths uniform in [4096, 16384] (`batch8_paged`),
one 8B-shaped layer with hidden-state input/output, rotating over three
weight copies so that the weights come from HBM (`layer8b`), and the tiny
fp32 two-layer model (`tiny`, latency-bound: us/step only). The matrix-core
plans (batch 16, batch 8, the prefill chunks) read tiled copies of the layer
matrices and the LM head (mk_pack_tiled; the same bits as row-major, which the
batch-16 ablation times too); --no-tiled keeps them row-major.
--phases B prints instead a per-operator summary of the in-kernel task
trace (where a step's time goes) at batch B; --cpu-extended times the oracle
on the first steps of the batch-16 and paged workloads (all rows).

Printed: ONE JSON line with tok/s (value), ms/step, HBM roofline of the
megakernel (algorithmic bytes / average launch time from HIP events on the
launch stream) and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PREFILL_CHUNK = 16  # prompt positions per prefill launch
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "persistent_decode_q8b_b1_hbm_traffic.md")


def kernel_source_hash() -> str:
    """sha256 over the device sources (name + bytes, sorted by name)."""
    import hashlib

    h = hashlib.sha256()
    d = os.path.join(ROOT, "persistent_task_graph_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the batch-1 megakernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when that summary is
    missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(l.split(":", 1) for l in f.read().splitlines() if l.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
    except OSError:
        return None
    if kv.get("source_sha256", "").strip() != kernel_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--prompt", type=int, default=1024, help="prompt length (prefilled in chunks of 16 positions)")
    ap.add_argument("--no-b16", action="store_true", help="skip the batch-16 measurement")
    ap.add_argument("--b16-steps", type=int, default=64)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged batch-8 long-context measurement")
    ap.add_argument("--paged-steps", type=int, default=32)
    ap.add_argument("--no-layer", action="store_true", help="skip the single-layer measurement")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the JIT-scheduler and kernel-per-op step times at batch 1 and 16")
    ap.add_argument("--ablation-steps", type=int, default=32)
    ap.add_argument("--multi-step", type=int, default=16, metavar="N",
                    help="also time the batch-1 decode with N greedy steps per launch (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", type=int, default=0, help="0 persistent, 1 kernel-per-op")
    ap.add_argument("--jit", type=int, default=0)
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--lds-preload", type=int, default=0, help="1: preload GEMV rows into LDS pages (batch <= 2)")
    ap.add_argument("--prefetch-kb", type=int, default=0,
                    help="KB of the awaited task's weights each worker prefetches (0: the plan default, -1: none)")
    ap.add_argument("--quick", action="store_true", help="tiny prompt, few steps (profiling runs)")
    ap.add_argument("--no-tiled", action="store_true",
                    help="row-major weights for the matrix-core plans too (default: their tiled copies)")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny-model step time")
    ap.add_argument("--no-w4", action="store_true", help="skip the 4-bit-weight (W4A16) batch-1 measurement")
    ap.add_argument("--w4-steps", type=int, default=64)
    ap.add_argument("--phases", type=int, default=0, metavar="B",
                    help="print the per-operator task-trace summary of the 8B model at batch B (1, 16 or 8 = paged) "
                         "and exit")
    ap.add_argument("--cpu-extended", action="store_true",
                    help="time the oracle on all rows of the first steps of the batch-16 and paged workloads and exit")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="run one plain elementwise copy (torch.neg) of MIB MiB of fp32 first, untimed: the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.cpu_extended:
        cpu_extended(args)
        return
    if args.phases:
        phases(args)
        return
    if args.quick:
        args.prompt, args.steps, args.warmup, args.b16_steps, args.paged_steps = 64, 8, 2, 8, 4

    import torch

    import synth
    from persistent_task_graph_amd import harness, mk

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.copy_calib > 0:
        n = args.copy_calib * (1 << 20) // 4
        xs = torch.ones(n, dtype=torch.float32, device=dev)
        ys = torch.empty_like(xs)
        torch.cuda.synchronize()
        torch.neg(xs, out=ys)
        torch.cuda.synchronize()
        del xs, ys
    shape = synth.Q8B
    wl = synth.WORKLOADS["q8b_b1"]
    t0 = time.time()
    weights = synth.model_weights(shape)
    log("weights generated in %.1fs" % (time.time() - t0))
    t0 = time.time()
    dm = harness.DeviceModel(shape, weights, dev)
    # the matrix-core plans (batch 16 and 8, the 16-position prefill chunks)
    # read tiled copies of the layer matrices and the LM head
    tiled = not args.no_tiled
    if tiled:
        dm.add_tiled()
    torch.cuda.synchronize()
    log("weights uploaded%s in %.1fs" % (" and tiled" if tiled else "", time.time() - t0))

    def wstruct(o):
        return dm.struct_tiled if o.get("tiled") else dm.struct
    opts = dict(mode=args.mode, jit=args.jit, kv_chunk=args.kv_chunk, workers=args.workers,
                lds_preload=args.lds_preload, prefetch_kb=args.prefetch_kb)

    # ---------------------------------------------------------------- batch 1
    B = 1
    n_abl = 0 if args.no_ablation else 5 * (args.ablation_steps + 4)  # at most five ablation runs
    n_multi = 0 if args.multi_step <= 0 else args.multi_step * (1 + max(1, args.steps // args.multi_step))
    cap = args.prompt + args.warmup + args.steps + n_abl + n_multi + 8
    kv = harness.DeviceKV(shape, B, cap)
    plan = harness.build_plan(shape, B, cap, **opts)
    info = plan.info()
    st = torch.cuda.current_stream()
    prompt = synth.tokens(wl, n=max(args.prompt, 1)).reshape(-1)
    d_tok = torch.zeros(B, dtype=torch.int32, device=dev)
    d_len = torch.zeros(B, dtype=torch.int32, device=dev)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device=dev)
    d_prompt = torch.from_numpy(prompt.astype(np.int32)).to(dev)
    prefill = None
    if args.prompt > 0:
        # the prompt in chunks of 16 positions per launch (a prefill plan);
        # the second, timed run rewrites the same bits into the cache
        pplan = harness.build_plan(shape, PREFILL_CHUNK, cap, prefill=1, mode=args.mode, workers=args.workers,
                                   tiled=tiled)
        plog = torch.empty(shape.vocab, dtype=torch.float32, device=dev)
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pplan.prefill(wstruct(dict(tiled=tiled)), kv.struct, d_prompt, 0, args.prompt, plog)
        torch.cuda.synchronize()
        pe0.record(st)
        pplan.prefill(wstruct(dict(tiled=tiled)), kv.struct, d_prompt, 0, args.prompt, plog)
        pe1.record(st)
        torch.cuda.synchronize()
        if pplan.device_error():
            raise SystemExit("device error during prefill")
        pplan.close()
        p_ms = pe0.elapsed_time(pe1)
        n_launch = -(-args.prompt // PREFILL_CHUNK)
        prefill = {"prompt_tokens": args.prompt, "positions_per_launch": PREFILL_CHUNK, "launches": n_launch,
                   "ms": round(p_ms, 3), "ms_per_launch": round(p_ms / n_launch, 4),
                   "value": round(args.prompt / (p_ms * 1e-3), 1), "unit": "prompt tokens/s"}
        logits[0].copy_(plog)
        d_len.fill_(args.prompt)
        plan.argmax(logits, d_tok)
        torch.cuda.synchronize()
        log("prefill of %d tokens: %.1f ms in %d launches (%.0f tokens/s)"
            % (args.prompt, p_ms, n_launch, prefill["value"]))

    def run(n, plan, kv, d_tok, d_len, logits, events=None, ws=None):
        # greedy decode: each launch also writes the next tokens and advances the lengths
        ws = dm.struct if ws is None else ws
        for i in range(n):
            if events is not None:
                events[i][0].record(st)
            plan.step_greedy(ws, kv.struct, d_tok, d_len, logits)
            if events is not None:
                events[i][1].record(st)

    def ablation(Bn, capn, kv, d_tok, d_len, logits, base=None):
        """ms/step of the same step with JIT attention through the scheduler
        waves, with JIT attention expanded by the completing QKV arrival on
        all workers, in kernel-per-operator mode (same results, bitwise),
        with the static (searched) schedule (its own fixed split length) and,
        for a plan on tiled weights, with the row-major ones (same bits)."""
        base = opts if base is None else base
        out = {"kv_len_start": int(d_len[0].item())}
        runs = [("jit_scheduler", dict(base, jit=1))]
        if Bn >= 5:  # JIT expanded by the completing QKV arrival: the batch >= 8 instances
            runs.append(("jit_inline", dict(base, jit=3)))
        runs += [("kernel_per_op", dict(base, mode=1)), ("static_schedule", dict(base, schedule=1))]
        if base.get("tiled"):
            runs.append(("row_major_weights", dict(base, tiled=False)))
        for name, o in runs:
            pl = harness.build_plan(shape, Bn, capn, **o)
            run(4, pl, kv, d_tok, d_len, logits, ws=wstruct(o))
            torch.cuda.synchronize()
            e0.record(st)
            run(args.ablation_steps, pl, kv, d_tok, d_len, logits, ws=wstruct(o))
            e1.record(st)
            torch.cuda.synchronize()
            err = pl.device_error()
            if err:
                raise SystemExit("device error %d in the %s ablation" % (err, name))
            out[name + "_ms_per_step"] = round(e0.elapsed_time(e1) / args.ablation_steps, 4)
            pl.close()
        return out

    run(args.warmup, plan, kv, d_tok, d_len, logits)
    torch.cuda.synchronize()
    len0 = int(d_len.item())
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    run(args.steps, plan, kv, d_tok, d_len, logits, ev)
    e1.record(st)
    torch.cuda.synchronize()
    err = plan.device_error()
    if err:
        raise SystemExit("device error %d during timed steps" % err)
    total_ms = e0.elapsed_time(e1)
    k_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = total_ms / args.steps
    # algorithmic bytes per launch: weights once + KV of L+1 keys read + append + embed row + logits
    bytes_per = [harness.step_bytes(shape, [len0 + i], B) for i in range(args.steps)]
    avg_bytes = float(np.mean(bytes_per))
    k_avg = float(k_ms.mean())
    achieved = avg_bytes / (k_avg * 1e-3) / 1e9
    tok_s = B * args.steps / (total_ms * 1e-3)
    log("B=1: %.3f ms/step (kernel avg %.3f, median %.3f, p99 %.3f), %.1f tok/s, %.0f GB/s = %.1f%% of 8 TB/s"
        % (ms_per_step, k_avg, np.median(k_ms), np.percentile(k_ms, 99), tok_s, achieved, 100 * achieved / PEAK_HBM_GBS))
    multi = None
    if args.multi_step > 0:
        # the same decode with N greedy steps per launch (tokens and lengths
        # fed forward on the device): one warm-up launch, then the timed ones
        N = args.multi_step
        nl = max(1, args.steps // N)
        out_tok = torch.empty((N, B), dtype=torch.int32, device=dev)
        plan.steps_greedy(dm.struct, kv.struct, d_tok, d_len, logits, N, out_tok)
        torch.cuda.synchronize()
        lenm = int(d_len.item())
        e0.record(st)
        for _ in range(nl):
            plan.steps_greedy(dm.struct, kv.struct, d_tok, d_len, logits, N, out_tok)
        e1.record(st)
        torch.cuda.synchronize()
        if plan.device_error():
            raise SystemExit("device error in the multi-step launches")
        ms_m = e0.elapsed_time(e1) / (nl * N)
        bytes_m = float(np.mean([harness.step_bytes(shape, [lenm + i], B) for i in range(nl * N)]))
        multi = {"steps_per_launch": N, "launches": nl, "ms_per_step": round(ms_m, 4),
                 "value": round(B / (ms_m * 1e-3), 2), "unit": "tokens/s", "kv_len_start": lenm,
                 "hbm_gbs": round(bytes_m / (ms_m * 1e-3) / 1e9, 1),
                 "hbm_frac": round(bytes_m / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log("B=1, %d steps per launch: %.3f ms/step, %.1f tok/s" % (N, ms_m, B / (ms_m * 1e-3)))
    plan.close()
    abl1 = None
    if not args.no_ablation:
        abl1 = ablation(B, cap, kv, d_tok, d_len, logits)
        log("B=1 ablation: %s" % abl1)
    del kv

    result = {
        "metric": "decode tokens/s at batch 1 (36-layer Qwen3-8B-shaped, bf16 weights)",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02), random prompt ids)",
        "config": {
            "workload": "q8b_b1: 36-layer Qwen3-8B-shaped decoder, batch 1, prompt %d (prefilled), greedy decode"
                        % args.prompt,
            "batch": B, "kv_len_start": len0, "mode": "persistent" if args.mode == 0 else "kernel_per_op",
            "workers": info.workers, "sched_waves": info.sched_waves, "kv_chunk": info.kv_chunk,
            "attention": "JIT (scheduler waves)" if info.jit else "AOT slots",
        },
        "kernel_ms": {"mean": round(k_avg, 4), "median": round(float(np.median(k_ms)), 4),
                      "p99": round(float(np.percentile(k_ms, 99)), 4)},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
            "kernel": "persistent decode-step megakernel (one launch per step)",
            "bytes_per_launch": int(avg_bytes),
        },
    }
    if abl1 is not None:
        result["ablation_b1"] = abl1
    if multi is not None:
        result["multi_step_b1"] = multi
    if prefill is not None:
        # the same prompt as single-token steps would take prompt x ms_per_step
        prefill["decode_path_ms_estimate"] = round(args.prompt * ms_per_step, 1)
        result["prefill_b1"] = prefill

    # ---------------------------------------------------------------- batch 16
    if not args.no_b16:
        wl16 = synth.WORKLOADS["q8b_b16"]
        B16 = wl16.batch
        lens = synth.seq_lengths(wl16)
        cap16 = int(lens.max()) + args.warmup + args.b16_steps + n_abl + 8
        t0 = time.time()
        kv16 = harness.DeviceKV(shape, B16, cap16)
        caches = synth.kv_contents(shape, lens, int(lens.max()) + 1)
        for b in range(B16):
            kv16.load_sequence(b, caches[b]["k"], caches[b]["v"], int(lens[b]))
        del caches
        torch.cuda.synchronize()
        log("B=16 KV ready in %.1fs" % (time.time() - t0))
        opts16 = dict(opts, tiled=tiled)
        plan16 = harness.build_plan(shape, B16, cap16, **opts16)
        d_tok16 = torch.from_numpy(synth.tokens(wl16)).to(dev)
        d_len16 = torch.from_numpy(lens.astype(np.int32)).to(dev)
        logits16 = torch.empty((B16, shape.vocab), dtype=torch.float32, device=dev)
        run(args.warmup, plan16, kv16, d_tok16, d_len16, logits16, ws=wstruct(opts16))
        torch.cuda.synchronize()
        l16 = d_len16.cpu().numpy().copy()
        ev16 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.b16_steps)]
        e0.record(st)
        run(args.b16_steps, plan16, kv16, d_tok16, d_len16, logits16, ev16, ws=wstruct(opts16))
        e1.record(st)
        torch.cuda.synchronize()
        err = plan16.device_error()
        if err:
            raise SystemExit("device error %d during batch-16 steps" % err)
        t16 = e0.elapsed_time(e1)
        k16 = np.array([a.elapsed_time(b) for a, b in ev16])
        b16_bytes = float(np.mean([harness.step_bytes(shape, (l16 + i).tolist(), B16) for i in range(args.b16_steps)]))
        ach16 = b16_bytes / (k16.mean() * 1e-3) / 1e9
        tok16 = B16 * args.b16_steps / (t16 * 1e-3)
        log("B=16: %.3f ms/step (kernel avg %.3f), %.1f tok/s, %.0f GB/s = %.1f%%"
            % (t16 / args.b16_steps, k16.mean(), tok16, ach16, 100 * ach16 / PEAK_HBM_GBS))
        result["batch16"] = {
            "workload": "q8b_b16: same model, batch 16, KV lengths log-uniform in [32, 4096] (seeded)",
            "value": round(tok16, 2), "unit": "tokens/s", "ms_per_step": round(t16 / args.b16_steps, 4),
            "kernel_ms_mean": round(float(k16.mean()), 4), "hbm_gbs": round(ach16, 1),
            "hbm_frac": round(ach16 / PEAK_HBM_GBS, 4), "bytes_per_launch": int(b16_bytes),
            "weights": "tiled" if tiled else "row-major",
        }
        plan16.close()
        if not args.no_ablation:
            result["batch16"]["ablation"] = ablation(B16, cap16, kv16, d_tok16, d_len16, logits16, base=opts16)
            log("B=16 ablation: %s" % result["batch16"]["ablation"])
        del kv16

    # ---------------------------------------------------------------- batch 8, paged, long context
    if not args.no_paged:
        wl8 = synth.WORKLOADS["q8b_b8_paged"]
        B8, st8 = wl8.batch, args.paged_steps
        lens8 = synth.seq_lengths(wl8)
        cap8 = int(lens8.max()) + args.warmup + st8 + 8
        table8 = synth.block_table([cap8] * B8, wl8.kv_block)
        t0 = time.time()
        kv8 = harness.DeviceKV(shape, B8, cap8, paged=True, block=wl8.kv_block, block_table=table8)
        # cache contents: seeded N(0,1) drawn on the device (timing does not
        # depend on the values; the parity tests use the host generator)
        gen = torch.Generator(device=dev)
        gen.manual_seed(synth.SEED_KV)
        for t in (kv8.k, kv8.v):
            for l in range(t.shape[0]):
                t[l].copy_(torch.randn(t[l].shape, generator=gen, device=dev).to(torch.bfloat16).view(torch.int16))
        torch.cuda.synchronize()
        log("B=8 paged KV ready in %.1fs (%d blocks)" % (time.time() - t0, kv8.n_blocks))
        opts8 = dict(opts, tiled=tiled)
        plan8 = harness.build_plan(shape, B8, cap8, paged=True, block=wl8.kv_block, max_blocks=table8.shape[1], **opts8)
        d_tok8 = torch.from_numpy(synth.tokens(wl8)).to(dev)
        d_len8 = torch.from_numpy(lens8.astype(np.int32)).to(dev)
        logits8 = torch.empty((B8, shape.vocab), dtype=torch.float32, device=dev)
        run(args.warmup, plan8, kv8, d_tok8, d_len8, logits8, ws=wstruct(opts8))
        torch.cuda.synchronize()
        l8 = d_len8.cpu().numpy().copy()
        ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(st8)]
        e0.record(st)
        run(st8, plan8, kv8, d_tok8, d_len8, logits8, ev8, ws=wstruct(opts8))
        e1.record(st)
        torch.cuda.synchronize()
        err = plan8.device_error()
        if err:
            raise SystemExit("device error %d during paged batch-8 steps" % err)
        t8 = e0.elapsed_time(e1)
        k8 = np.array([a.elapsed_time(b) for a, b in ev8])
        b8_bytes = float(np.mean([harness.step_bytes(shape, (l8 + i).tolist(), B8) for i in range(st8)]))
        ach8 = b8_bytes / (k8.mean() * 1e-3) / 1e9
        tok8 = B8 * st8 / (t8 * 1e-3)
        log("B=8 paged: %.3f ms/step (kernel avg %.3f), %.1f tok/s, %.0f GB/s = %.1f%%"
            % (t8 / st8, k8.mean(), tok8, ach8, 100 * ach8 / PEAK_HBM_GBS))
        result["batch8_paged"] = {
            "workload": "q8b_b8_paged: same model, batch 8, paged KV (16-token blocks, permuted block table), "
                        "KV lengths uniform in [4096, 16384] (seeded)",
            "value": round(tok8, 2), "unit": "tokens/s", "ms_per_step": round(t8 / st8, 4),
            "kernel_ms_mean": round(float(k8.mean()), 4), "hbm_gbs": round(ach8, 1),
            "hbm_frac": round(ach8 / PEAK_HBM_GBS, 4), "bytes_per_launch": int(b8_bytes),
            "weights": "tiled" if tiled else "row-major",
        }
        plan8.close()
        del kv8

    # ---------------------------------------------------------------- one 8B layer, hidden I/O
    if not args.no_layer:
        wlL = synth.WORKLOADS["layer8b"]
        shL = wlL.shape
        lensL = synth.seq_lengths(wlL)
        stL = wlL.steps
        capL = int(lensL.max()) + args.warmup + stL + 8
        # three copies of the layer's weights (1.16 GB), used in turn: a step
        # never finds its weights in the 256 MB memory-side cache, so the
        # rate is an HBM rate (the copies are equal: results do not change)
        wL = synth.model_weights(shL)
        dmLs = [harness.DeviceModel(shL, wL, dev) for _ in range(3)]
        kvL = harness.DeviceKV(shL, 1, capL)
        cL = synth.kv_sequence(shL, 0, int(lensL[0]), capL)
        kvL.load_sequence(0, cL["k"], cL["v"], int(lensL[0]))
        planL = harness.build_plan(shL, 1, capL, **opts)
        xs = [torch.from_numpy(synth.hidden_inputs(shL, 1, t)).to(dev) for t in range(args.warmup + stL)]
        xo = torch.empty((1, shL.hidden), dtype=torch.float32, device=dev)
        d_lenL = torch.from_numpy(lensL.astype(np.int32)).to(dev)
        for t in range(args.warmup):
            planL.step_hidden(dmLs[t % 3].struct, kvL.struct, xs[t], d_lenL, xo)
            d_lenL += 1
        torch.cuda.synchronize()
        l0 = int(d_lenL.item())
        evL = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(stL)]
        for t in range(stL):
            evL[t][0].record(st)
            planL.step_hidden(dmLs[t % 3].struct, kvL.struct, xs[args.warmup + t], d_lenL, xo)
            evL[t][1].record(st)
            d_lenL += 1
        torch.cuda.synchronize()
        if planL.device_error():
            raise SystemExit("device error during single-layer steps")
        kL = np.array([a.elapsed_time(b) for a, b in evL])
        bL = float(np.mean([harness.step_bytes(shL, [l0 + i], 1) for i in range(stL)]))
        achL = bL / (kL.mean() * 1e-3) / 1e9
        log("layer8b: %.2f us/layer-step (median %.2f), %.0f GB/s = %.1f%%"
            % (kL.mean() * 1e3, np.median(kL) * 1e3, achL, 100 * achL / PEAK_HBM_GBS))
        result["layer8b"] = {
            "workload": "layer8b: one Qwen3-8B-shaped decoder layer, hidden state in/out, batch 1, KV 512 -> 576",
            "value": round(float(kL.mean()) * 1e3, 2), "unit": "us/layer-step",
            "median_us": round(float(np.median(kL)) * 1e3, 2), "hbm_gbs": round(achL, 1),
            "hbm_frac": round(achL / PEAK_HBM_GBS, 4), "bytes_per_launch": int(bL),
            "note": "386 MB of weights per step, three weight copies used in turn (1.16 GB): each step reads its "
                    "weights from HBM, not from the 256 MB memory-side cache",
        }
        planL.close()
        del dmLs

    # ---------------------------------------------------------------- 4-bit layer matrices (W4A16), batch 1
    if not args.no_w4:
        del dm
        torch.cuda.empty_cache()
        wl4 = synth.WORKLOADS["q8b_w4_b1"]
        sh4 = wl4.shape
        t0 = time.time()
        dm4 = harness.DeviceModel(sh4, synth.model_weights(sh4), dev)
        L04 = int(synth.seq_lengths(wl4)[0])
        cap4 = L04 + args.warmup + args.w4_steps + 8
        kv4 = harness.DeviceKV(sh4, 1, cap4)
        c4 = synth.kv_sequence(sh4, 0, L04, cap4)
        kv4.load_sequence(0, c4["k"], c4["v"], L04)
        del c4
        log("W4 model ready in %.1fs" % (time.time() - t0))
        plan4 = harness.build_plan(sh4, 1, cap4, **opts)
        d_tok4 = torch.from_numpy(synth.tokens(wl4)).to(dev)
        d_len4 = torch.full((1,), L04, dtype=torch.int32, device=dev)
        logits4 = torch.empty((1, sh4.vocab), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            plan4.step_greedy(dm4.struct, kv4.struct, d_tok4, d_len4, logits4)
        torch.cuda.synchronize()
        l4 = int(d_len4.item())
        ev4 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.w4_steps)]
        e0.record(st)
        for i in range(args.w4_steps):
            ev4[i][0].record(st)
            plan4.step_greedy(dm4.struct, kv4.struct, d_tok4, d_len4, logits4)
            ev4[i][1].record(st)
        e1.record(st)
        torch.cuda.synchronize()
        if plan4.device_error():
            raise SystemExit("device error during W4 steps")
        t4 = e0.elapsed_time(e1)
        k4 = np.array([a.elapsed_time(b) for a, b in ev4])
        b4 = float(np.mean([harness.step_bytes(sh4, [l4 + i], 1) for i in range(args.w4_steps)]))
        ach4 = b4 / (k4.mean() * 1e-3) / 1e9
        log("W4 B=1: %.3f ms/step (kernel avg %.3f), %.1f tok/s, %.0f GB/s = %.1f%%"
            % (t4 / args.w4_steps, k4.mean(), args.w4_steps / (t4 * 1e-3), ach4, 100 * ach4 / PEAK_HBM_GBS))
        result["w4_b1"] = {
            "workload": "q8b_w4_b1: the same 36-layer model with 4-bit layer matrices (group 128, bf16 scales; bf16 "
                        "embedding and LM head), batch 1, 1024 cached random keys, greedy decode",
            "value": round(args.w4_steps / (t4 * 1e-3), 2), "unit": "tokens/s",
            "ms_per_step": round(t4 / args.w4_steps, 4), "kernel_ms_mean": round(float(k4.mean()), 4),
            "hbm_gbs": round(ach4, 1), "hbm_frac": round(ach4 / PEAK_HBM_GBS, 4), "bytes_per_launch": int(b4),
        }
        plan4.close()
        del kv4
        # the same 4-bit model at batch 16 (matrix cores), log-uniform KV lengths
        wl16 = synth.WORKLOADS["q8b_b16"]
        lens16 = synth.seq_lengths(wl16)
        cap16w = int(lens16.max()) + args.warmup + args.w4_steps + 8
        kv16w = harness.DeviceKV(sh4, 16, cap16w)
        gen = torch.Generator(device=dev)
        gen.manual_seed(synth.SEED_KV)
        for tt in (kv16w.k, kv16w.v):
            for li in range(tt.shape[0]):
                tt[li].copy_(torch.randn(tt[li].shape, generator=gen, device=dev).to(torch.bfloat16).view(torch.int16))
        plan16w = harness.build_plan(sh4, 16, cap16w, **opts)
        d_tok16w = torch.from_numpy(synth.tokens(wl16, stream=3)).to(dev)
        d_len16w = torch.from_numpy(lens16.astype(np.int32)).to(dev)
        logits16w = torch.empty((16, sh4.vocab), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            plan16w.step_greedy(dm4.struct, kv16w.struct, d_tok16w, d_len16w, logits16w)
        torch.cuda.synchronize()
        l16 = d_len16w.cpu().numpy().astype(np.int64)
        e0.record(st)
        for i in range(args.w4_steps):
            plan16w.step_greedy(dm4.struct, kv16w.struct, d_tok16w, d_len16w, logits16w)
        e1.record(st)
        torch.cuda.synchronize()
        if plan16w.device_error():
            raise SystemExit("device error during W4 batch-16 steps")
        t16w = e0.elapsed_time(e1) / args.w4_steps
        b16w = float(np.mean([harness.step_bytes(sh4, (l16 + i).tolist(), 16) for i in range(args.w4_steps)]))
        ach16w = b16w / (t16w * 1e-3) / 1e9
        log("W4 B=16: %.3f ms/step, %.1f tok/s, %.0f GB/s = %.1f%%"
            % (t16w, 16 / (t16w * 1e-3), ach16w, 100 * ach16w / PEAK_HBM_GBS))
        result["w4_b16"] = {
            "workload": "q8b_w4_b16: the 4-bit model at batch 16 (matrix-core GEMV, codes dequantized in registers), "
                        "KV lengths log-uniform in [32, 4096] (seeded device-side N(0,1) K/V), greedy decode",
            "value": round(16 / (t16w * 1e-3), 2), "unit": "tokens/s", "ms_per_step": round(t16w, 4),
            "hbm_gbs": round(ach16w, 1), "hbm_frac": round(ach16w / PEAK_HBM_GBS, 4), "bytes_per_launch": int(b16w),
        }
        plan16w.close()
        del dm4, kv16w

    # ---------------------------------------------------------------- tiny fp32 model (latency-bound)
    if not args.no_tiny:
        wlT = synth.WORKLOADS["tiny"]
        shT = wlT.shape
        capT = wlT.capacity() + args.warmup + 8
        lensT = synth.seq_lengths(wlT)
        dmT = harness.DeviceModel(shT, synth.model_weights(shT), dev)
        kvT = harness.DeviceKV(shT, 1, capT)
        cT = synth.kv_sequence(shT, 0, int(lensT[0]), capT)
        kvT.load_sequence(0, cT["k"], cT["v"], int(lensT[0]))
        planT = harness.build_plan(shT, 1, capT)
        d_tokT = torch.from_numpy(synth.tokens(wlT)).to(dev)
        d_lenT = torch.from_numpy(lensT.astype(np.int32)).to(dev)
        logitsT = torch.empty((1, shT.vocab), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            planT.step_greedy(dmT.struct, kvT.struct, d_tokT, d_lenT, logitsT)
        torch.cuda.synchronize()
        evT = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(wlT.steps)]
        e0.record(st)
        for t in range(wlT.steps):
            evT[t][0].record(st)
            planT.step_greedy(dmT.struct, kvT.struct, d_tokT, d_lenT, logitsT)
            evT[t][1].record(st)
        e1.record(st)
        torch.cuda.synchronize()
        if planT.device_error():
            raise SystemExit("device error during tiny-model steps")
        kT = np.array([a.elapsed_time(b) for a, b in evT])
        log("tiny: %.1f us/step (kernel median %.1f us)" % (e0.elapsed_time(e1) / wlT.steps * 1e3, np.median(kT) * 1e3))
        result["tiny"] = {
            "workload": "tiny: 2-layer fp32 decoder (hidden 256, 4 heads x 64, FFN 1024, vocab 1024), batch 1, "
                        "KV 32 + warm-up, %d greedy steps" % wlT.steps,
            "value": round(e0.elapsed_time(e1) / wlT.steps * 1e3, 2), "unit": "us/step",
            "kernel_us_median": round(float(np.median(kT)) * 1e3, 2),
            "note": "about 9.4 MB per step, held in caches: latency-bound, no HBM fraction",
        }
        planT.close()

    # ---------------------------------------------------------------- CPU oracle sample
    if not args.no_cpu:
        import oracle

        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        orc = oracle.Oracle(shape, weights)
        kvlen = 1024
        cache = synth.kv_contents(shape, np.array([kvlen]), kvlen + 64)[0]
        tok = int(prompt[0])
        n = 0
        t0 = time.time()
        while True:
            logits_c = orc.model_forward(cache, tok, kvlen + n)
            tok = int(np.argmax(logits_c))
            n += 1
            if time.time() - t0 >= args.cpu_seconds or n >= 64:
                break
        dt = time.time() - t0
        result["cpu_baseline"] = {
            "value": round(n / dt, 4), "unit": "tokens/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": "%d greedy decode steps of the same 36-layer model, batch 1, KV length %d..%d "
                      "(random N(0,1) KV), plain C oracle with OpenMP over output rows" % (n, kvlen, kvlen + n - 1),
            "cpu_model": cpu_model(),
        }
        log("CPU oracle: %d steps in %.1fs (%.3f tok/s, %d threads)" % (n, dt, n / dt, oracle.get_threads()))
        del orc, cache
        # the oracle on one thread: the tiny model (all 16 steps) and the
        # single 8B layer (8 steps)
        oracle.set_threads(1)
        single = {}
        for name, nsteps in (("tiny", 16), ("layer8b", 8)):
            wlS = synth.WORKLOADS[name]
            shS = wlS.shape
            wS = synth.model_weights(shS)
            orcS = oracle.Oracle(shS, wS)
            L0 = int(synth.seq_lengths(wlS)[0])
            cS = synth.kv_sequence(shS, 0, L0, L0 + nsteps + 1)
            t0 = time.time()
            tokS = int(synth.tokens(wlS)[0])
            for i in range(nsteps):
                if shS.embed_head:
                    tokS = int(np.argmax(orcS.model_forward(cS, tokS, L0 + i)))
                else:
                    orcS.hidden_forward(cS, L0 + i, synth.hidden_inputs(shS, 1, i)[0])
            dtS = time.time() - t0
            unit = "ms/step" if shS.embed_head else "ms/layer-step"
            single[name] = {"value": round(dtS / nsteps * 1e3, 3), "unit": unit, "steps": nsteps}
            log("CPU oracle, 1 thread, %s: %.3f %s" % (name, dtS / nsteps * 1e3, unit))
        oracle.set_threads(threads)
        result["cpu_baseline"]["single_thread"] = single

    print(json.dumps(result), flush=True)


def cpu_extended(args):
    """The oracle on all host cores for the first steps of the batch-16 and
    paged batch-8 workloads, every row (no GPU involved)."""
    import oracle
    import synth

    shape = synth.Q8B
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    orc = oracle.Oracle(shape, synth.model_weights(shape))
    out = {"cpu_model": cpu_model(), "cores": oracle.get_threads()}
    for name in ("q8b_b16", "q8b_b8_paged"):
        wl = synth.WORKLOADS[name]
        lens = synth.seq_lengths(wl)
        toks = synth.tokens(wl)
        steps = 8
        t_all = 0.0
        for b in range(wl.batch):
            c = synth.kv_sequence(shape, b, int(lens[b]), int(lens[b]) + steps + 1)
            tok = int(toks[b])
            t0 = time.time()
            for i in range(steps):
                tok = int(np.argmax(orc.model_forward(c, tok, int(lens[b]) + i)))
            t_all += time.time() - t0
            del c
        out[name] = {"rows": wl.batch, "steps": steps, "seconds": round(t_all, 2),
                     "s_per_step": round(t_all / steps, 3), "tokens_per_s": round(wl.batch * steps / t_all, 3)}
        log("CPU oracle %s: %d rows x %d steps in %.1fs" % (name, wl.batch, steps, t_all))
    print(json.dumps({"cpu_oracle_extended": out}), flush=True)


def phases(args):
    """Per-operator summary of the in-kernel task trace of the 8B model: for
    each operator, the mean over layers of the level's span (first task ready
    to last task done) and the mean per-task times between the trace marks."""
    import torch

    import synth
    from persistent_task_graph_amd import harness, mk

    torch.cuda.set_device(0)
    dev = "cuda"
    shape = synth.Q8B
    name = {1: "q8b_b1", 16: "q8b_b16", 8: "q8b_b8_paged"}[args.phases]
    wl = synth.WORKLOADS[name]
    B = wl.batch
    lens = synth.seq_lengths(wl)
    if name == "q8b_b1":
        lens = np.array([1100])
    cap = int(lens.max()) + 16
    tiled = B >= 3 and not args.no_tiled  # the matrix-core plans read tiled weights, as in the bench
    dm = harness.DeviceModel(shape, synth.model_weights(shape), dev, tiled=tiled)
    table = synth.block_table([cap] * B, wl.kv_block) if wl.paged else None
    kv = harness.DeviceKV(shape, B, cap, paged=wl.paged, block=wl.kv_block, block_table=table)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.SEED_KV)
    for t in (kv.k, kv.v):
        for l in range(t.shape[0]):
            t[l].copy_(torch.randn(t[l].shape, generator=gen, device=dev).to(torch.bfloat16).view(torch.int16))
    plan = harness.build_plan(shape, B, cap, paged=wl.paged, block=wl.kv_block,
                              max_blocks=table.shape[1] if table is not None else 0, trace=4096,
                              mode=args.mode, jit=args.jit, kv_chunk=args.kv_chunk, workers=args.workers,
                              lds_preload=args.lds_preload, prefetch_kb=args.prefetch_kb, tiled=tiled)
    d_tok = torch.from_numpy(synth.tokens(wl)).to(dev)
    d_len = torch.from_numpy(lens.astype(np.int32)).to(dev)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device=dev)
    for _ in range(4):
        plan.step_greedy(dm.struct_tiled if tiled else dm.struct, kv.struct, d_tok, d_len, logits)
    torch.cuda.synchronize()
    tr = plan.trace()
    if plan.device_error():
        raise SystemExit("device error in the traced steps")
    ops = {mk.OP_EMBED: "embed", mk.OP_QKV: "qkv", mk.OP_ATTN: "attention", mk.OP_O: "o_proj",
           mk.OP_GATEUP: "gate_up", mk.OP_DOWN: "down", mk.OP_LM: "lm_head"}
    t0 = int(tr["t_wait"].min())
    rows = {}
    for op, nm in ops.items():
        r = tr[tr["op"] == op]
        if op == mk.OP_ATTN:
            r = r[r["t_a"] > 0]  # slots the step left empty run no body
        if len(r) == 0:
            continue
        # tasks of one level share the layer; group by layer through the task id
        # order within the step: the trace holds one step, so group by t_ready clusters
        ready = (r["t_ready"].astype(np.int64) - t0) / 100.0  # us (100 MHz ticks)
        done = (r["t_done"].astype(np.int64) - t0) / 100.0
        per_task = done - ready
        rows[nm] = {"tasks": int(len(r)), "task_us_mean": round(float(per_task.mean()), 2),
                    "task_us_p90": round(float(np.percentile(per_task, 90)), 2)}
        # per-layer operators: the level's span, first task ready to last task
        # done (the tasks of one layer's level are consecutive in ready order)
        nl = shape.n_layers if nm not in ("embed", "lm_head") else 1
        if len(r) % nl == 0:
            order = np.argsort(ready)
            k = len(r) // nl
            spans = [float(done[order[i * k:(i + 1) * k]].max() - ready[order[i * k:(i + 1) * k]].min())
                     for i in range(nl)]
            rows[nm]["level_span_us_mean"] = round(float(np.mean(spans)), 2)
        for a, b, key in (("t_ready", "t_a", "to_mark_a"), ("t_a", "t_b", "a_to_b"), ("t_b", "t_c", "b_to_c"),
                          ("t_c", "t_d", "c_to_d"), ("t_d", "t_done", "d_to_done")):
            m = (r[a] > 0) & (r[b] > 0)
            if m.any():
                rows[nm][key + "_us"] = round(float(((r[b][m].astype(np.int64) - r[a][m].astype(np.int64)) / 100.0).mean()), 2)
    step_us = (int(tr["t_done"].max()) - t0) / 100.0
    out = {"workload": name, "batch": B, "step_us_traced": round(step_us, 1), "per_op": rows,
           "marks": {"gemv": "a operands ready, b rows done, c outputs stored, d stores complete",
                     "attention": "a prologue done, b K/V pass done, c waves merged, d partial stored"}}
    print(json.dumps(out, indent=1), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
