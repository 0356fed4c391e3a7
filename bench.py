"""Decode throughput of the persistent task-graph megakernel on one MI355X.

Workload (the headline): the 36-layer Qwen3-8B-shaped decoder (hidden 4096,
32 query / 8 KV heads of 128, SwiGLU 12288, vocab 151936, bf16 weights
~N(0, 0.02) from a fixed seed), batch 1, a prompt of 1024 random token ids
prefilled by teacher-forced decode steps (outside the timed region), then
greedy decode. One timed step = one mk_decode_step (the whole step in one
persistent launch) + mk_argmax + the caller's seq_lens increment.
Further numbers, reported inside the same JSON object: the same model at
batch 16 with KV lengths log-uniform in [32, 4096] (`batch16`), at batch 8
with a paged cache and KV lengths uniform in [4096, 16384] (`batch8_paged`),
and one 8B-shaped layer with hidden-state input/output (`layer8b`).

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
    ap.add_argument("--prompt", type=int, default=1024, help="prefill length (teacher-forced steps)")
    ap.add_argument("--no-b16", action="store_true", help="skip the batch-16 measurement")
    ap.add_argument("--b16-steps", type=int, default=64)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged batch-8 long-context measurement")
    ap.add_argument("--paged-steps", type=int, default=32)
    ap.add_argument("--no-layer", action="store_true", help="skip the single-layer measurement")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the JIT-scheduler and kernel-per-op step times at batch 1 and 16")
    ap.add_argument("--ablation-steps", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", type=int, default=0, help="0 persistent, 1 kernel-per-op")
    ap.add_argument("--jit", type=int, default=0)
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--quick", action="store_true", help="tiny prompt, few steps (profiling runs)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="run one plain elementwise copy (torch.neg) of MIB MiB of fp32 first, untimed: the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
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
    torch.cuda.synchronize()
    log("weights uploaded in %.1fs" % (time.time() - t0))
    opts = dict(mode=args.mode, jit=args.jit, kv_chunk=args.kv_chunk, workers=args.workers)

    # ---------------------------------------------------------------- batch 1
    B = 1
    n_abl = 0 if args.no_ablation else 2 * (args.ablation_steps + 4)
    cap = args.prompt + args.warmup + args.steps + n_abl + 8
    kv = harness.DeviceKV(shape, B, cap)
    plan = harness.build_plan(shape, B, cap, **opts)
    info = plan.info()
    st = torch.cuda.current_stream()
    prompt = synth.tokens(wl, n=max(args.prompt, 1)).reshape(-1)
    d_tok = torch.zeros(B, dtype=torch.int32, device=dev)
    d_len = torch.zeros(B, dtype=torch.int32, device=dev)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device=dev)
    t0 = time.time()
    d_prompt = torch.from_numpy(prompt.astype(np.int32)).to(dev)
    for i in range(args.prompt):  # teacher-forced prefill through the decode path
        d_tok.copy_(d_prompt[i:i + 1])
        plan.step(dm.struct, kv.struct, d_tok, d_len, logits)
        d_len += 1
    plan.argmax(logits, d_tok)
    torch.cuda.synchronize()
    log("prefill of %d tokens in %.1fs" % (args.prompt, time.time() - t0))
    err = plan.device_error()
    if err:
        raise SystemExit("device error %d during prefill" % err)

    def run(n, plan, kv, d_tok, d_len, logits, events=None):
        # greedy decode: each launch also writes the next tokens and advances the lengths
        for i in range(n):
            if events is not None:
                events[i][0].record(st)
            plan.step_greedy(dm.struct, kv.struct, d_tok, d_len, logits)
            if events is not None:
                events[i][1].record(st)

    def ablation(Bn, capn, kv, d_tok, d_len, logits):
        """ms/step of the same step with JIT attention through the scheduler
        waves, and in kernel-per-operator mode (same results, bitwise)."""
        out = {"kv_len_start": int(d_len[0].item())}
        for name, o in (("jit_scheduler", dict(opts, jit=1)), ("kernel_per_op", dict(opts, mode=1))):
            pl = harness.build_plan(shape, Bn, capn, **o)
            run(4, pl, kv, d_tok, d_len, logits)
            torch.cuda.synchronize()
            e0.record(st)
            run(args.ablation_steps, pl, kv, d_tok, d_len, logits)
            e1.record(st)
            torch.cuda.synchronize()
            if pl.device_error():
                raise SystemExit("device error in the %s ablation" % name)
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
        plan16 = harness.build_plan(shape, B16, cap16, **opts)
        d_tok16 = torch.from_numpy(synth.tokens(wl16)).to(dev)
        d_len16 = torch.from_numpy(lens.astype(np.int32)).to(dev)
        logits16 = torch.empty((B16, shape.vocab), dtype=torch.float32, device=dev)
        run(args.warmup, plan16, kv16, d_tok16, d_len16, logits16)
        torch.cuda.synchronize()
        l16 = d_len16.cpu().numpy().copy()
        ev16 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.b16_steps)]
        e0.record(st)
        run(args.b16_steps, plan16, kv16, d_tok16, d_len16, logits16, ev16)
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
        }
        plan16.close()
        if not args.no_ablation:
            result["batch16"]["ablation"] = ablation(B16, cap16, kv16, d_tok16, d_len16, logits16)
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
        plan8 = harness.build_plan(shape, B8, cap8, paged=True, block=wl8.kv_block, max_blocks=table8.shape[1], **opts)
        d_tok8 = torch.from_numpy(synth.tokens(wl8)).to(dev)
        d_len8 = torch.from_numpy(lens8.astype(np.int32)).to(dev)
        logits8 = torch.empty((B8, shape.vocab), dtype=torch.float32, device=dev)
        run(args.warmup, plan8, kv8, d_tok8, d_len8, logits8)
        torch.cuda.synchronize()
        l8 = d_len8.cpu().numpy().copy()
        ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(st8)]
        e0.record(st)
        run(st8, plan8, kv8, d_tok8, d_len8, logits8, ev8)
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
        dmL = harness.DeviceModel(shL, synth.model_weights(shL), dev)
        kvL = harness.DeviceKV(shL, 1, capL)
        cL = synth.kv_sequence(shL, 0, int(lensL[0]), capL)
        kvL.load_sequence(0, cL["k"], cL["v"], int(lensL[0]))
        planL = harness.build_plan(shL, 1, capL, **opts)
        xs = [torch.from_numpy(synth.hidden_inputs(shL, 1, t)).to(dev) for t in range(args.warmup + stL)]
        xo = torch.empty((1, shL.hidden), dtype=torch.float32, device=dev)
        d_lenL = torch.from_numpy(lensL.astype(np.int32)).to(dev)
        for t in range(args.warmup):
            planL.step_hidden(dmL.struct, kvL.struct, xs[t], d_lenL, xo)
            d_lenL += 1
        torch.cuda.synchronize()
        l0 = int(d_lenL.item())
        evL = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(stL)]
        for t in range(stL):
            evL[t][0].record(st)
            planL.step_hidden(dmL.struct, kvL.struct, xs[args.warmup + t], d_lenL, xo)
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
            "note": "386 MB of weights per step; the 256 MB memory-side cache holds part of them between steps",
        }
        planL.close()

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
        }
        log("CPU oracle: %d steps in %.1fs (%.3f tok/s, %d threads)" % (n, dt, n / dt, oracle.get_threads()))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
