// Device loops of the persistent megakernel and the kernel entry points.
// Included by kernels.hip, which is compiled once per (weight type, batch
// tile) so the instantiations build in parallel.
#pragma once

#include "tasks.h"

namespace mk {
namespace {  // kernels get internal linkage: each instantiation unit registers its own

// ---------------------------------------------------------------- JIT ring

// Pop one ready attention task (FIFO). Only thread 0 of a worker calls it.
__device__ __forceinline__ bool jit_try_pop(const KParams& p, int& layer, int& bg, int& split) {
    const int64_t h = ld_relaxed64(&p.ctrl->jit_head);
    RingSlot* sl = &p.jit[h & p.jit_mask];
    if (ld_acquire64(&sl->tag) != h + 1) return false;
    const int p0 = sl->p0, p1 = sl->p1;
    int64_t expect = h;
    if (!__hip_atomic_compare_exchange_strong(&p.ctrl->jit_head, &expect, h + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT))
        return false;
    layer = p0 >> 16;
    bg = p0 & 0xFFFF;
    split = p1;
    return true;
}

// ---------------------------------------------------------------- scheduler waves

__device__ __forceinline__ void scheduler_wave(const KParams& p) {
    const int lane = threadIdx.x & 63;
    const int64_t want = (int64_t)p.L * (int64_t)(p.epoch + 1u);  // mailbox messages consumed by step end
    uint64_t t0 = now_ticks();
    for (;;) {
        int64_t h = 0;
        int layer = -1;
        int status = 0;  // 0 retry, 1 got message, 2 done, 3 abort
        if (lane == 0) {
            h = ld_relaxed64(&p.ctrl->mb_head);
            if (h >= want) status = 2;
            else if (aborted(p.ctrl)) status = 3;
            else {
                RingSlot* sl = &p.mb[h & p.mb_mask];
                if (ld_acquire64(&sl->tag) == h + 1) {
                    const int l = sl->p0;
                    int64_t e = h;
                    if (__hip_atomic_compare_exchange_strong(&p.ctrl->mb_head, &e, h + 1, __ATOMIC_RELAXED,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                        status = 1;
                        layer = l;
                    }
                } else if (now_ticks() - t0 > p.watchdog_ticks) {
                    raise_abort(p.ctrl);
                    status = 3;
                }
            }
        }
        status = __shfl(status, 0, 64);
        if (status == 2 || status == 3) return;
        if (status == 0) {
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        layer = __shfl(layer, 0, 64);
        t0 = now_ticks();
        // expand: tasks (b, g, s) for every sequence, in sequence order
        int total = 0;
        for (int b = 0; b < p.B; ++b) {
            const int pos = p.seq_lens[b];
            const bool ovf = pos < 0 || pos + 1 > p.cap;
            const int ns = ovf ? 1 : (pos + 1 + p.chunk - 1) / p.chunk;
            total += ns * p.Hkv;
        }
        int64_t base = 0;
        if (lane == 0)
            base = __hip_atomic_fetch_add(&p.ctrl->jit_tail, (int64_t)total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        base = __shfl(base, 0, 64);
        int off = 0;
        for (int b = 0; b < p.B; ++b) {
            const int pos = p.seq_lens[b];
            const bool ovf = pos < 0 || pos + 1 > p.cap;
            const int ns = ovf ? 1 : (pos + 1 + p.chunk - 1) / p.chunk;
            const int nb = ns * p.Hkv;
            for (int i = lane; i < nb; i += 64) {
                const int g = i / ns, sp = i % ns;
                const int64_t q = base + off + i;
                RingSlot* sl = &p.jit[q & p.jit_mask];
                sl->p0 = (layer << 16) | (b * p.Hkv + g);
                sl->p1 = sp;
                __hip_atomic_store(&sl->tag, q + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
            off += nb;
        }
    }
}

// ---------------------------------------------------------------- worker

template <typename WT, int NB>
__device__ __forceinline__ void worker_loop(const KParams& p, const Lds& s) {
    const int w = blockIdx.x;
    const int qb = p.qoff[w], qe = p.qoff[w + 1];
    const uint32_t ep1 = p.epoch + 1u;
    for (int qi = qb; qi < qe; ++qi) {
        const TaskRec t = p.tasks[p.queue[qi]];
        if (t.wait_ev >= 0) {
            const uint32_t target = p.evrec[t.wait_ev].required * ep1;
            uint64_t t0 = now_ticks();
            for (;;) {
                if (threadIdx.x == 0) {
                    int cmd = 2;
                    const uint32_t c = ld_relaxed(&p.ev[t.wait_ev]);
                    if ((int32_t)(c - target) >= 0) cmd = 0;
                    else if (aborted(p.ctrl)) cmd = 3;
                    else {
                        int jl, jbg, js;
                        if (p.jit_on && jit_try_pop(p, jl, jbg, js)) {
                            cmd = 1;
                            s.cmd[1] = jl;
                            s.cmd[2] = jbg;
                            s.cmd[3] = js;
                        } else if (now_ticks() - t0 > p.watchdog_ticks) {
                            raise_abort(p.ctrl);
                            cmd = 3;
                        }
                    }
                    s.cmd[0] = cmd;
                }
                __syncthreads();
                const int cmd = s.cmd[0];
                const int jl = s.cmd[1], jbg = s.cmd[2], js = s.cmd[3];
                __syncthreads();
                if (cmd == 0) break;
                if (cmd == 3) return;
                if (cmd == 1) {
                    fence_acquire();
                    attention_task<WT>(p, jl, jbg, js, s);
                    t0 = now_ticks();
                } else {
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            fence_acquire();
        }
        if (t.op == OP_ATTN) {
            attention_task<WT>(p, t.layer, t.a0, t.a1, s);
            continue;
        }
        run_gemv_task<WT, NB>(p, t, s);
        signal_event(p, t.sig_ev, s);
    }
}

extern __shared__ float mk_dyn_lds[];

template <typename WT, int NB>
__global__ __launch_bounds__(kThreads) void k_persistent(KParams p) {
    const Lds s = carve_lds(mk_dyn_lds, p.Hq / p.Hkv, p.chunk);
    if ((int)blockIdx.x >= p.n_workers) {
        if (p.jit_on) scheduler_wave(p);
        return;
    }
    worker_loop<WT, NB>(p, s);
}

template <typename WT, int NB>
__global__ __launch_bounds__(kThreads) void k_level_gemv(KParams p, const int32_t* ids) {
    const Lds s = carve_lds(mk_dyn_lds, p.Hq / p.Hkv, p.chunk);
    const TaskRec t = p.tasks[ids[blockIdx.x]];
    run_gemv_task<WT, NB>(p, t, s);
}

template <typename WT>
__global__ __launch_bounds__(kThreads) void k_level_attn(KParams p, int layer) {
    const Lds s = carve_lds(mk_dyn_lds, p.Hq / p.Hkv, p.chunk);
    const int bg = blockIdx.x / p.max_splits, sp = blockIdx.x % p.max_splits;
    attention_task<WT>(p, layer, bg, sp, s);
}

}  // namespace
}  // namespace mk

