// Device loops of the persistent megakernel and the kernel entry points.
// Included by kernels.hip, which is compiled once per (weight type, batch
// tile) so the instantiations build in parallel.
#pragma once

#include "stream.h"

namespace mk {
#ifdef MK_LDS_STREAM
constexpr bool kLdsStream = true;
#else
constexpr bool kLdsStream = false;
#endif
}  // namespace mk

namespace mk {
namespace {  // kernels get internal linkage: each instantiation unit registers its own

// ---------------------------------------------------------------- JIT inbox

// Pop the next attention task dealt to this worker (single consumer: only
// thread 0 of the owning workgroup reads its inbox; `head` lives in a
// register and is written back when the workgroup exits).
__device__ __forceinline__ const RingSlot* inbox_slot(const KParams& p, int64_t head) {
    return &p.inbox[(int64_t)blockIdx.x * (p.inbox_mask + 1) + (head & p.inbox_mask)];
}
// `tag` is the slot's tag, loaded by the caller together with its other
// polling loads
__device__ __forceinline__ bool inbox_try_pop(const KParams& p, int64_t tag, int64_t& head, int& layer, int& bg,
                                              int& split) {
    const RingSlot* sl = inbox_slot(p, head);
    if (tag != head + 1) return false;
    const int p0 = ld_co(&sl->p0), p1 = ld_co(&sl->p1);
    head++;
    layer = p0 >> 16;
    bg = p0 & 0xFFFF;
    split = p1;
    return true;
}

// ---------------------------------------------------------------- scheduler waves

__device__ __forceinline__ void scheduler_wave(const KParams& p) {
    const int lane = threadIdx.x & 63;
    const int64_t want = (int64_t)p.L * (int64_t)(p.epoch + 1u);  // mailbox messages consumed by step end
    const int chunk = attn_chunk(p);
    uint64_t t0 = now_ticks();
    for (;;) {
        int64_t h = 0;
        int layer = -1;
        int status = 0;  // 0 retry, 1 got message, 2 done, 3 abort
        if (lane == 0) {
            h = ld_relaxed64(&p.ctrl->mb_head);
            const bool ab = aborted(p.ctrl);  // loaded together with the head
            if (h >= want) status = 2;
            else if (ab) status = 3;
            else {
                RingSlot* sl = &p.mb[h & p.mb_mask];
                if (ld_relaxed64(&sl->tag) == h + 1) {
                    const int l = ld_co(&sl->p0);
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
            const int ns = ovf ? 1 : (pos + 1 + chunk - 1) / chunk;
            total += ns * p.Hkv;
        }
        // deal the tasks round-robin to the eligible workers' inboxes,
        // continuing where the previous expansion stopped
        int64_t start = 0;
        if (lane == 0)
            start = __hip_atomic_fetch_add(&p.ctrl->rr, (int64_t)total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        start = __shfl(start, 0, 64);
        for (int i = lane; i < total; i += 64) {
            int b = 0, off = 0, ns = 1;
            for (;; ++b) {
                const int pos = p.seq_lens[b];
                const bool ovf = pos < 0 || pos + 1 > p.cap;
                ns = ovf ? 1 : (pos + 1 + chunk - 1) / chunk;
                if (i < off + ns * p.Hkv || b == p.B - 1) break;
                off += ns * p.Hkv;
            }
            const int local = i - off, g = local / ns, sp = local % ns;
            const int w = p.elig[(start + i) % p.n_elig];
            const int64_t q = __hip_atomic_fetch_add(&p.inbox_tail[w], (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            RingSlot* sl = &p.inbox[(int64_t)w * (p.inbox_mask + 1) + (q & p.inbox_mask)];
            st_co(&sl->p0, (layer << 16) | (b * p.Hkv + g));
            st_co(&sl->p1, sp);
            wait_stores();
            __hip_atomic_store(&sl->tag, q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- worker

// task trace (thread 0 only)
__device__ __forceinline__ void trace_put(const KParams& p, const Lds& s, int kind, int id, int op, uint64_t tw,
                                          uint64_t tr) {
    if (!p.trace || threadIdx.x != 0) return;
    const int w = blockIdx.x;
    const int i = p.trace_n[w];
    if (i < p.trace_cap) {
        mk_trace_rec r;
        r.kind = kind;
        r.id = id;
        r.worker = w;
        r.op = op;
        r.t_wait = tw;
        r.t_ready = tr;
        r.t_done = now_ticks();
        r.t_a = s.marks[0];
        r.t_b = s.marks[1];
        r.t_c = s.marks[2];
        r.t_d = s.marks[3];
        p.trace[(int64_t)w * p.trace_cap + i] = r;
    }
    p.trace_n[w] = i + 1;
    s.marks[0] = s.marks[1] = s.marks[2] = s.marks[3] = 0;
}

template <typename WT, int NB>
__device__ __forceinline__ void worker_loop(const KParams& p, const Lds& s, uint4* ring_mem) {
    const int w = blockIdx.x;
    const int qb = p.qoff[w], qe = p.qoff[w + 1];
    constexpr int NP = ev_planes(NB);  // event-count planes this instance uses
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (p.trace && threadIdx.x == 0) {
        p.trace_n[w] = 0;
        s.marks[0] = s.marks[1] = s.marks[2] = s.marks[3] = 0;
    }
    int64_t head = (threadIdx.x == 0 && p.jit_on) ? p.inbox_head[w] : 0;
    // optional batch-1 variant: weight pages stream through a per-wave LDS
    // ring fed by direct-to-LDS loads (stream.h) instead of registers
    constexpr bool kStream = kLdsStream && NB == 1;
    Stream st;
    const uint4* ring = ring_mem + wave * kRingPages * 64;
    if constexpr (kStream) {
        st.issued = st.consumed = 0;
        st.ldone = false;
        st.ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)ring;
        loader_seek<WT>(p, st, qb, qe, wave);
        loader_fill<WT>(p, st, 0, qe, wave, lane);
    }
    // Several greedy decode steps may run in one launch (the MPK article,
    // §2.1: the whole computation in one kernel): step s waits on events at
    // epoch + s and starts once step s - 1 has written its tokens and lengths.
    for (int step = 0; step < p.n_steps; ++step) {
    const uint32_t ep1 = p.epoch + (uint32_t)step + 1u;
    int chunk = 0;  // the step's attention chunk, found before the first attention task
    Prefetch pf;
    pf.next = pf.end = 0;
    pf.chunk_kb = 0;
    if constexpr (!kStream)
        if (qb < qe) pf = prefetch_setup<WT>(p, p.tasks[p.queue[qb]]);
    Prefetch pf_next;
    pf_next.next = pf_next.end = 0;
    pf_next.chunk_kb = 0;
    for (int qi = qb; qi < qe; ++qi) {
        const int tid_task = p.queue[qi];
        const TaskRec t = p.tasks[tid_task];
        // the layer's weight pointers are read now, not after the event fires
        const LayerPtrs lwt = p.lw[t.layer];
        // the next task's weight cursor is looked up now, off the critical
        // path (its table reads complete while this task waits and runs)
        if constexpr (!kStream)
            if (qi + 1 < qe) pf_next = prefetch_setup<WT>(p, p.tasks[p.queue[qi + 1]]);
        const uint64_t tw = p.trace ? now_ticks() : 0;
        uint64_t tr = tw;
        // Wait for the task's event, running JIT attention tasks from this
        // worker's inbox meanwhile. An AOT attention task runs through the
        // same call once its event has fired, so the (large) attention body
        // is expanded at one site only.
        bool waiting = t.wait_ev >= 0, aot_attn = t.op == OP_ATTN;
        // an AOT attention slot runs split task t.a0 of the step, found from
        // seq_lens before it waits and handed to the run below through LDS
        // (past the poll loop's barriers); bg = -1 marks a slot the step
        // leaves empty
        if (aot_attn) {
            if (chunk == 0) chunk = attn_chunk(p);
            int abg = t.a0, asp = t.a1;  // a static-schedule task carries its split
            if (!(t.flags & kTaskStaticAttn) && !attn_locate(p, chunk, t.a0, abg, asp)) abg = -1;
            else if constexpr (!kStream) pf = attn_prefetch_setup<WT>(p, t.layer, abg, asp, chunk);
            if (threadIdx.x == 0) {
                s.cmd[12] = abg;
                s.cmd[13] = asp;
            }
        }
        // a GEMV task's first rows go to the LDS preload slots while it waits
        if constexpr (!kStream && NB <= 2)
            if (p.pre_slots > 0) {
                preload_setup<WT>(p, t, s);
                preload_step<WT>(s);
            }
        const uint32_t target = waiting ? p.evrec[t.wait_ev].required * ep1 : 0u;
        uint64_t t0 = now_ticks();
        for (;;) {
            int cmd = 0, jl = t.layer, jbg = t.a0, js = t.a1;
            if (waiting) {
                if (threadIdx.x == 0) {
                    int c = 2;
                    // the count planes, the abort flag and the inbox tag are
                    // loaded together: one memory round trip per poll, not
                    // one per check (the abort flag had been read only after
                    // the count came back, doubling the time to see an event)
                    uint32_t v = 0;
#pragma unroll
                    for (int j = 0; j < NP; ++j) v += ld_relaxed(&p.ev[j * p.ev_stride + t.wait_ev]);
                    const bool ab = aborted(p.ctrl);
                    const int64_t tag = p.jit_on ? ld_relaxed64(&inbox_slot(p, head)->tag) : 0;
                    if ((int32_t)(v - target) >= 0) c = 0;
                    else if (ab) c = 3;
                    else {
                        int a, bb, cc;
                        if (p.jit_on && inbox_try_pop(p, tag, head, a, bb, cc)) {
                            c = 1;
                            s.cmd[1] = a;
                            s.cmd[2] = bb;
                            s.cmd[3] = cc;
                        } else if (now_ticks() - t0 > p.watchdog_ticks) {
                            raise_abort(p.ctrl);
                            c = 3;
                        }
                    }
                    s.cmd[0] = c;
                }
                __syncthreads();
                cmd = s.cmd[0];
                if (cmd == 1) {
                    jl = s.cmd[1];
                    jbg = s.cmd[2];
                    js = s.cmd[3];
                }
                __syncthreads();
                if (cmd == 3) {
                    if (threadIdx.x == 0 && p.jit_on) p.inbox_head[w] = head;
                    if constexpr (kStream) wait_vm<0>();
                    return;
                }
                if (cmd == 2) {
                    if constexpr (!kStream) {
                        if constexpr (NB <= 2)
                            if (p.pre_slots > 0) preload_step<WT>(s);
                        prefetch_step(pf);
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                if (cmd == 0) {
                    waiting = false;
                    if (p.trace) tr = now_ticks();
                }
            }
            if (cmd == 0) {
                if (!aot_attn) break;
                aot_attn = false;
                jbg = s.cmd[12];
                js = s.cmd[13];
                if (jbg < 0) break;
            }
            const uint64_t tj = p.trace ? now_ticks() : 0;
            if (chunk == 0) chunk = attn_chunk(p);
            attention_task<WT>(p, jl, jbg, js, chunk, s, (int)blockIdx.x & (NP - 1));
            if (cmd == 0) break;  // that was this AOT attention task
            trace_put(p, s, 1, (jl << 24) | ((jbg & 0xFFF) << 12) | (js & 0xFFF), OP_ATTN, tj, tj);
            t0 = now_ticks();
        }
        if (t.op != OP_ATTN) {
            bool gemv_sig = true;  // false: a K-split part that did not merge its group
            if constexpr (kStream) {
                if (is_streamed(t.op)) run_stream_task<WT>(p, st, ring, qe, t, s);
                else if (t.op == OP_EMBED) embed_task<WT>(p, t);
            } else {
                gemv_sig = run_gemv_task<WT, NB>(p, t, s, lwt, (NB <= 2 && p.pre_slots > 0) ? preload_done_rows(s) : 0);
            }
            // JIT expanded by the completing QKV arrival: batch >= 8
            // instances only (the expansion code in the batch <= 4 loops
            // costs those steps 1-3% even when it never runs)
            bool signalled = !gemv_sig;
            if constexpr (NB >= 8)
                if (p.jit_on == 2 && !signalled) {
                    signal_gemv_jit_inline(p, t.sig_ev, s, (int)blockIdx.x & (NP - 1));
                    signalled = true;
                }
            if (!signalled) signal_event(p, t.sig_ev, s, (int)blockIdx.x & (NP - 1));
        }
        if constexpr (!kStream) {
            if (qi + 1 < qe) {
                pf = pf_next;
                prefetch_step(pf);
            }
        }
        trace_put(p, s, 0, tid_task, t.op, tw, tr);
    }
    if (p.greedy_tokens) {
        // greedy step: the last worker to leave its queue writes the next
        // tokens and advances the lengths (no worker reads them any more in
        // this step), then releases the step
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(p.exit_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1u == (uint32_t)p.n_workers) {
                greedy_finish(p, step);
                __hip_atomic_store(p.exit_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                wait_stores();
                __hip_atomic_store(&p.ctrl->step_done, ep1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (step + 1 < p.n_steps) {
            // step barrier: wait for the release, then drop cached lines of
            // this launch's earlier steps (activations, tokens, lengths) as
            // the kernel entry does for earlier launches
            if (threadIdx.x == 0) {
                const uint64_t tb = now_ticks();
                int c = 0;
                for (;;) {
                    const uint32_t done = ld_relaxed(&p.ctrl->step_done);
                    const bool ab = aborted(p.ctrl);  // loaded together with the step word
                    if ((int32_t)(done - ep1) >= 0) break;
                    if (ab) { c = 1; break; }
                    if (now_ticks() - tb > p.watchdog_ticks) { raise_abort(p.ctrl); c = 1; break; }
                    __builtin_amdgcn_s_sleep(1);
                }
                s.cmd[0] = c;
            }
            __syncthreads();
            const int c = s.cmd[0];
            __syncthreads();
            if (c) break;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    }  // step
    if (threadIdx.x == 0 && p.jit_on) p.inbox_head[w] = head;
    if constexpr (kStream) wait_vm<0>();
}

extern __shared__ __attribute__((aligned(16))) float mk_dyn_lds[];

template <typename WT, int NB>
__global__ __launch_bounds__(kThreads) void k_persistent(KParams p) {
    const Lds s = carve_lds(mk_dyn_lds);
    // drop L2 lines cached in earlier steps: activations are then read with
    // plain loads (see buf_load16_act)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if ((int)blockIdx.x >= p.n_workers) {
        // four scheduler waves per scheduler workgroup
        if (p.jit_on && (threadIdx.x >> 6) < 4) scheduler_wave(p);
        return;
    }
    if constexpr (kLdsStream && NB == 1) {
        __shared__ __attribute__((aligned(1024))) uint4 ring_mem[kWaves * kRingPages * 64];
        worker_loop<WT, NB>(p, s, ring_mem);
    } else {
        worker_loop<WT, NB>(p, s, nullptr);
    }
}

template <typename WT, int NB>
// Kernel-per-operator launches: the previous level's outputs are visible
// through the launch's own acquire (the same guarantee ordinary stream-ordered
// kernels rely on), so activations are read with plain loads here too.
__global__ __launch_bounds__(kThreads) void k_level_gemv(KParams p, const int32_t* ids) {
    const Lds s = carve_lds(mk_dyn_lds);
    const TaskRec t = p.tasks[ids[blockIdx.x]];
    const LayerPtrs lwt = p.lw[t.layer];
    run_gemv_task<WT, NB>(p, t, s, lwt);
}

template <typename WT>
__global__ __launch_bounds__(kThreads) void k_level_attn(KParams p, int layer) {
    const Lds s = carve_lds(mk_dyn_lds);
    const int bg = blockIdx.x / p.max_splits, sp = blockIdx.x % p.max_splits;
    attention_task<WT>(p, layer, bg, sp, attn_chunk(p), s);
}

}  // namespace
}  // namespace mk

