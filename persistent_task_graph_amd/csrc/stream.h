// Paged-LDS weight streaming for batch-1 GEMV tasks (persistent mode).
//
// The MPK article (devpress.csdn.net, §3.1 "分页共享内存管理" and §3.2
// "任务预取与流水线") splits on-chip memory into pages that a task's
// preload phase fills while earlier tasks compute. Here every wave of a
// worker owns a ring of NS one-kilobyte pages in LDS. Because weights are
// static, the wave's whole sequence of weight pages over its queue of GEMV
// tasks is known from the plan: the wave keeps NS page loads in flight at
// all times, so the next task's leading pages are requested while the
// current task finishes, while the worker waits for the next task's event,
// and while it runs attention tasks.
//
// A page holds 64 lanes x 16 bytes of one weight row: segment (wave + 4j)
// of row r of matrix m, the same K split the register GEMV uses. Pages go
// straight from memory to LDS (buffer_load ... lds), issued from inline
// assembly so that the compiler does not serialise LDS reads behind them;
// the consumer waits with vmcnt(NS-1): loads complete in issue order, so
// when NS-1 page loads issued after page c are still allowed in flight,
// page c (and any older memory operation) has completed.
#pragma once

#include "tasks.h"

namespace mk {

constexpr int kRingPages = 16;  // pages per wave (16 KB); 64 KB per worker (power of two)
typedef int i32x4 __attribute__((ext_vector_type(4)));

// One streamed task as seen by a wave: rows [r0, r1) of up to three
// matrices (QKV: q|k|v rows, gate/up: both matrices per row, else one).
struct StreamTask {
    const char *m0, *m1, *m2;
    int op, r0, r1, K, nm, rows0, rows1;  // rows0/rows1: q rows and q+k rows (QKV)
};

__device__ __forceinline__ bool is_streamed(int op) {
    return op == OP_QKV || op == OP_O || op == OP_GATEUP || op == OP_DOWN || op == OP_LM;
}

template <typename WT>
__device__ __forceinline__ StreamTask stream_task(const KParams& p, const TaskRec& t) {
    StreamTask s;
    s.op = t.op;
    s.r0 = t.a0;
    s.r1 = t.a1;
    s.rows0 = s.rows1 = 1 << 30;
    s.nm = 1;
    s.m0 = s.m1 = s.m2 = nullptr;
    switch (t.op) {
        case OP_QKV: {
            const LayerPtrs& w = p.lw[t.layer];
            s.m0 = (const char*)w.wq;
            s.m1 = (const char*)w.wk;
            s.m2 = (const char*)w.wv;
            s.K = p.H;
            s.rows0 = p.QD;
            s.rows1 = p.QD + p.KD;
            break;
        }
        case OP_O: s.m0 = (const char*)p.lw[t.layer].wo; s.K = p.QD; break;
        case OP_GATEUP:
            s.m0 = (const char*)p.lw[t.layer].w_gate;
            s.m1 = (const char*)p.lw[t.layer].w_up;
            s.K = p.H;
            s.nm = 2;
            break;
        case OP_DOWN: s.m0 = (const char*)p.lw[t.layer].w_down; s.K = p.F; break;
        default: s.m0 = (const char*)p.lm_head; s.K = p.H; break;  // OP_LM
    }
    return s;
}

// base address of row r of matrix m of a streamed task
template <typename WT>
__device__ __forceinline__ const char* stream_row(const StreamTask& s, int r, int m) {
    const int64_t rb = (int64_t)s.K * (int64_t)sizeof(WT);
    if (s.nm == 2) return (m == 0 ? s.m0 : s.m1) + (int64_t)r * rb;
    if (r < s.rows0) return s.m0 + (int64_t)r * rb;
    if (r < s.rows1) return s.m1 + (int64_t)(r - s.rows0) * rb;
    return s.m2 + (int64_t)(r - s.rows1) * rb;
}

// Per-wave stream state. The loader walks (task, row, matrix, segment) ahead
// of the consumer by up to kRingPages pages.
struct Stream {
    // loader cursor
    int lq, lr, lm, lj, lnsw;
    StreamTask lt;
    bool ldone;
    // page counters
    int issued, consumed;
    uint32_t ring_lds;  // LDS byte address of this wave's ring
};

template <typename WT>
__device__ __forceinline__ int wave_segments(int K, int wave) {
    constexpr int SEG = 64 * Vec16<WT>::N;
    const int nseg = (K + SEG - 1) / SEG;
    return nseg > wave ? (nseg - wave + kWaves - 1) / kWaves : 0;
}

// advance the loader to the next streamed task at or after queue index q
template <typename WT>
__device__ __forceinline__ void loader_seek(const KParams& p, Stream& st, int q, int qe, int wave) {
    for (; q < qe; ++q) {
        const TaskRec t = p.tasks[p.queue[q]];
        if (!is_streamed(t.op)) continue;
        st.lt = stream_task<WT>(p, t);
        st.lnsw = wave_segments<WT>(st.lt.K, wave);
        if (st.lnsw == 0 || st.lt.r1 <= st.lt.r0) continue;
        st.lq = q;
        st.lr = st.lt.r0;
        st.lm = 0;
        st.lj = 0;
        return;
    }
    st.ldone = true;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most n memory operations issued by this wave are in flight
__device__ __forceinline__ void wait_vm_dyn(int n) {
    switch (n <= 0 ? 0 : (n > kRingPages ? kRingPages : n)) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<1>(); break;
        case 2: wait_vm<2>(); break;
        case 3: wait_vm<3>(); break;
        case 4: wait_vm<4>(); break;
        case 5: wait_vm<5>(); break;
        case 6: wait_vm<6>(); break;
        case 7: wait_vm<7>(); break;
        case 8: wait_vm<8>(); break;
        case 9: wait_vm<9>(); break;
        case 10: wait_vm<10>(); break;
        case 11: wait_vm<11>(); break;
        case 12: wait_vm<12>(); break;
        case 13: wait_vm<13>(); break;
        case 14: wait_vm<14>(); break;
        case 15: wait_vm<15>(); break;
        default: wait_vm<16>(); break;
    }
}

// pages per row for the loader's current task
__device__ __forceinline__ int loader_row_pages(const Stream& st) { return st.lt.nm * st.lnsw; }

// Issue whole rows while the ring has room (loads complete in order, so a
// row's pages are consumed only after the pages before them).
template <typename WT>
__device__ __forceinline__ void loader_fill(const KParams& p, Stream& st, int consumed, int qe, int wave, int lane) {
    constexpr int SEG = 64 * Vec16<WT>::N;
    while (!st.ldone && st.issued + loader_row_pages(st) <= consumed + kRingPages) {
        const uint32_t rowbytes = (uint32_t)st.lt.K * (uint32_t)sizeof(WT);
        for (int m = 0; m < st.lt.nm; ++m) {
            const uint64_t a = (uint64_t)(uintptr_t)stream_row<WT>(st.lt, st.lr, m);
            i32x4 rs;
            rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
            rs.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
            rs.z = __builtin_amdgcn_readfirstlane((int)rowbytes);
            rs.w = 0x00020000;
            for (int j = 0; j < st.lnsw; ++j) {
                const uint32_t k = (uint32_t)((wave + kWaves * j) * SEG + lane * Vec16<WT>::N);
                const uint32_t voff = k < (uint32_t)st.lt.K ? k * (uint32_t)sizeof(WT) : kOOB;
                const uint32_t lds =
                    __builtin_amdgcn_readfirstlane(st.ring_lds + (uint32_t)(st.issued & (kRingPages - 1)) * 1024u);
                asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rs)
                             : "memory", "m0");
                st.issued++;
            }
        }
        if (++st.lr == st.lt.r1) loader_seek<WT>(p, st, st.lq + 1, qe, wave);
    }
}

// Streamed GEMV task (batch 1): same arithmetic as gemv_ksplit with NB = 1,
// weights taken from the wave's page ring in stream order.
template <typename WT, int NSW, bool DUAL, typename OutFn>
__device__ __forceinline__ void gemv_stream(const KParams& p, Stream& st, const uint4* ring, int qe, int r0, int r1,
                                            int K, const float* x, const WT* gain, float eps, OutFn out, const Lds& s,
                                            bool tr) {
    using V = Vec16<WT>;
    constexpr int E = V::N, SEG = 64 * E;
    constexpr int NM = DUAL ? 2 : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nsw = wave_segments<WT>(K, wave);
    // x (agent-coherent) and the norm gain for this wave's segments
    const __amdgpu_buffer_rsrc_t xr_rs = make_rsrc(x, (uint32_t)K * 4u);
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(gain, gain ? (uint32_t)K * (uint32_t)sizeof(WT) : 0u);
    float xr[NSW][E];
    float g[NSW][E];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const int k = (wave + kWaves * j) * SEG + lane * E;
        const bool kv = j < nsw && k < K;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const uint4 v = buf_load16_act(xr_rs, kv ? (uint32_t)(k + e) * 4u : kOOB, 0);
            xr[j][e + 0] = __uint_as_float(v.x);
            xr[j][e + 1] = __uint_as_float(v.y);
            xr[j][e + 2] = __uint_as_float(v.z);
            xr[j][e + 3] = __uint_as_float(v.w);
        }
        if (gain) V::widen(buf_load16(g_rs, kv ? (uint32_t)k * (uint32_t)sizeof(WT) : kOOB, 0), g[j]);
        else
#pragma unroll
            for (int e = 0; e < E; ++e) g[j][e] = 1.f;
    }
    if (gain) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NSW; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) ss += xr[j][e] * xr[j][e];
        ss = wave_sum(ss);
        if (lane == 0) s.red[wave * 16] = ss;
        __syncthreads();
        if (tid == 0) {
            float t = s.red[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) t += s.red[w * 16];
            s.rstd[0] = 1.0f / sqrtf(t / (float)K + eps);
        }
    }
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) xr[j][e] = xr[j][e] * g[j][e];
    if (tr && tid == 0) s.marks[0] = now_ticks();

    constexpr int WIN = kPartFloats / (kWaves * NM);
    for (int rg = r0; rg < r1; rg += WIN) {
        const int rend = min(rg + WIN, r1);
        // rows in batches of R (about eight pages) so that the reductions of a
        // batch overlap; every page of a batch is read before any is used
        constexpr int R = (8 / (NM * NSW)) > 0 ? 8 / (NM * NSW) : 1;
        for (int r = rg; r < rend; r += R) {
            const int nr = min(R, rend - r);
            const int G = nr * NM * nsw;
            wait_vm_dyn(st.issued - st.consumed - G);
            uint4 w[R][NM][NSW];
#pragma unroll
            for (int u = 0; u < R; ++u)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int j = 0; j < NSW; ++j)
                        if (u < nr && j < nsw)
                            w[u][m][j] = ring[((st.consumed + (u * NM + m) * nsw + j) & (kRingPages - 1)) * 64 + lane];
            st.consumed += G;
            // the freed slots are refilled only after their reads returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            loader_fill<WT>(p, st, st.consumed, qe, wave, lane);
            float acc[R][NM];
#pragma unroll
            for (int u = 0; u < R; ++u)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    acc[u][m] = 0.f;
#pragma unroll
                    for (int j = 0; j < NSW; ++j) {
                        if (j >= nsw) continue;
                        float wf[E];
                        V::widen(w[u][m][j], wf);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[u][m] = fmaf(wf[e], xr[j][e], acc[u][m]);
                    }
                }
#pragma unroll
            for (int u = 0; u < R; ++u)
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[u][m] = wave_sum(acc[u][m]);
            if (lane == 0) {
#pragma unroll
                for (int u = 0; u < R; ++u)
                    if (u < nr)
#pragma unroll
                        for (int m = 0; m < NM; ++m) s.part[((wave * WIN) + (r + u - rg)) * NM + m] = acc[u][m];
            }
        }
        if (tr && tid == 0) s.marks[1] = now_ticks();
        __syncthreads();
        for (int i = tid; i < rend - rg; i += kThreads) {
            float t[2] = {0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float a = s.part[i * NM + m];
#pragma unroll
                for (int wv = 1; wv < kWaves; ++wv) a += s.part[((wv * WIN) + i) * NM + m];
                t[m] = a;
            }
            out(rg + i, 0, t[0], t[1]);
        }
        __syncthreads();
    }
}

template <typename WT, bool DUAL, typename OutFn>
__device__ __forceinline__ void gemv_stream_dispatch(const KParams& p, Stream& st, const uint4* ring, int qe, int r0,
                                                     int r1, int K, const float* x, const WT* gain, OutFn out,
                                                     const Lds& s) {
    constexpr int SEG = 64 * Vec16<WT>::N;
    const int nsw = ((K + SEG - 1) / SEG + kWaves - 1) / kWaves;
    const bool tr = p.trace != nullptr;
    if (nsw <= 1) gemv_stream<WT, 1, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
    else if (nsw <= 2) gemv_stream<WT, 2, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
    else if (nsw <= 3) gemv_stream<WT, 3, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
    else if (nsw <= 4) gemv_stream<WT, 4, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
    else if (nsw <= 6) gemv_stream<WT, 6, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
    else gemv_stream<WT, 8, DUAL>(p, st, ring, qe, r0, r1, K, x, gain, p.eps, out, s, tr);
}

// The batch-1 GEMV task bodies on the page stream (epilogues as in
// run_gemv_task).
template <typename WT>
__device__ __forceinline__ void run_stream_task(const KParams& p, Stream& st, const uint4* ring, int qe,
                                                const TaskRec& t, const Lds& s) {
    const int l = t.layer, H = p.H, r0 = t.a0, r1 = t.a1;
    switch (t.op) {
        case OP_QKV: {
            const LayerPtrs w = p.lw[l];
            const int ld = p.QD + 2 * p.KD;
            float* o = layer_buf(p, l, p.off_qkv);
            (void)ld;
            auto out = [&](int r, int, float v, float) { st_co(&o[r], v * s.rstd[0]); };
            gemv_stream_dispatch<WT, false>(p, st, ring, qe, r0, r1, H, layer_in(p, l), (const WT*)w.attn_norm, out, s);
            break;
        }
        case OP_O: {
            const float* xin = layer_in(p, l);
            float* o = layer_buf(p, l, p.off_xmid);
            auto out = [&](int r, int, float v, float) { st_co(&o[r], ld_act(&xin[r]) + v); };
            gemv_stream_dispatch<WT, false>(p, st, ring, qe, r0, r1, p.QD, layer_buf(p, l, p.off_attn), (const WT*)nullptr,
                                            out, s);
            break;
        }
        case OP_GATEUP: {
            const LayerPtrs w = p.lw[l];
            float* o = layer_buf(p, l, p.off_h);
            auto out = [&](int r, int, float gv, float uv) {
                const float rs = s.rstd[0];
                const float gg = gv * rs, uu = uv * rs;
                st_co(&o[r], (gg / (1.0f + __expf(-gg))) * uu);
            };
            gemv_stream_dispatch<WT, true>(p, st, ring, qe, r0, r1, H, layer_buf(p, l, p.off_xmid), (const WT*)w.mlp_norm,
                                           out, s);
            break;
        }
        case OP_DOWN: {
            const float* xm = layer_buf(p, l, p.off_xmid);
            float* o = layer_out(p, l);
            auto out = [&](int r, int, float v, float) { st_co(&o[r], ld_act(&xm[r]) + v); };
            gemv_stream_dispatch<WT, false>(p, st, ring, qe, r0, r1, p.F, layer_buf(p, l, p.off_h), (const WT*)nullptr,
                                            out, s);
            break;
        }
        case OP_LM: {
            float* o = p.logits;
            auto out = [&](int r, int, float v, float) { o[r] = v * s.rstd[0]; };
            gemv_stream_dispatch<WT, false>(p, st, ring, qe, r0, r1, H, p.x_final, (const WT*)p.final_norm, out, s);
            if (p.greedy_tokens) lm_greedy(p, r0, r1);
            break;
        }
        default: break;
    }
}

}  // namespace mk
