// Task bodies. The same __device__ functions run inside the persistent
// megakernel and inside the kernel-per-operator launches, so the two modes
// produce identical bits: every reduction below has a fixed order that
// depends only on the shape (never on which workgroup, task or schedule
// runs it), no floating-point atomics are used, and contraction is off.
#pragma once

#include "device.h"

namespace mk {

// ---------------------------------------------------------------- LDS layout
// Carved from one dynamic shared buffer; sizes in floats.
struct Lds {
    float* red;   // 64: reductions / broadcast
    int* cmd;     // 16 ints
    float* rstd;  // 16
    float* part;  // kWaves * 256 * 4: GEMV cross-wave partial sums (2 matrices x 2 rows)
    float* q;     // 8 * 128: rotated query heads of one KV group
    float* kn;    // 2 * 128: new k, v (rounded to the cache type)
    float* p;     // G * chunk: scores, then probabilities
    float* acc;   // kWaves * 8 * 128: P.V partials per wave
    float* ml;    // 2 * 8: (m, l) per head
};

__host__ __device__ constexpr int lds_floats_fixed() { return 64 + 16 + 16 + kWaves * 256 * 4 + 8 * 128 + 2 * 128 + kWaves * 8 * 128 + 16; }
__host__ __device__ inline int lds_bytes_for(int G, int chunk) { return 4 * (lds_floats_fixed() + G * chunk); }

__device__ __forceinline__ Lds carve_lds(float* base, int G, int chunk) {
    Lds s;
    float* p = base;
    s.red = p; p += 64;
    s.cmd = (int*)p; p += 16;
    s.rstd = p; p += 16;
    s.part = p; p += kWaves * 256 * 4;
    s.q = p; p += 8 * 128;
    s.kn = p; p += 2 * 128;
    s.acc = p; p += kWaves * 8 * 128;
    s.ml = p; p += 16;
    s.p = p;
    (void)G; (void)chunk;
    return s;
}

// ---------------------------------------------------------------- activations

__device__ __forceinline__ float* layer_buf(const KParams& p, int l, int64_t off) { return p.act + l * p.act_stride + off; }
__device__ __forceinline__ const float* layer_in(const KParams& p, int l) {
    return l == 0 ? p.x0 : (l == p.L ? p.x_final : layer_buf(p, l - 1, p.off_xnext));
}
__device__ __forceinline__ float* layer_out(const KParams& p, int l) {
    return l == p.L - 1 ? p.x_final : layer_buf(p, l, p.off_xnext);
}

// rstd[b] = 1 / sqrt(mean_k x[b,k]^2 + eps) for b < B, into s.rstd (all
// threads see it after return). Fixed per-thread strides, fixed tree.
template <int NB>
__device__ __forceinline__ void block_rstd(const float* x, int ldx, int K, int B, float eps, const Lds& s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float ss[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        ss[b] = 0.f;
        if (b < B)
            for (int k = tid * 4; k < K; k += kThreads * 4) {
                const float4 v = *(const float4*)(x + (int64_t)b * ldx + k);
                ss[b] += v.x * v.x;
                ss[b] += v.y * v.y;
                ss[b] += v.z * v.z;
                ss[b] += v.w * v.w;
            }
        ss[b] = wave_sum(ss[b]);
    }
    if (lane == 0)
#pragma unroll
        for (int b = 0; b < NB; ++b) s.red[wave * 16 + b] = ss[b];
    __syncthreads();
    if (tid < NB) {
        float t = s.red[tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += s.red[w * 16 + tid];
        s.rstd[tid] = 1.0f / sqrtf(t / (float)K + eps);
    }
    __syncthreads();
}

// ---------------------------------------------------------------- GEMV (B <= 2)
// K split across the four waves (segment s of 64 lanes x 16 bytes goes to
// wave s % 4); each lane keeps its x values (times the norm gain) in
// registers; each wave reduces its partial dot products with a butterfly,
// and the four wave partials are added in wave order. Output row r gets
//   y[b, r] = (sum_w sum_lane sum_seg sum_e W[r,k] * g[k] * x[b,k]) * rstd[b].
// NSW = segments per wave (compile time), U = rows in flight per wave.
template <typename WT, int NB, int NSW, int U, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_ksplit(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain, RowFn rowp,
                            OutFn out, const Lds& s) {
    using V = Vec16<WT>;
    constexpr int E = V::N, SEG = 64 * E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nseg = (K + SEG - 1) / SEG;
    float xr[NSW][NB][E];
    int kof[NSW];
    bool kval[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const int sg = wave + kWaves * j;
        kof[j] = sg * SEG + lane * E;
        kval[j] = sg < nseg && kof[j] < K;
        float g[E];
        if (gain && kval[j]) V::widen(*(const uint4*)(gain + kof[j]), g);
        else
#pragma unroll
            for (int e = 0; e < E; ++e) g[e] = 1.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (kval[j] && b < B) v = *(const float4*)(x + (int64_t)b * ldx + kof[j] + e);
                xr[j][b][e + 0] = v.x * g[e + 0];
                xr[j][b][e + 1] = v.y * g[e + 1];
                xr[j][b][e + 2] = v.z * g[e + 2];
                xr[j][b][e + 3] = v.w * g[e + 3];
            }
        }
    }
    constexpr int NM = DUAL ? 2 : 1;
    for (int rg = r0; rg < r1; rg += 256) {
        const int rend = min(rg + 256, r1);
        for (int r = rg; r < rend; r += U) {
            uint4 w[U][NM][NSW];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = min(r + u, rend - 1);
                const WT* pr[2];
                rowp(row, pr[0], pr[1]);
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int j = 0; j < NSW; ++j)
                        w[u][m][j] = kval[j] ? *(const uint4*)(pr[m] + kof[j]) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float acc[NB];
#pragma unroll
                    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
#pragma unroll
                    for (int j = 0; j < NSW; ++j) {
                        float wf[E];
                        V::widen(w[u][m][j], wf);
#pragma unroll
                        for (int e = 0; e < E; ++e)
#pragma unroll
                            for (int b = 0; b < NB; ++b) acc[b] = fmaf(wf[e], xr[j][b][e], acc[b]);
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const float v = wave_sum(acc[b]);
                        if (lane == 0 && r + u < rend) s.part[((wave * 256) + (r + u - rg)) * 2 * NB + m * NB + b] = v;
                    }
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < (rend - rg) * NB; i += kThreads) {
            const int rr = i / NB, b = i % NB;
            float t[2];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float a = s.part[(rr)*2 * NB + m * NB + b];
#pragma unroll
                for (int wv = 1; wv < kWaves; ++wv) a += s.part[((wv * 256) + rr) * 2 * NB + m * NB + b];
                t[m] = a;
            }
            if (b < B) out(rg + rr, b, t[0], DUAL ? t[1] : 0.f);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- GEMV (B >= 3)
// One row per wave at a time, K across the lanes, x read from the cache.
// The per-row arithmetic (lane partial sums over segments, butterfly) is
// fixed by the shape, so the result does not depend on the task tiling.
template <typename WT, int NB, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_rowwave(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain, RowFn rowp,
                             OutFn out) {
    using V = Vec16<WT>;
    constexpr int E = V::N, SEG = 64 * E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NM = DUAL ? 2 : 1;
    for (int r = r0 + wave; r < r1; r += kWaves) {
        const WT* pr[2];
        rowp(r, pr[0], pr[1]);
        float acc[NM][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = 0.f;
#pragma unroll 2
        for (int k = lane * E; k < K; k += SEG) {
            uint4 w[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) w[m] = *(const uint4*)(pr[m] + k);
            float g[E];
            if (gain) V::widen(*(const uint4*)(gain + k), g);
            else
#pragma unroll
                for (int e = 0; e < E; ++e) g[e] = 1.f;
            float wf[NM][E];
#pragma unroll
            for (int m = 0; m < NM; ++m) V::widen(w[m], wf[m]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b >= B) continue;
                float xv[E];
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const float4 v = *(const float4*)(x + (int64_t)b * ldx + k + e);
                    xv[e] = v.x * g[e];
                    xv[e + 1] = v.y * g[e + 1];
                    xv[e + 2] = v.z * g[e + 2];
                    xv[e + 3] = v.w * g[e + 3];
                }
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[m][b] = fmaf(wf[m][e], xv[e], acc[m][b]);
            }
        }
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float a0 = wave_sum(acc[0][b]);
            const float a1 = DUAL ? wave_sum(acc[NM - 1][b]) : 0.f;
            if (lane == b) { t0 = a0; t1 = a1; }
        }
        if (lane < B) out(r, lane, t0, t1);
    }
}

template <typename WT, int NB, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_dispatch(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain,
                                              RowFn rowp, OutFn out, const Lds& s) {
    if constexpr (NB <= 2) {
        constexpr int SEG = 64 * Vec16<WT>::N;
        const int nsw = ((K + SEG - 1) / SEG + kWaves - 1) / kWaves;
        if (nsw <= 1) gemv_ksplit<WT, NB, 1, 16, DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out, s);
        else if (nsw <= 2) gemv_ksplit<WT, NB, 2, 16 / (DUAL ? 2 : 1), DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out, s);
        else if (nsw <= 4) gemv_ksplit<WT, NB, 4, 8 / (DUAL ? 2 : 1), DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out, s);
        else if (nsw <= 6) gemv_ksplit<WT, NB, 6, 4 / (DUAL ? 2 : 1), DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out, s);
        else gemv_ksplit<WT, NB, 8, 4 / (DUAL ? 2 : 1), DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out, s);
    } else {
        (void)s;
        gemv_rowwave<WT, NB, DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out);
    }
}

// ---------------------------------------------------------------- GEMV tasks

template <typename WT, int NB>
__device__ __forceinline__ void run_gemv_task(const KParams& p, const TaskRec& t, const Lds& s) {
    const int l = t.layer, B = p.B, H = p.H;
    const int r0 = t.a0, r1 = t.a1;
    switch (t.op) {
        case OP_EMBED: {
            const WT* E = (const WT*)p.embed;
            const int n = r1 - r0;
            for (int i = threadIdx.x; i < n * B; i += kThreads) {
                const int b = i / n, r = r0 + i % n;
                int tok = p.tokens[b];
                if (tok < 0 || tok >= p.V) {
                    if (r == r0) raise_error(p.ctrl, MK_ERR_TOKEN);
                    tok = 0;
                }
                p.x0_w[(int64_t)b * H + r] = load_scalar<WT>(E, (int64_t)tok * H + r);
            }
            break;
        }
        case OP_QKV: {
            const LayerPtrs w = p.lw[l];
            const float* x = layer_in(p, l);
            block_rstd<NB>(x, H, H, B, p.eps, s);
            const int QD = p.QD, KD = p.KD, ld = QD + 2 * KD;
            const WT* wq = (const WT*)w.wq;
            const WT* wk = (const WT*)w.wk;
            const WT* wv = (const WT*)w.wv;
            float* o = layer_buf(p, l, p.off_qkv);
            auto rowp = [&](int r, const WT*& a, const WT*& b2) {
                a = r < QD ? wq + (int64_t)r * H : (r < QD + KD ? wk + (int64_t)(r - QD) * H : wv + (int64_t)(r - QD - KD) * H);
                b2 = a;
            };
            auto out = [&](int r, int b, float v, float) { o[(int64_t)b * ld + r] = v * s.rstd[b]; };
            gemv_dispatch<WT, NB, false>(r0, r1, H, x, H, B, (const WT*)w.attn_norm, rowp, out, s);
            break;
        }
        case OP_O: {
            const LayerPtrs w = p.lw[l];
            const float* a = layer_buf(p, l, p.off_attn);
            const float* xin = layer_in(p, l);
            float* o = layer_buf(p, l, p.off_xmid);
            const WT* wo = (const WT*)w.wo;
            const int K = p.QD;
            auto rowp = [&](int r, const WT*& a0, const WT*& b2) { a0 = wo + (int64_t)r * K; b2 = a0; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                o[i] = xin[i] + v;
            };
            gemv_dispatch<WT, NB, false>(r0, r1, K, a, K, B, (const WT*)nullptr, rowp, out, s);
            break;
        }
        case OP_GATEUP: {
            const LayerPtrs w = p.lw[l];
            const float* x = layer_buf(p, l, p.off_xmid);
            block_rstd<NB>(x, H, H, B, p.eps, s);
            float* o = layer_buf(p, l, p.off_h);
            const WT* wg = (const WT*)w.w_gate;
            const WT* wu = (const WT*)w.w_up;
            const int F = p.F;
            auto rowp = [&](int r, const WT*& a0, const WT*& b2) {
                a0 = wg + (int64_t)r * H;
                b2 = wu + (int64_t)r * H;
            };
            auto out = [&](int r, int b, float g, float u) {
                const float rs = s.rstd[b];
                const float gg = g * rs, uu = u * rs;
                o[(int64_t)b * F + r] = (gg / (1.0f + __expf(-gg))) * uu;
            };
            gemv_dispatch<WT, NB, true>(r0, r1, H, x, H, B, (const WT*)w.mlp_norm, rowp, out, s);
            break;
        }
        case OP_DOWN: {
            const LayerPtrs w = p.lw[l];
            const float* h = layer_buf(p, l, p.off_h);
            const float* xm = layer_buf(p, l, p.off_xmid);
            float* o = layer_out(p, l);
            const WT* wd = (const WT*)w.w_down;
            const int F = p.F;
            auto rowp = [&](int r, const WT*& a0, const WT*& b2) { a0 = wd + (int64_t)r * F; b2 = a0; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                o[i] = xm[i] + v;
            };
            gemv_dispatch<WT, NB, false>(r0, r1, F, h, F, B, (const WT*)nullptr, rowp, out, s);
            break;
        }
        case OP_LM: {
            const float* x = p.x_final;
            block_rstd<NB>(x, H, H, B, p.eps, s);
            const WT* wl = (const WT*)p.lm_head;
            float* o = p.logits;
            const int V = p.V;
            auto rowp = [&](int r, const WT*& a0, const WT*& b2) { a0 = wl + (int64_t)r * H; b2 = a0; };
            auto out = [&](int r, int b, float v, float) { o[(int64_t)b * V + r] = v * s.rstd[b]; };
            gemv_dispatch<WT, NB, false>(r0, r1, H, x, H, B, (const WT*)p.final_norm, rowp, out, s);
            break;
        }
        default: break;
    }
}

// ---------------------------------------------------------------- signalling

// Make this workgroup's writes visible device-wide, then count one
// arrival on event e (MPK article §2.1: trigger_count / required_count).
// The arrival that completes a JIT-triggering event posts a message to the
// scheduler mailbox (§2.2: the data-dependent successor is launched JIT).
__device__ __forceinline__ void signal_event(const KParams& p, int e, const Lds& s) {
    fence_release();
    __syncthreads();
    if (threadIdx.x == 0 && e >= 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.ev[e], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const EventRec er = p.evrec[e];
        if (er.jit_layer >= 0 && old + 1u == er.required * (p.epoch + 1u)) {
            // the completing arrival forwards every producer's writes to the
            // scheduler: acquire what the earlier releases published first
            fence_acquire();
            const int64_t pos = __hip_atomic_fetch_add(&p.ctrl->mb_tail, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            RingSlot* sl = &p.mb[pos & p.mb_mask];
            sl->p0 = er.jit_layer;
            sl->p1 = 0;
            __hip_atomic_store(&sl->tag, pos + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    (void)s;
}

// ---------------------------------------------------------------- attention

__device__ __forceinline__ int64_t kv_offset(const KParams& p, int l, int b, int g, int pos) {
    if (!p.paged) return (int64_t)l * p.kv_layer_stride + ((int64_t)(b * p.Hkv + g) * p.cap + pos) * p.D;
    const int blk = p.block_table[(int64_t)b * p.max_blocks + pos / p.kv_block];
    return (int64_t)l * p.kv_layer_stride + ((int64_t)blk * p.Hkv + g) * p.kv_block * p.D + (int64_t)(pos % p.kv_block) * p.D;
}

// RMSNorm over one head (D = 64 or 128) held by a wave as D/64 values per
// lane (element j in lane j % 64, slot j / 64), then rotate-half RoPE.
template <typename WT>
__device__ __forceinline__ void head_norm_rope(float* v, int D, const WT* gain, bool norm, float eps, const float2* rope_row) {
    const int lane = threadIdx.x & 63;
    const int per = D / 64;
    if (norm) {
        float ss = 0.f;
        for (int i = 0; i < per; ++i) ss += v[i] * v[i];
        ss = wave_sum(ss);
        const float rs = 1.0f / sqrtf(ss / (float)D + eps);
        for (int i = 0; i < per; ++i) v[i] = (v[i] * rs) * load_scalar<WT>(gain, lane + 64 * i);
    }
    if (per == 2) {
        // pair (lane, lane + 64) sits in one lane
        const float2 cs = rope_row[lane];
        const float a = v[0], b = v[1];
        v[0] = a * cs.x - b * cs.y;
        v[1] = b * cs.x + a * cs.y;
    } else {
        // D = 64: pair (i, i + 32) spans lanes i and i + 32
        const float other = __shfl_xor(v[0], 32, 64);
        const int i = lane & 31;
        const float2 cs = rope_row[i];
        if (lane < 32) v[0] = v[0] * cs.x - other * cs.y;
        else v[0] = v[0] * cs.x + other * cs.y;
    }
}

// One split of the split-KV decode attention for (layer, b, g, split):
// positions [split*C, min((split+1)*C, pos+1)). Writes the split's partial
// (m, l, acc) and, if it is the last to arrive for (b, g), combines all
// splits in split order and (persistent mode) signals the layer's
// attention event. The split that holds position pos first normalises,
// rotates and appends the new k and v (rounded to the cache type).
template <typename WT>
__device__ __forceinline__ void attention_task(const KParams& p, int l, int bg, int split, const Lds& s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hkv = p.Hkv, D = p.D, G = p.Hq / p.Hkv, C = p.chunk;
    const int b = bg / Hkv, g = bg % Hkv;
    const int pos = p.seq_lens[b];
    const bool overflow = pos < 0 || pos + 1 > p.cap;
    const int keys = pos + 1;
    const int ns = overflow ? 1 : (keys + C - 1) / C;
    if (split >= ns) return;  // reserved AOT slot beyond this sequence's length
    float* out = layer_buf(p, l, p.off_attn) + (int64_t)b * p.QD + (int64_t)g * G * D;
    const float* qkv = layer_buf(p, l, p.off_qkv) + (int64_t)b * (p.QD + 2 * p.KD);
    const LayerPtrs& lw = p.lw[l];

    if (overflow) {
        for (int i = tid; i < G * D; i += kThreads) out[i] = 0.f;
        if (tid == 0) raise_error(p.ctrl, MK_ERR_KV_OVERFLOW);
        if (p.persistent) signal_event(p, ev_attn(l), s);
        return;
    }
    const int j0 = split * C, j1 = min(j0 + C, keys);
    const bool owner = (j1 == keys);
    const float2* rope_row = p.rope + (int64_t)pos * (D / 2);
    const WT* qn = (const WT*)lw.q_norm;
    const WT* kn = (const WT*)lw.k_norm;

    // 1. query heads of this group: norm + RoPE into LDS
    for (int hh = wave; hh < G; hh += kWaves) {
        float v[2];
        const int per = D / 64;
        for (int i = 0; i < per; ++i) v[i] = qkv[(int64_t)(g * G + hh) * D + lane + 64 * i];
        head_norm_rope<WT>(v, D, qn, p.qk_norm != 0, p.eps, rope_row);
        for (int i = 0; i < per; ++i) s.q[hh * D + lane + 64 * i] = v[i];
    }
    // 2. owner: new k (norm + RoPE) and v, rounded to the cache type, appended
    if (owner && wave < 2) {
        float v[2];
        const int per = D / 64;
        const int64_t base = wave == 0 ? (int64_t)p.QD + (int64_t)g * D : (int64_t)p.QD + p.KD + (int64_t)g * D;
        for (int i = 0; i < per; ++i) v[i] = qkv[base + lane + 64 * i];
        if (wave == 0) head_norm_rope<WT>(v, D, kn, p.qk_norm != 0, p.eps, rope_row);
        WT* dst = (WT*)(wave == 0 ? p.kv_k : p.kv_v) + kv_offset(p, l, b, g, pos);
        for (int i = 0; i < per; ++i) {
            const WT c = from_float<WT>(v[i]);
            dst[lane + 64 * i] = c;
            s.kn[wave * 128 + lane + 64 * i] = to_float<WT>(c);
        }
    }
    __syncthreads();

    // 3. scores s_j = (q_h . k_j) * scale for j in [j0, j1)
    using VK = Vec16<WT>;
    constexpr int E = VK::N;
    const int lpr = D / E;          // lanes per K row
    const int ppw = 64 / lpr;       // rows per wave load
    const int rr = lane / lpr, cc = lane % lpr;
    const int n = j1 - j0;
    float qreg[8][E];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
#pragma unroll
        for (int e = 0; e < E; ++e) qreg[hh][e] = hh < G ? s.q[hh * D + cc * E + e] : 0.f;
    const WT* kbase = (const WT*)p.kv_k;
    for (int j = wave * ppw + rr; j - rr < n; j += kWaves * ppw) {
        const int jj = j0 + j;
        float kf[E];
        const bool valid = j < n;
        if (valid && jj == pos) {
#pragma unroll
            for (int e = 0; e < E; ++e) kf[e] = s.kn[cc * E + e];
        } else if (valid) {
            const uint4 kv = *(const uint4*)(kbase + kv_offset(p, l, b, g, jj) + cc * E);
            VK::widen(kv, kf);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) kf[e] = 0.f;
        }
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            if (hh >= G) break;
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) d = fmaf(qreg[hh][e], kf[e], d);
            for (int o = lpr / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
            if (valid && cc == 0) s.p[hh * C + j] = d * p.scale;
        }
    }
    __syncthreads();

    // 4. per-head max and exp-sum over this split (fixed strides and tree)
    for (int hh = wave; hh < G; hh += kWaves) {
        float m = -INFINITY;
        for (int j = lane; j < n; j += 64) m = fmaxf(m, s.p[hh * C + j]);
        m = wave_max(m);
        float sum = 0.f;
        for (int j = lane; j < n; j += 64) {
            const float e = __expf(s.p[hh * C + j] - m);
            s.p[hh * C + j] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            s.ml[2 * hh] = m;
            s.ml[2 * hh + 1] = sum;
        }
    }
    __syncthreads();

    // 5. acc[h][d] = sum_j p[h][j] V[j][d]
    const WT* vbase = (const WT*)p.kv_v;
    float acc[8][E];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
    for (int j = wave * ppw + rr; j < n; j += kWaves * ppw) {
        const int jj = j0 + j;
        float vf[E];
        if (jj == pos) {
#pragma unroll
            for (int e = 0; e < E; ++e) vf[e] = s.kn[128 + cc * E + e];
        } else {
            const uint4 vv = *(const uint4*)(vbase + kv_offset(p, l, b, g, jj) + cc * E);
            VK::widen(vv, vf);
        }
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            if (hh >= G) break;
            const float pj = s.p[hh * C + j];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[hh][e] = fmaf(pj, vf[e], acc[hh][e]);
        }
    }
    // reduce over the row groups of the wave (lanes with equal cc)
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        if (hh >= G) break;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float v = acc[hh][e];
            for (int o = lpr; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
            acc[hh][e] = v;
        }
    }
    if (rr == 0) {
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            if (hh >= G) break;
#pragma unroll
            for (int e = 0; e < E; ++e) s.acc[(wave * 8 + hh) * 128 + cc * E + e] = acc[hh][e];
        }
    }
    __syncthreads();

    // 6. partial record: acc[G*D], then m[G], l[G]
    const int rec = G * D + 2 * G;
    float* part = p.partials + ((int64_t)bg * p.max_splits + split) * rec;
    for (int i = tid; i < G * D; i += kThreads) {
        const int hh = i / D, d = i % D;
        float a = s.acc[hh * 128 + d];
        for (int w = 1; w < kWaves; ++w) a += s.acc[(w * 8 + hh) * 128 + d];
        part[i] = a;
    }
    if (tid < 2 * G) part[G * D + tid] = s.ml[tid];  // interleaved (m, l) pairs

    // 7. last arrival combines the splits in split order
    fence_release();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.arrive[bg], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s.cmd[8] = (old + 1u == (uint32_t)ns) ? 1 : 0;
    }
    __syncthreads();
    const bool last = s.cmd[8] != 0;
    __syncthreads();
    if (!last) return;
    fence_acquire();
    const float* part0 = p.partials + (int64_t)bg * p.max_splits * rec;
    for (int i = tid; i < G * D; i += kThreads) {
        const int hh = i / D;
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, part0[(int64_t)sp * rec + G * D + 2 * hh]);
        float num = 0.f, den = 0.f;
        for (int sp = 0; sp < ns; ++sp) {
            const float* pr = part0 + (int64_t)sp * rec;
            const float wgt = __expf(pr[G * D + 2 * hh] - M);
            den = fmaf(wgt, pr[G * D + 2 * hh + 1], den);
            num = fmaf(wgt, pr[i], num);
        }
        out[i] = num / den;
    }
    if (tid == 0) __hip_atomic_store(&p.arrive[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.persistent) signal_event(p, ev_attn(l), s);
}

}  // namespace mk
