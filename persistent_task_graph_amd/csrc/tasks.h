// Task bodies. The same __device__ functions run inside the persistent
// megakernel and inside the kernel-per-operator launches, so the two modes
// produce identical bits: every reduction below has a fixed order that
// depends only on the shape (never on which workgroup, task or schedule
// runs it), no floating-point atomics are used, and contraction is off.
#pragma once

#include <type_traits>

#include "device.h"

namespace mk {

// ---------------------------------------------------------------- LDS layout
// Carved from one dynamic shared buffer; sizes in floats. A workgroup runs
// one task at a time, so the GEMV partial sums and the attention regions
// share one union after the common header.
struct Lds {
    float* red;   // kWaves * 16: reductions / broadcast
    int* cmd;     // 16 ints
    float* rstd;  // 16
    float* part;  // kPartFloats: GEMV cross-wave partial sums (union member)
    float* q;     // 8 * 128: rotated query heads of one KV group
    float* kn;    // 2 * 128: new k, v (rounded to the cache type)
    float* acc;   // kWaves * 8 * 128: P.V partials per wave
    float* wml;   // kWaves * 16: per wave (m[8], l[8])
    float* ml;    // 2 * 8: (m, l) per head of the split
    float* cmb;   // kCmbSplits * (8 * 128 + 16): partials staged for the combine
    float* pt;    // kWaves * 32 * 8: attention probabilities per wave [row][head]
    int* btab;    // paged cache: block-table entries of the split
    uint64_t* marks;  // 4 trace phase marks
    uint4* pre;   // kWaves * kPreSlots: next GEMV task's weights preloaded while waiting
    int* pst;     // kWaves * kPstInts: each wave's preload cursor
};

constexpr int kCmbSplits = 16;  // splits merged per staged chunk (one load round for up to 16)
constexpr int kPartFloats = 8192;  // GEMV cross-wave partial sums
constexpr int kPstInts = 24;  // preload cursor of one wave (ints)
constexpr int kLdsHeader = kWaves * 16 + 16 + 16 + 8 + kWaves * kPstInts;
constexpr int kAttnFloats = 8 * 128 + 2 * 128 + kWaves * 8 * 128 + kWaves * 16 + 16 + kCmbSplits * (8 * 128 + 16) +
                            kWaves * 32 * 8;
// GEMV and embedding tasks touch only the header and the partial sums
__host__ __device__ constexpr int lds_bytes_gemv() { return 4 * (kLdsHeader + kPartFloats); }
// W4 matrix-core GEMV: a pass's scales, [TMAX][NM][16 rows][K / 128] floats:
// at most 3 x 2 tiles (gate/up) of K / 128 <= 96 groups (K <= 12288)
constexpr int kW4ScaleLdsBytes = 4 * 3 * 2 * 16 * 96;
// Preload pages: after the partial sums, 1 KB slots per wave, each holding
// one wave-wide 16-byte-per-lane load of the next GEMV task's weights (the
// MPK article's paged shared memory, §3.1, filled during the wait, §3.2).
// They overlay the attention regions, which no task uses while a worker
// waits for a GEMV event (ahead-of-time queues only).
constexpr int kPreSlots = 30;
__host__ __device__ constexpr int lds_bytes_preload() { return lds_bytes_gemv() + kWaves * kPreSlots * 1024; }
// block-table entries one split of `chunk` keys can span
__host__ __device__ constexpr int attn_btab_ints(int chunk, int kv_block) { return chunk / kv_block + 2; }
__host__ __device__ inline int lds_bytes_for(int chunk_max, int kv_block, bool paged) {
    const int attn = kAttnFloats + (paged ? attn_btab_ints(chunk_max, kv_block) : 0);
    return 4 * (kLdsHeader + (attn > kPartFloats ? attn : kPartFloats));
}

__device__ __forceinline__ Lds carve_lds(float* base) {
    Lds s;
    float* p = base;
    s.red = p; p += kWaves * 16;
    s.cmd = (int*)p; p += 16;
    s.marks = (uint64_t*)p; p += 8;
    s.rstd = p; p += 16;
    s.pst = (int*)p; p += kWaves * kPstInts;
    s.part = p;  // the attention regions below overlay the partial sums
    s.q = p; p += 8 * 128;
    s.kn = p; p += 2 * 128;
    s.acc = p; p += kWaves * 8 * 128;
    s.wml = p; p += kWaves * 16;
    s.ml = p; p += 16;
    s.cmb = p; p += kCmbSplits * (8 * 128 + 16);
    s.pt = p; p += kWaves * 32 * 8;
    s.btab = (int*)p;
    s.pre = (uint4*)(s.part + kPartFloats);
    return s;
}

// ---------------------------------------------------------------- activations

// Keys per attention split in this step (the same for every task and mode).
// Evaluated by one whole wave: lane i holds sequence i (and i + 64, ...),
// and the split counts are summed exactly across the wave.
__device__ __forceinline__ int attn_chunk(const KParams& p) {
    const int lane = threadIdx.x & 63;
    const int k0 = lane < p.B ? attn_keys(p.seq_lens[lane]) : 0;
    auto total = [&](int c) {
        int t = k0 > 0 ? n_splits_for(k0, c) : 0;
        for (int b = lane + 64; b < p.B; b += 64) t += n_splits_for(attn_keys(p.seq_lens[b]), c);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
        return (long long)t * p.Hkv;
    };
    return attn_chunk_search(total, p.chunk, p.chunk_max, p.attn_target);
}

// Split task k of the step, counted in (b, g, split) order, for chunk C:
// its (b * Hkv + g, split), or false when the step has fewer tasks.
// Uniform across the workgroup (scalar loads of seq_lens).
__device__ __forceinline__ bool attn_locate(const KParams& p, int C, int k, int& bg, int& split) {
    for (int b = 0; b < p.B; ++b) {
        const int pos = p.seq_lens[b];
        const int ns = (pos < 0 || pos + 1 > p.cap) ? 1 : (pos + C) / C;
        if (k < ns * p.Hkv) {
            bg = b * p.Hkv + k / ns;
            split = k % ns;
            return true;
        }
        k -= ns * p.Hkv;
    }
    return false;
}

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
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(B * ldx) * 4u);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        ss[b] = 0.f;
        if (b < B)
            for (int k = tid * 4; k < K; k += kThreads * 4) {
                const uint4 u = buf_load16_act(xr, (uint32_t)(b * ldx + k) * 4u, 0);
                const float4 v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                             __uint_as_float(u.w));
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
// NSW = segments per wave (compile time), U = rows per group. Weight loads
// are double-buffered: group i+1 is in flight while group i is consumed.
// Rows past the tile and segments past K load through an out-of-range
// offset (zeros, no memory traffic), so every load is issued unconditionally.
// The first pre_rows rows of the task may already sit in this wave's LDS
// preload slots (slot (r - r0) * NM * NSW + m * NSW + j holds what the load
// of row r, matrix m, segment j would return); they are read from there,
// the arithmetic is the same.
template <typename WT, int NB, int NSW, int U, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_ksplit(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain,
                                            float eps, RowFn rowp, OutFn out, const Lds& s, bool tr, int pre_rows) {
    using V = Vec16<WT>;
    constexpr int E = V::N, SEG = 64 * E;
    constexpr int NM = DUAL ? 2 : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nseg = (K + SEG - 1) / SEG;
    uint32_t voff[NSW];
    bool kvalid[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const int k = (wave + kWaves * j) * SEG + lane * E;
        kvalid[j] = wave + kWaves * j < nseg && k < K;
        voff[j] = kvalid[j] ? (uint32_t)k * (uint32_t)sizeof(WT) : kOOB;
    }
    constexpr int WIN = kPartFloats / (kWaves * NM * NB);  // rows per LDS window
    auto load = [&](uint4 (&w)[U][NM][NSW], int r, int rend) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool rv = r + u < rend;
            RowRef rf[2];
            rowp(rv ? r + u : rend - 1, rf[0], rf[1]);
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < NSW; ++j) w[u][m][j] = buf_load16_w(rf[m].r, rv ? voff[j] : kOOB, rf[m].soff);
        }
    };
    // preloaded rows [r0, rp) lie in the first window; their DMA loads were
    // issued while the worker waited and have landed once this wave's loads
    // are complete
    const int rp = r0 + min(pre_rows, min(WIN, r1 - r0));
    if (rp > r0) __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    lds_u4* pre = (lds_u4*)(s.pre + wave * (kPreSlots * 64));
    auto lds_load = [&](uint4 (&w)[U][NM][NSW], int r, int rend) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < NSW; ++j) {
                    // rows past rend and k past K read slot 0 and use zeros
                    const bool ok = r + u < rend && kvalid[j];
                    const int n = ok ? ((r + u - r0) * NM + m) * NSW + j : 0;
                    const u32x4 v = pre[n * 64 + lane];
                    w[u][m][j] = ok ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(0u, 0u, 0u, 0u);
                }
    };
    // the first weight group goes out before the (latency-bound) x loads
    uint4 wa[U][NM][NSW], wb[U][NM][NSW];
    load(wa, rp, min(r0 + WIN, r1));

    // x (agent-coherent: written earlier in this step) and the norm gain
    const __amdgpu_buffer_rsrc_t xr_rs = make_rsrc(x, (uint32_t)(B * ldx) * 4u);
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(gain, gain ? (uint32_t)K * (uint32_t)sizeof(WT) : 0u);
    float xr[NSW][NB][E];
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t xo = (kvalid[j] && b < B) ? (uint32_t)(b * ldx) * 4u + voff[j] / (uint32_t)sizeof(WT) * 4u : kOOB;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const uint4 v = buf_load16_act(xr_rs, xo, (uint32_t)e * 4u);
                xr[j][b][e + 0] = __uint_as_float(v.x);
                xr[j][b][e + 1] = __uint_as_float(v.y);
                xr[j][b][e + 2] = __uint_as_float(v.z);
                xr[j][b][e + 3] = __uint_as_float(v.w);
            }
        }
    float g[NSW][E];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        if (gain) V::widen(buf_load16(g_rs, voff[j], 0), g[j]);
        else
#pragma unroll
            for (int e = 0; e < E; ++e) g[j][e] = 1.f;
    }
    if (gain) {
        // RMSNorm statistic: the four waves' segments cover K exactly once;
        // lane sums in (segment, element) order, butterfly, then waves in order
        float ss[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            ss[b] = 0.f;
#pragma unroll
            for (int j = 0; j < NSW; ++j)
#pragma unroll
                for (int e = 0; e < E; ++e) ss[b] += xr[j][b][e] * xr[j][b][e];
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
        // s.rstd is read by `out` only after the window barrier below
    }
    if (tr && tid == 0) s.marks[0] = now_ticks();
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < E; ++e) xr[j][b][e] = xr[j][b][e] * g[j][e];

    auto consume = [&](const uint4 (&w)[U][NM][NSW], int r, int rend, int rg) {
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
                    if (lane == 0 && r + u < rend) s.part[((wave * WIN) + (r + u - rg)) * NM * NB + m * NB + b] = v;
                }
            }
        }
    };
    for (int rg = r0; rg < r1; rg += WIN) {
        const int rend = min(rg + WIN, r1);
        if (rg != r0) load(wa, rg, rend);
        int rs = rg;
        if (rg == r0 && rp > r0) {
            for (int r = r0; r < rp; r += U) {
                lds_load(wb, r, rp);
                consume(wb, r, rp, rg);
            }
            rs = rp;
        }
        for (int r = rs; r < rend; r += 2 * U) {
            load(wb, r + U, rend);
            consume(wa, r, rend, rg);
            load(wa, r + 2 * U, rend);
            consume(wb, r + U, rend, rg);
        }
        if (tr && tid == 0) s.marks[1] = now_ticks();
        __syncthreads();
        for (int i = tid; i < (rend - rg) * NB; i += kThreads) {
            const int rr = i / NB, b = i % NB;
            float t[2] = {0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float a = s.part[rr * NM * NB + m * NB + b];
#pragma unroll
                for (int wv = 1; wv < kWaves; ++wv) a += s.part[((wv * WIN) + rr) * NM * NB + m * NB + b];
                t[m] = a;
            }
            if (b < B) out(rg + rr, b, t[0], t[1]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- GEMV (B >= 3)
// One row per wave at a time, K across the lanes, x read through the cache.
// The per-row arithmetic (lane partial sums over segments, butterfly) is
// fixed by the shape, so the result does not depend on the task tiling.
template <typename WT, int NB, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_rowwave(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain,
                                             RowFn rowp, OutFn out) {
    using V = Vec16<WT>;
    constexpr int E = V::N, SEG = 64 * E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NM = DUAL ? 2 : 1;
    const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(x, (uint32_t)(B * ldx) * 4u);
    for (int r = r0 + wave; r < r1; r += kWaves) {
        RowRef rf[2];
        rowp(r, rf[0], rf[1]);
        float acc[NM][NB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = 0.f;
#pragma unroll 2
        for (int k = lane * E; k < K; k += SEG) {
            uint4 w[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) w[m] = buf_load16_w(rf[m].r, (uint32_t)k * (uint32_t)sizeof(WT), rf[m].soff);
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
                    const uint4 v = buf_load16_act(x_rs, (uint32_t)(b * ldx + k + e) * 4u, 0);
                    xv[e] = __uint_as_float(v.x) * g[e];
                    xv[e + 1] = __uint_as_float(v.y) * g[e + 1];
                    xv[e + 2] = __uint_as_float(v.z) * g[e + 2];
                    xv[e + 3] = __uint_as_float(v.w) * g[e + 3];
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
            if (lane == b) {
                t0 = a0;
                t1 = a1;
            }
        }
        if (lane < B) out(r, lane, t0, t1);
    }
}

// ---------------------------------------------------------------- GEMV with 4-bit weights (B <= 2)
// W4 matrix buffer (one per [rows, K] matrix): 4-bit codes in row order, two
// per byte (low nibble first), rows * K / 2 bytes; then, from that size
// rounded up to 256 bytes, one bf16 scale per 128 inputs of a row. The
// weight is (code - 8) * scale.
#ifdef MK_W4_KERNELS
constexpr bool kW4MfmaKernels = true;  // batch >= 4 instances for W4 plans
#else
constexpr bool kW4MfmaKernels = false;
#endif
constexpr int kW4Group = 128;
__host__ __device__ constexpr int64_t w4_scale_offset(int64_t rows, int64_t K) { return (rows * K / 2 + 255) / 256 * 256; }

// v & m computed where the compiler cannot see the result's zero bits
__device__ __forceinline__ uint32_t opaque_and(uint32_t v, uint32_t m) {
    uint32_t r;
    asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(m));
    return r;
}

// One W4 matrix tile: codes and scales of rows [lo, lo + n)
struct W4Tile {
    __amdgpu_buffer_rsrc_t q, sc;
    int lo, n;
    uint32_t qrow, srow;  // bytes per row of codes, of scales
};
__device__ __forceinline__ W4Tile w4_tile(const void* m, int K, int rows, int lo_, int hi_) {
    W4Tile t;
    t.lo = max(0, min(lo_, rows));
    const int hi = max(t.lo, min(hi_, rows));
    t.n = hi - t.lo;
    t.qrow = (uint32_t)K / 2u;
    t.srow = (uint32_t)(K / kW4Group) * 2u;
    const char* base = (const char*)m;
    t.q = make_rsrc(base + (int64_t)t.lo * t.qrow, (uint32_t)t.n * t.qrow);
    t.sc = make_rsrc(base + w4_scale_offset(rows, K) + (int64_t)t.lo * t.srow, (uint32_t)t.n * t.srow);
    return t;
}

// Same shape as gemv_ksplit: K in segments of 1024 inputs (64 lanes x 16
// codes, one 8-byte load per lane), segment s to wave s % 4; each lane keeps
// its 16 inputs (times the norm gain) and their sum in registers. A lane's
// 16 codes share one scale, so its part of row r is
//   scale * (sum_e code_e * x_e - 8 * sum_e x_e),
// summed over its segments, then over the wave (butterfly) and the waves
// in order. Rows past the tile and inputs past K load zeros (out of range).
// RowFn(r) gives the tile holding row r (and the second matrix's, for DUAL).
template <int NB, int NSW, int U, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_w4(int r0, int r1, int K, const float* x, int ldx, int B, const bf16_t* gain,
                                        float eps, RowFn rowp, OutFn out, const Lds& s, bool tr) {
    constexpr int E = 16, SEG = 64 * E;
    constexpr int NM = DUAL ? 2 : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nseg = (K + SEG - 1) / SEG;
    uint32_t qoff[NSW], soff[NSW];
    bool kvalid[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const int k = (wave + kWaves * j) * SEG + lane * E;
        kvalid[j] = wave + kWaves * j < nseg && k < K;
        qoff[j] = kvalid[j] ? (uint32_t)k / 2u : kOOB;
        soff[j] = kvalid[j] ? (uint32_t)(k / kW4Group) * 2u : kOOB;
    }
    constexpr int WIN = kPartFloats / (kWaves * NM * NB);
    struct Row {
        uint2 q[NM][NSW];
        uint32_t sc[NM][NSW];
    };
    auto load = [&](Row (&w)[U], int r, int rend) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool rv = r + u < rend;
            W4Tile ta, tb;
            int rr;  // the row inside its tile
            rowp(rv ? r + u : rend - 1, ta, tb, rr);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const W4Tile& t = m == 0 ? ta : tb;
#pragma unroll
                for (int j = 0; j < NSW; ++j) {
                    const uint32_t qo = rv ? qoff[j] : kOOB, so = rv ? soff[j] : kOOB;
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(t.q, qo, (uint32_t)rr * t.qrow, kStreamAux);
                    w[u].q[m][j] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
                    w[u].sc[m][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(t.sc, so, (uint32_t)rr * t.srow, 0);
                }
            }
        }
    };
    Row wa[U], wb[U];
    load(wa, r0, min(r0 + WIN, r1));

    const __amdgpu_buffer_rsrc_t xr_rs = make_rsrc(x, (uint32_t)(B * ldx) * 4u);
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(gain, gain ? (uint32_t)K * 2u : 0u);
    float xr[NSW][NB][E];
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t xo = (kvalid[j] && b < B) ? (uint32_t)(b * ldx + (wave + kWaves * j) * SEG + lane * E) * 4u : kOOB;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const uint4 v = buf_load16_act(xr_rs, xo, (uint32_t)e * 4u);
                xr[j][b][e + 0] = __uint_as_float(v.x);
                xr[j][b][e + 1] = __uint_as_float(v.y);
                xr[j][b][e + 2] = __uint_as_float(v.z);
                xr[j][b][e + 3] = __uint_as_float(v.w);
            }
        }
    float g[NSW][E];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        if (gain) {
            const uint32_t go = kvalid[j] ? (uint32_t)((wave + kWaves * j) * SEG + lane * E) * 2u : kOOB;
            Vec16<bf16_t>::widen(buf_load16(g_rs, go, 0), &g[j][0]);
            Vec16<bf16_t>::widen(buf_load16(g_rs, go, 16), &g[j][8]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) g[j][e] = 1.f;
        }
    }
    if (gain) {
        float ss[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            ss[b] = 0.f;
#pragma unroll
            for (int j = 0; j < NSW; ++j)
#pragma unroll
                for (int e = 0; e < E; ++e) ss[b] += xr[j][b][e] * xr[j][b][e];
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
    }
    if (tr && tid == 0) s.marks[0] = now_ticks();
    float sx[NSW][NB];  // sum of the lane's 16 inputs (times the gain)
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                xr[j][b][e] = xr[j][b][e] * g[j][e];
                t += xr[j][b][e];
            }
            sx[j][b] = t;
        }

    auto consume = [&](const Row (&w)[U], int r, int rend, int rg) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float acc[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b] = 0.f;
#pragma unroll
                for (int j = 0; j < NSW; ++j) {
                    // codes 0..15 of the lane: byte i of the 8 holds codes 2i, 2i + 1.
                    // The masks are opaque to the compiler, so each masked byte
                    // converts with one v_cvt_f32_ubyte{0..3} (it would otherwise
                    // fold mask and shift into a bit-field extract plus a convert)
                    const uint32_t lo0 = opaque_and(w[u].q[m][j].x, 0x0F0F0F0Fu);
                    const uint32_t hi0 = opaque_and(w[u].q[m][j].x >> 4, 0x0F0F0F0Fu);
                    const uint32_t lo1 = opaque_and(w[u].q[m][j].y, 0x0F0F0F0Fu);
                    const uint32_t hi1 = opaque_and(w[u].q[m][j].y >> 4, 0x0F0F0F0Fu);
                    float c[E];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        c[2 * i] = (float)((lo0 >> (8 * i)) & 0xFFu);
                        c[2 * i + 1] = (float)((hi0 >> (8 * i)) & 0xFFu);
                        c[8 + 2 * i] = (float)((lo1 >> (8 * i)) & 0xFFu);
                        c[8 + 2 * i + 1] = (float)((hi1 >> (8 * i)) & 0xFFu);
                    }
                    const float sc = __uint_as_float(w[u].sc[m][j] << 16);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        float d = 0.f;
#pragma unroll
                        for (int e = 0; e < E; ++e) d = fmaf(c[e], xr[j][b][e], d);
                        acc[b] = fmaf(sc, fmaf(-8.0f, sx[j][b], d), acc[b]);
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float v = wave_sum(acc[b]);
                    if (lane == 0 && r + u < rend) s.part[((wave * WIN) + (r + u - rg)) * NM * NB + m * NB + b] = v;
                }
            }
        }
    };
    for (int rg = r0; rg < r1; rg += WIN) {
        const int rend = min(rg + WIN, r1);
        if (rg != r0) load(wa, rg, rend);
        for (int r = rg; r < rend; r += 2 * U) {
            load(wb, r + U, rend);
            consume(wa, r, rend, rg);
            load(wa, r + 2 * U, rend);
            consume(wb, r + U, rend, rg);
        }
        if (tr && tid == 0) s.marks[1] = now_ticks();
        __syncthreads();
        for (int i = tid; i < (rend - rg) * NB; i += kThreads) {
            const int rr = i / NB, b = i % NB;
            float t[2] = {0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float a = s.part[rr * NM * NB + m * NB + b];
#pragma unroll
                for (int wv = 1; wv < kWaves; ++wv) a += s.part[((wv * WIN) + rr) * NM * NB + m * NB + b];
                t[m] = a;
            }
            if (b < B) out(rg + rr, b, t[0], t[1]);
        }
        __syncthreads();
    }
}

template <int NB, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_w4_dispatch(int r0, int r1, int K, const float* x, int ldx, int B, const bf16_t* gain,
                                                 float eps, RowFn rowp, OutFn out, const Lds& s, bool tr) {
    const int nsw = (K / 1024 + kWaves - 1) / kWaves;
    if (nsw <= 1) gemv_w4<NB, 1, 2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr);
    else if (nsw <= 2) gemv_w4<NB, 2, 2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr);
    else gemv_w4<NB, 3, 1, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr);
}

// segments per wave per row of the B <= 2 GEMV for K inputs of type WT
// (the template instance gemv_dispatch picks; the preload uses the same)
template <typename WT>
__host__ __device__ constexpr int ksplit_nsw(int K) {
    constexpr int SEG = 64 * (16 / (int)sizeof(WT));
    const int n = ((K + SEG - 1) / SEG + kWaves - 1) / kWaves;
    return n <= 4 ? (n < 1 ? 1 : n) : (n <= 6 ? 6 : 8);
}

template <typename WT, int NB, bool DUAL, typename RowFn, typename OutFn>
__device__ __forceinline__ void gemv_dispatch(int r0, int r1, int K, const float* x, int ldx, int B, const WT* gain,
                                              float eps, RowFn rowp, OutFn out, const Lds& s, bool tr,
                                              int pre_rows = 0) {
    if constexpr (NB <= 2) {
        constexpr int D2 = DUAL ? 2 : 1;
        const int nsw = ksplit_nsw<WT>(K);
        // rows per group: small groups keep the fully unrolled loop short,
        // which measured faster than deeper groups for every task size here
        // (instruction fetch and fixed latencies dominate short tasks; the
        // stream of a long task is bound by HBM either way)
        if (nsw <= 1) gemv_ksplit<WT, NB, 1, 16 / D2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
        else if (nsw <= 2) gemv_ksplit<WT, NB, 2, 2 / D2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
        else if (nsw <= 3) gemv_ksplit<WT, NB, 3, 5 / D2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
        else if (nsw <= 4) gemv_ksplit<WT, NB, 4, 4 / D2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
        else if (nsw <= 6) gemv_ksplit<WT, NB, 6, 1, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
        else gemv_ksplit<WT, NB, 8, 2 / D2, DUAL>(r0, r1, K, x, ldx, B, gain, eps, rowp, out, s, tr, pre_rows);
    } else {
        if (gain) block_rstd<NB>(x, ldx, K, B, eps, s);
        gemv_rowwave<WT, NB, DUAL>(r0, r1, K, x, ldx, B, gain, rowp, out);
    }
}

// Buffer resource over rows [lo, hi) of a row-major matrix with K columns
// (rows clipped to [0, rows)); row r is at byte (r - lo) * K * es.
template <typename WT>
struct MatTile {
    __amdgpu_buffer_rsrc_t r;
    int lo, n;
    uint32_t rowbytes;
    __device__ __forceinline__ MatTile(const WT* m, int K, int rows, int lo_, int hi_) {
        lo = max(0, min(lo_, rows));
        const int hi = max(lo, min(hi_, rows));
        n = hi - lo;
        rowbytes = (uint32_t)K * (uint32_t)sizeof(WT);
        r = make_rsrc(m + (int64_t)lo * K, (uint32_t)(hi - lo) * rowbytes);
    }
    __device__ __forceinline__ void row(int rr, RowRef& o) const {
        o.r = r;
        o.soff = (uint32_t)(rr - lo) * rowbytes;
    }
};

// ---------------------------------------------------------------- GEMV on MFMA (bf16, B >= 3)
// With a batch of several sequences the GEMV is a thin matrix product
// Y[r][b] = sum_k W[r][k] xg[b][k] (xg = x * norm gain), done here on the
// 16x16x32 bf16 matrix cores: a 16-row weight tile is the A operand (lane
// l holds 8 consecutive k of row l % 16), the batch is the N dimension
// (lane l holds the same 8 k of sequence l % 16). The fp32 activations are
// split into two bf16 terms, xg = hi + lo with lo = bf16(xg - hi), and both
// are multiplied, so the product keeps about 16 significant bits of xg
// (relative error ~2^-17) instead of bf16's 8.
// K is cut into 64-k blocks dealt to the waves round-robin (block j to wave
// j % 4); a block is two MFMA k-steps, so every weight row is read in whole
// 128-byte lines, and each wave loads and converts only its own x values:
// no LDS staging and no barrier inside the loop. Weights and x of the next
// block are in flight while the current one is multiplied. The four waves'
// partial tiles are added in wave order through LDS. A task's rows are
// taken in passes of TMAX tiles; rows past a run and k past K load through
// an out-of-range offset (zeros, no traffic).
typedef __bf16 mk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mk_f32x4 __attribute__((ext_vector_type(4)));

// one run of output rows backed by one matrix (two for gate/up)
struct MSeg {
    __amdgpu_buffer_rsrc_t a, b;  // rows [0, n) of the matrix (matrices); W4: their codes
    int n;                        // rows in the run
    int out0;                     // output row of the run's first row
    __amdgpu_buffer_rsrc_t sa, sb;  // W4: the rows' group scales (bf16 [n][K / 128])
};

__device__ __forceinline__ mk_f32x4 mfma_bf16(const uint4& a, const mk_bf16x8& b, mk_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mk_bf16x8, a), b, c, 0, 0, 0);
}

// W4M: the matrices are W4 buffers (codes two per byte, offset 8, and bf16
// scales per 128 inputs). A lane's 8 codes of a k-step become the exact bf16
// values code - 8 for the A operand; a block's two k-steps (64 inputs, one
// scale group) are multiplied into a fresh tile, which is then scaled row by
// row (the scales staged in LDS per pass) and added to the accumulator. (Codes
// as 128 + code, one byte permute per pair, with 136 times the sum of x taken
// off afterwards, measured 10x the error: the matrix cores add the large
// partial sums less exactly.)
// TL: the matrices are in the tiled layout (MK_WEIGHTS_TILED): row 8u + i,
// column 32 s + 8 j + e of a run at u * 8 * K + s * 256 + (8 j + i) * 8 + e,
// so the 16 lanes (row, group j) of a load read 256 consecutive bytes and
// the whole load two 512-byte runs; the operands, and so the bits, are the
// row-major path's.
template <int NB, bool DUAL, int TMAX, int NSEG, typename OutFn, int NST = 2, bool W4M = false, bool TL = false>
// kofs, kfull (K split): the K columns run from kofs, in rows of kfull
// columns (0: K); x points at column kofs of its rows.
__device__ __forceinline__ void gemv_mfma(const MSeg (&seg)[NSEG], int K, const float* x, int ldx, int B,
                                          const bf16_t* gain, float eps, OutFn out, const Lds& s, bool tr,
                                          int kofs = 0, int kfull = 0) {
    constexpr int NM = DUAL ? 2 : 1;
    static_assert(kWaves * TMAX * NM * 256 <= kPartFloats, "partial tiles exceed the LDS window");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int krow = kfull > 0 ? kfull : K;  // columns per weight row
    const uint32_t rowbytes = W4M ? (uint32_t)krow / 2u : (uint32_t)krow * 2u;  // bytes per weight row (codes for W4)
    const uint32_t srow = (uint32_t)(K / kW4Group) * 2u;                  // W4: scale bytes per row
    const int ngroups = K / kW4Group;
    float* scs = s.part + kPartFloats;  // W4: [TMAX][NM][16 rows][ngroups] scales of the pass
    const int nblk = (K + 63) >> 6;
    const int nmine = (nblk - wave + kWaves - 1) / kWaves;  // blocks of this wave
    const __amdgpu_buffer_rsrc_t xr_rs = make_rsrc(x, (uint32_t)(B * ldx) * 4u);
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(gain, gain ? (uint32_t)K * 2u : 0u);
    const bool bok = li < B;

    int ntile = 0;
#pragma unroll
    for (int q = 0; q < NSEG; ++q) ntile += (seg[q].n + 15) >> 4;

    float ss = 0.f;  // sum of x^2 over this lane's (sequence li, k) values
    for (int t0 = 0; t0 < ntile; t0 += TMAX) {
        // this pass's tile table (uniform): resources, row offset, valid rows, output row
        __amdgpu_buffer_rsrc_t ta[TMAX], tb[TMAX], tsa[TMAX], tsb[TMAX];
        uint32_t tsoff[TMAX], tsoffs[TMAX];
        int tval[TMAX], tout[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            // run q holding task tile t0 + t, and the tile's index gt in it
            int gt = t0 + t, q = NSEG;
#pragma unroll
            for (int qq = 0; qq < NSEG; ++qq) {
                const int nt = (seg[qq].n + 15) >> 4;
                if (q == NSEG) {
                    if (gt < nt) q = qq;
                    else gt -= nt;
                }
            }
            ta[t] = seg[0].a;
            tb[t] = seg[0].b;
            tsa[t] = seg[0].sa;
            tsb[t] = seg[0].sb;
            tsoff[t] = tsoffs[t] = 0;
            tval[t] = 0;
            tout[t] = 0;
#pragma unroll
            for (int qq = 0; qq < NSEG; ++qq)
                if (q == qq) {
                    ta[t] = seg[qq].a;
                    tb[t] = seg[qq].b;
                    tsa[t] = seg[qq].sa;
                    tsb[t] = seg[qq].sb;
                    tsoff[t] = (uint32_t)(gt * 16) * rowbytes;
                    tsoffs[t] = (uint32_t)(gt * 16) * srow;
                    tval[t] = min(16, seg[qq].n - gt * 16);
                    tout[t] = seg[qq].out0 + gt * 16;
                }
        }
        if constexpr (W4M) {
            // the pass's scales as floats (rows past the run: 0); read after
            // the barrier, rewritten only after the pass's closing barrier
#pragma unroll
            for (int t = 0; t < TMAX; ++t)
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    for (int i = tid; i < 16 * ngroups; i += kThreads) {
                        const int row = i / ngroups, g = i % ngroups;
                        float v = 0.f;
                        if (t0 + t < ntile && row < tval[t]) {
                            const uint32_t h = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                m == 0 ? tsa[t] : tsb[t], (uint32_t)row * srow + (uint32_t)g * 2u, tsoffs[t], 0);
                            v = __uint_as_float(h << 16);
                        }
                        scs[((t * NM + m) * 16 + row) * ngroups + g] = v;
                    }
            __syncthreads();
        }
        struct Stage {
            uint4 w[TMAX][NM][2];
            uint32_t q[TMAX][NM][2];  // W4: 8 codes of the lane's k-step
            uint4 x[2][2];
            uint4 g[2];
            int blk;
        };
        // block i of this wave: k = 64 * (wave + 4 i) + 32 c + 8 lk
        auto load = [&](Stage& st, int i) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int k = ((wave + kWaves * i) << 6) + c * 32 + lk * 8;
                const bool kok = k < K && i < nmine;
                const uint32_t xo = (kok && bok) ? (uint32_t)(li * ldx + k) * 4u : kOOB;
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    if constexpr (W4M) {
                        const uint32_t vo = (kok && li < tval[t]) ? (uint32_t)li * rowbytes + (uint32_t)k / 2u : kOOB;
                        st.q[t][0][c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ta[t], vo, tsoff[t], kStreamAux);
                        if constexpr (DUAL) st.q[t][1][c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(tb[t], vo, tsoff[t], kStreamAux);
                    } else if constexpr (TL) {
                        const uint32_t vo = (kok && li < tval[t])
                                                ? (uint32_t)(li >> 3) * 8u * rowbytes + (uint32_t)((kofs + k) >> 5) * 512u +
                                                      (uint32_t)((lk << 3) | (li & 7)) * 16u
                                                : kOOB;
                        st.w[t][0][c] = buf_load16_wt(ta[t], vo, tsoff[t]);
                        if constexpr (DUAL) st.w[t][1][c] = buf_load16_wt(tb[t], vo, tsoff[t]);
                    } else {
                        const uint32_t vo = (kok && li < tval[t]) ? (uint32_t)li * rowbytes + (uint32_t)(kofs + k) * 2u : kOOB;
                        st.w[t][0][c] = buf_load16_w(ta[t], vo, tsoff[t]);
                        if constexpr (DUAL) st.w[t][1][c] = buf_load16_w(tb[t], vo, tsoff[t]);
                    }
                }
                st.x[c][0] = buf_load16_act(xr_rs, xo, 0);
                st.x[c][1] = buf_load16_act(xr_rs, xo, 16);
                st.g[c] = buf_load16(g_rs, kok ? (uint32_t)k * 2u : kOOB, 0);
            }
            st.blk = i;
        };
        mk_f32x4 acc[TMAX][NM];
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[t][m] = mk_f32x4{0.f, 0.f, 0.f, 0.f};
        const bool stat = gain != nullptr && t0 == 0;
        // k-step c of x (times the gain) as hi + lo bf16 terms, with hardware
        // round-to-nearest-even conversions (v_cvt_pk_bf16_f32)
        auto split = [&](const Stage& st, int c, mk_bf16x8& hi, mk_bf16x8& lo) {
            float xv[8], gv[8];
            xv[0] = __uint_as_float(st.x[c][0].x); xv[1] = __uint_as_float(st.x[c][0].y);
            xv[2] = __uint_as_float(st.x[c][0].z); xv[3] = __uint_as_float(st.x[c][0].w);
            xv[4] = __uint_as_float(st.x[c][1].x); xv[5] = __uint_as_float(st.x[c][1].y);
            xv[6] = __uint_as_float(st.x[c][1].z); xv[7] = __uint_as_float(st.x[c][1].w);
            if (gain) Vec16<bf16_t>::widen(st.g[c], gv);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) gv[e] = 1.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (stat) ss += xv[e] * xv[e];
                const float a = xv[e] * gv[e];
                const __bf16 h = (__bf16)a;
                hi[e] = h;
                lo[e] = (__bf16)(a - (float)h);
            }
        };
        auto compute = [&](const Stage& st) {
            if constexpr (W4M) {
                mk_bf16x8 hi[2], lo[2];
                split(st, 0, hi[0], lo[0]);
                split(st, 1, hi[1], lo[1]);
                // the block's 64 inputs share scale group (64 (wave + 4 blk)) / 128;
                // lane l's tile rows are 4 (l / 16) + r. One tile at a time: its
                // two k-steps into a fresh product, then scaled into the accumulator
                const int g = (wave + kWaves * st.blk) >> 1;
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    if (t0 + t >= ntile) continue;
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        mk_f32x4 tp = mk_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            // code e of the lane sits in bits 4e .. 4e + 3 (low nibble first);
                            // with its top bit flipped, the nibble read as a signed 4-bit
                            // field is code - 8, which bf16 holds exactly
                            const uint32_t q = st.q[t][m][c] ^ 0x88888888u;
                            mk_bf16x8 aq;
#pragma unroll
                            for (int e = 0; e < 8; ++e) aq[e] = (__bf16)(float)((int)(q << (28 - 4 * e)) >> 28);
                            tp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, hi[c], tp, 0, 0, 0);
                            tp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, lo[c], tp, 0, 0, 0);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[t][m][r] = fmaf(scs[((t * NM + m) * 16 + 4 * lk + r) * ngroups + g], tp[r], acc[t][m][r]);
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    mk_bf16x8 hi, lo;
                    split(st, c, hi, lo);
#pragma unroll
                    for (int t = 0; t < TMAX; ++t) {
                        if (t0 + t >= ntile) continue;
#pragma unroll
                        for (int m = 0; m < NM; ++m) {
                            acc[t][m] = mfma_bf16(st.w[t][m][c], hi, acc[t][m]);
                            acc[t][m] = mfma_bf16(st.w[t][m][c], lo, acc[t][m]);
                        }
                    }
                }
            }
        };
        if constexpr (NST == 2) {
            Stage sa, sb;
            load(sa, 0);
            if (tr && tid == 0 && t0 == 0) s.marks[0] = now_ticks();
            for (int i = 0; i < nmine; i += 2) {
                load(sb, i + 1);
                compute(sa);
                load(sa, i + 2);
                if (i + 1 < nmine) compute(sb);
            }
        } else {
            // three stages: two blocks in flight while one is multiplied
            Stage sa, sb, sc;
            load(sa, 0);
            load(sb, 1);
            if (tr && tid == 0 && t0 == 0) s.marks[0] = now_ticks();
            for (int i = 0; i < nmine; i += 3) {
                load(sc, i + 2);
                compute(sa);
                load(sa, i + 3);
                if (i + 1 < nmine) compute(sb);
                load(sb, i + 4);
                if (i + 2 < nmine) compute(sc);
            }
        }
        if (stat) {
            // norm statistic: lanes b, b+16, b+32, b+48 of each wave, then waves in order
            ss = column_sum<16>(ss);
            if (lane < 16) s.red[wave * 16 + lane] = ss;
        }
        // partial tiles: D layout, lane l holds rows 4*(l/16)+r of sequence l % 16
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
#pragma unroll
            for (int m = 0; m < NM; ++m)
                if (t0 + t < ntile)
                    *reinterpret_cast<mk_f32x4*>(&s.part[((wave * TMAX + t) * NM + m) * 256 + lane * 4]) = acc[t][m];
        __syncthreads();
        if (stat && tid < 16) {
            float tt = s.red[tid];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) tt += s.red[w * 16 + tid];
            s.rstd[tid] = 1.0f / sqrtf(tt / (float)K + eps);
        }
        if (tr && tid == 0) s.marks[1] = now_ticks();
        __syncthreads();
        {
            // row in tile, sequence: 16 consecutive lanes store 16 consecutive
            // rows of one sequence, so their 4-byte stores merge into one write
            const int i = tid & 15, b = tid >> 4;
            const int pl = ((i >> 2) * 16 + b) * 4 + (i & 3);
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t0 + t >= ntile) continue;
                float v[NM];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float a = s.part[(t * NM + m) * 256 + pl];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) a += s.part[((w * TMAX + t) * NM + m) * 256 + pl];
                    v[m] = a;
                }
                if (i < tval[t] && b < B) out(tout[t] + i, b, v[0], v[NM - 1]);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- GEMV tasks

// x_0[b, r] = E[token_b, r] for rows [a0, a1) (token ids outside the
// vocabulary raise MK_ERR_TOKEN and read row 0)
template <typename WT>
__device__ __forceinline__ void embed_task(const KParams& p, const TaskRec& t) {
    const WT* E = (const WT*)p.embed;
    const int H = p.H, B = p.B, r0 = t.a0, n = t.a1 - t.a0;
    for (int i = threadIdx.x; i < n * B; i += kThreads) {
        const int b = i / n, r = r0 + i % n;
        int tok = p.tokens[b];
        if (tok < 0 || tok >= p.V) {
            if (r == r0) raise_error(p.ctrl, MK_ERR_TOKEN);
            tok = 0;
        }
        st_co(&p.x0_w[(int64_t)b * H + r], load_scalar<WT>(E, (int64_t)tok * H + r));
    }
}

// ---------------------------------------------------------------- greedy step

// Orderable key of logit v at vocabulary index i: a larger value wins, and
// on equal values the lower index (-0 counts as +0; NaN is never passed).
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
}

// Greedy step, end: turn each sequence's argmax key into its next token,
// reset the key and advance the sequence's length; step `step` of a
// multi-step launch also records the tokens in out_tokens. Runs once per
// step, on one thread, after every reader of the step's lengths has
// finished. Agent-coherent stores: the next step of the same launch reads
// tokens and lengths on other CUs.
__device__ __forceinline__ void greedy_finish(const KParams& p, int step) {
    for (int b = 0; b < p.B; ++b) {
        const unsigned long long k = __hip_atomic_exchange(&p.amax[b], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int32_t tok = k ? (int32_t)(0xFFFFFFFFu - (uint32_t)k) : 0;
        st_co(&p.greedy_tokens[b], tok);
        st_co(&p.greedy_lens[b], __hip_atomic_load(&p.greedy_lens[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1);
        if (p.out_tokens) p.out_tokens[(int64_t)step * p.B + b] = tok;
    }
}

// Greedy step, after an LM-head task has stored logit rows [r0, r1): fold
// them into each sequence's argmax key (same choice as k_argmax). The keys
// become tokens in greedy_finish, called when the lengths have no reader
// left: in the persistent kernel by the last worker to leave its queue (an
// AOT attention slot that the step leaves empty still reads the lengths,
// and a worker holding one may come late), in kernel-per-op mode by the last
// LM-head task (every earlier launch has ended by then).
__device__ __forceinline__ void lm_greedy(const KParams& p, int r0, int r1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    wait_stores();
    __syncthreads();
    // wave w folds sequences w, w + 4, ... (no workgroup barrier per sequence)
    for (int b = wave; b < p.B; b += kWaves) {
        const float* row = p.logits + (int64_t)b * p.V;
        unsigned long long k = 0;  // 0: no candidate (all NaN)
        for (int c = r0; c < r1; c += 16 * 64) {
            // all of a lane's loads of the chunk are in flight together
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = c + 64 * i + lane;
                v[i] = r < r1 ? row[r] : __builtin_nanf("");
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (v[i] == v[i]) k = max(k, argmax_key(v[i], c + 64 * i + lane));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) k = max(k, (unsigned long long)__shfl_xor((long long)k, o, 64));
        if (lane == 0 && k) __hip_atomic_fetch_max(&p.amax[b], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_stores();  // the maxima are performed before this task counts as done
    __syncthreads();
    if (p.persistent || tid != 0) return;
    const uint32_t old = __hip_atomic_fetch_add(p.lm_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u != (uint32_t)p.n_lm_tasks) return;
    greedy_finish(p, 0);
    __hip_atomic_store(p.lm_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Element offset of (layer l, sequence b, KV head g, position pos) in the
// cache, or -1 for a paged position whose block-table entry lies outside
// the pool (the entry is the caller's data: it is checked, not trusted).
__device__ __forceinline__ int64_t kv_offset(const KParams& p, int l, int b, int g, int pos) {
    if (p.prefill) b = 0;  // prefill plans: every row is a position of sequence 0
    if (!p.paged) return (int64_t)l * p.kv_layer_stride + ((int64_t)(b * p.Hkv + g) * p.cap + pos) * p.D;
    const int blk = p.block_table[(int64_t)b * p.max_blocks + pos / p.kv_block];
    if ((unsigned)blk >= (unsigned)p.n_pool_blocks) return -1;
    return (int64_t)l * p.kv_layer_stride + ((int64_t)blk * p.Hkv + g) * p.kv_block * p.D + (int64_t)(pos % p.kv_block) * p.D;
}

// RMSNorm over one head (D = 64 or 128) held by a wave as D/64 values per
// lane (element j in lane j % 64, slot j / 64), then rotate-half RoPE. The
// gains g (same slots) and this lane's (cos, sin) are loaded by the caller
// ahead of time.
template <int D>
__device__ __forceinline__ void head_norm_rope(float (&v)[2], const float (&g)[2], bool norm, float eps, float2 cs) {
    const int lane = threadIdx.x & 63;
    constexpr int per = D / 64;
    if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < per; ++i) ss += v[i] * v[i];
        ss = wave_sum(ss);
        const float rs = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
        for (int i = 0; i < per; ++i) v[i] = (v[i] * rs) * g[i];
    }
    if constexpr (per == 2) {
        // pair (lane, lane + 64) sits in one lane
        const float a = v[0], b = v[1];
        v[0] = a * cs.x - b * cs.y;
        v[1] = b * cs.x + a * cs.y;
    } else {
        // D = 64: pair (i, i + 32) spans lanes i and i + 32
        const float other = halves_partner(v[0]);
        if (lane < 32) v[0] = v[0] * cs.x - other * cs.y;
        else v[0] = v[0] * cs.x + other * cs.y;
    }
}

// Prefill plans: rows [a0, a1) of the append level, each (b, g) = (row of
// the chunk, KV head): the new key (QK-norm, RoPE at seq_lens[b]) and value,
// rounded to the cache type, stored at position seq_lens[b] of sequence 0
// with agent-coherent stores (the attention level reads them on other CUs).
// One wave per (b, g).
template <typename WT, int D>
__device__ __forceinline__ void append_rows(const KParams& p, const TaskRec& t, const LayerPtrs& w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l = t.layer;
    for (int bg = t.a0 + wave; bg < t.a1; bg += kWaves) {
        const int b = bg / p.Hkv, g = bg % p.Hkv;
        const int pos = p.seq_lens[b];
        if (pos < 0 || pos + 1 > p.cap) continue;  // its attention task reports the overflow
        const float* qkv = layer_buf(p, l, p.off_qkv) + (int64_t)b * (p.QD + 2 * p.KD);
        float k[2] = {0.f, 0.f}, v[2] = {0.f, 0.f}, gk[2] = {1.f, 1.f};
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            k[i] = ld_act(&qkv[(int64_t)p.QD + g * D + lane + 64 * i]);
            v[i] = ld_act(&qkv[(int64_t)p.QD + p.KD + g * D + lane + 64 * i]);
            if (p.qk_norm) gk[i] = load_scalar<WT>((const WT*)w.k_norm, lane + 64 * i);
        }
        const float2 cs = p.rope[(int64_t)pos * (D / 2) + (D == 128 ? lane : (lane & 31))];
        head_norm_rope<D>(k, gk, p.qk_norm != 0, p.eps, cs);
        const int64_t off = kv_offset(p, l, b, g, pos);
        if (off < 0) {
            if (lane == 0) raise_error(p.ctrl, MK_ERR_BLOCK_TABLE);
            continue;
        }
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            st_co(&((WT*)p.kv_k)[off + lane + 64 * i], from_float<WT>(k[i]));
            st_co(&((WT*)p.kv_v)[off + lane + 64 * i], from_float<WT>(v[i]));
        }
    }
}

// A GEMV task of a plan whose layer matrices are W4 (batch <= 2); the LM
// head and the embedding stay bf16 and take the ordinary path.
template <int NB>
__device__ __forceinline__ void run_w4_task(const KParams& p, const TaskRec& t, const Lds& s, const LayerPtrs& w) {
    const int l = t.layer, B = p.B, H = p.H, r0 = t.a0, r1 = t.a1;
    const bool tr = p.trace != nullptr;
    switch (t.op) {
        case OP_QKV: {
            const float* x = layer_in(p, l);
            const int QD = p.QD, KD = p.KD, ld = QD + 2 * KD;
            const W4Tile tq = w4_tile(w.wq, H, QD, r0, r1), tk = w4_tile(w.wk, H, KD, r0 - QD, r1 - QD),
                         tv = w4_tile(w.wv, H, KD, r0 - QD - KD, r1 - QD - KD);
            float* o = layer_buf(p, l, p.off_qkv);
            auto rowp = [&](int r, W4Tile& a, W4Tile& b2, int& rr) {
                if (r < QD) { a = tq; rr = r - tq.lo; }
                else if (r < QD + KD) { a = tk; rr = r - QD - tk.lo; }
                else { a = tv; rr = r - QD - KD - tv.lo; }
                b2 = a;
            };
            auto out = [&](int r, int b, float v, float) { st_co(&o[(int64_t)b * ld + r], v * s.rstd[b]); };
            gemv_w4_dispatch<NB, false>(r0, r1, H, x, H, B, (const bf16_t*)w.attn_norm, p.eps, rowp, out, s, tr);
            break;
        }
        case OP_O: {
            const float* a = layer_buf(p, l, p.off_attn);
            const float* xin = layer_in(p, l);
            float* o = layer_buf(p, l, p.off_xmid);
            const W4Tile to = w4_tile(w.wo, p.QD, H, r0, r1);
            auto rowp = [&](int r, W4Tile& a0, W4Tile& b2, int& rr) { a0 = b2 = to; rr = r - to.lo; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xin[i]) + v);
            };
            gemv_w4_dispatch<NB, false>(r0, r1, p.QD, a, p.QD, B, (const bf16_t*)nullptr, p.eps, rowp, out, s, tr);
            break;
        }
        case OP_GATEUP: {
            const float* x = layer_buf(p, l, p.off_xmid);
            float* o = layer_buf(p, l, p.off_h);
            const int F = p.F;
            const W4Tile tg = w4_tile(w.w_gate, H, F, r0, r1), tu = w4_tile(w.w_up, H, F, r0, r1);
            auto rowp = [&](int r, W4Tile& a0, W4Tile& b2, int& rr) { a0 = tg; b2 = tu; rr = r - tg.lo; };
            auto out = [&](int r, int b, float g, float u) {
                const float rs = s.rstd[b];
                const float gg = g * rs, uu = u * rs;
                st_co(&o[(int64_t)b * F + r], (gg / (1.0f + __expf(-gg))) * uu);
            };
            gemv_w4_dispatch<NB, true>(r0, r1, H, x, H, B, (const bf16_t*)w.mlp_norm, p.eps, rowp, out, s, tr);
            break;
        }
        case OP_DOWN: {
            const float* h = layer_buf(p, l, p.off_h);
            const float* xm = layer_buf(p, l, p.off_xmid);
            float* o = layer_out(p, l);
            const W4Tile td = w4_tile(w.w_down, p.F, H, r0, r1);
            auto rowp = [&](int r, W4Tile& a0, W4Tile& b2, int& rr) { a0 = b2 = td; rr = r - td.lo; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xm[i]) + v);
            };
            gemv_w4_dispatch<NB, false>(r0, r1, p.F, h, p.F, B, (const bf16_t*)nullptr, p.eps, rowp, out, s, tr);
            break;
        }
        default: break;
    }
    trace_mark(p, s.marks, 2);
}

// A GEMV task of a plan whose layer matrices are W4, batch >= 3: the
// matrix-core GEMV with the codes dequantized in registers (the same tiles,
// passes and outputs as the bf16 path).
template <int NB>
__device__ __forceinline__ void run_w4_mfma_task(const KParams& p, const TaskRec& t, const Lds& s, const LayerPtrs& w) {
    const int l = t.layer, B = p.B, H = p.H, r0 = t.a0, r1 = t.a1;
    const bool tr = p.trace != nullptr;
    switch (t.op) {
        case OP_QKV: {
            const float* x = layer_in(p, l);
            const int QD = p.QD, KD = p.KD, ld = QD + 2 * KD;
            const W4Tile tq = w4_tile(w.wq, H, QD, r0, r1), tk = w4_tile(w.wk, H, KD, r0 - QD, r1 - QD),
                         tv = w4_tile(w.wv, H, KD, r0 - QD - KD, r1 - QD - KD);
            float* o = layer_buf(p, l, p.off_qkv);
            auto out = [&](int r, int b, float v, float) { st_co(&o[(int64_t)b * ld + r], v * s.rstd[b]); };
            const MSeg sg[3] = {{tq.q, tq.q, tq.n, tq.lo, tq.sc, tq.sc},
                                {tk.q, tk.q, tk.n, QD + tk.lo, tk.sc, tk.sc},
                                {tv.q, tv.q, tv.n, QD + KD + tv.lo, tv.sc, tv.sc}};
            gemv_mfma<NB, false, 2, 3, decltype(out), 2, true>(sg, H, x, H, B, (const bf16_t*)w.attn_norm, p.eps, out, s, tr);
            break;
        }
        case OP_O: {
            const float* a = layer_buf(p, l, p.off_attn);
            const float* xin = layer_in(p, l);
            float* o = layer_buf(p, l, p.off_xmid);
            const int K = p.QD;
            const W4Tile to = w4_tile(w.wo, K, H, r0, r1);
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xin[i]) + v);
            };
            const MSeg sg[1] = {{to.q, to.q, to.n, to.lo, to.sc, to.sc}};
            gemv_mfma<NB, false, 1, 1, decltype(out), 3, true>(sg, K, a, K, B, (const bf16_t*)nullptr, p.eps, out, s, tr);
            break;
        }
        case OP_GATEUP: {
            const float* x = layer_buf(p, l, p.off_xmid);
            float* o = layer_buf(p, l, p.off_h);
            const int F = p.F;
            const W4Tile tg = w4_tile(w.w_gate, H, F, r0, r1), tu = w4_tile(w.w_up, H, F, r0, r1);
            auto out = [&](int r, int b, float g, float u) {
                const float rs = s.rstd[b];
                const float gg = g * rs, uu = u * rs;
                st_co(&o[(int64_t)b * F + r], (gg / (1.0f + __expf(-gg))) * uu);
            };
            const MSeg sg[1] = {{tg.q, tu.q, tg.n, tg.lo, tg.sc, tu.sc}};
            gemv_mfma<NB, true, 3, 1, decltype(out), 2, true>(sg, H, x, H, B, (const bf16_t*)w.mlp_norm, p.eps, out, s, tr);
            break;
        }
        case OP_DOWN: {
            const float* h = layer_buf(p, l, p.off_h);
            const float* xm = layer_buf(p, l, p.off_xmid);
            float* o = layer_out(p, l);
            const int F = p.F;
            const W4Tile td = w4_tile(w.w_down, F, H, r0, r1);
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xm[i]) + v);
            };
            const MSeg sg[1] = {{td.q, td.q, td.n, td.lo, td.sc, td.sc}};
            gemv_mfma<NB, false, 1, 1, decltype(out), 3, true>(sg, F, h, F, B, (const bf16_t*)nullptr, p.eps, out, s, tr);
            break;
        }
        default: break;
    }
    trace_mark(p, s.marks, 2);
}

// Pipeline stages of the matrix-core GEMV with tiled weights: QKV and
// gate/up (several tiles per pass), O and down (one tile per pass).
#ifndef MK_TILED_NST_QG
#define MK_TILED_NST_QG 2
#endif
#ifndef MK_TILED_NST_OD
#define MK_TILED_NST_OD 3
#endif
// Runs f(std::true_type) for a plan with tiled weights, else
// f(std::false_type). The W4 instances never see tiled weights (plans reject
// the combination), so they compile the row-major path only.
template <typename F>
__device__ __forceinline__ void mfma_dispatch(const KParams& p, F f) {
    if constexpr (!kW4MfmaKernels) {
        if (p.wtiled) {
            f(std::true_type{});
            return;
        }
    }
    f(std::false_type{});
}

// One K part of a K-split O or down projection (matrix-core path): rows
// [a0, a1) over columns [kp K / ks, (kp + 1) K / ks) of the input, into the
// row group's partial tile; the last part of the group to arrive adds the ks
// partials in part order, adds the residual and stores the rows (the
// combine rule of the split attention: a fixed order, whatever the arrival
// order). Returns whether this task signals the event (the merging part
// only). Partial layout: group at p.kpart + a0 * ks * 16, part kp at
// kp * (a1 - a0) * 16, row i at i * 16, one float per sequence.
template <int NB>
__device__ __forceinline__ bool run_ksplit(const KParams& p, const TaskRec& t, const Lds& s, const LayerPtrs& w) {
    const int kp = t.kpart & 0xFF, ks = t.kpart >> 8;
    const int l = t.layer, B = p.B, H = p.H, r0 = t.a0, r1 = t.a1, nr = r1 - r0;
    const bool down = t.op == OP_DOWN;
    const int K = down ? p.F : p.QD;
    const int kw = K / ks, k0 = kp * kw;
    float* part = p.kpart + (int64_t)r0 * ks * 16;
    const MatTile<bf16_t> td((const bf16_t*)(down ? w.w_down : w.wo), K, H, r0, r1);
    auto out = [&](int r, int b, float v, float) { st_co(&part[((int64_t)kp * nr + (r - r0)) * 16 + b], v); };
    const MSeg sg[1] = {{td.r, td.r, td.n, td.lo}};
    const float* xin = layer_buf(p, l, down ? p.off_h : p.off_attn) + k0;
    mfma_dispatch(p, [&](auto tl) {
        gemv_mfma<NB, false, 4, 1, decltype(out), 2, false, decltype(tl)::value>(
            sg, kw, xin, K, B, (const bf16_t*)nullptr, p.eps, out, s, p.trace != nullptr, k0, K);
    });
    // arrival on the group's counter once this part's stores are complete
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.karrive[t.kgroup], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.cmd[9] = (old + 1u == (uint32_t)ks) ? 1 : 0;
    }
    __syncthreads();
    const bool last = s.cmd[9] != 0;
    __syncthreads();
    if (!last) return false;
    // merge: each thread takes 4 sequences of one row, all parts' loads in
    // flight together
    // residual: O adds to the layer input into x_mid, down to x_mid into the layer output
    const float* xm = down ? layer_buf(p, l, p.off_xmid) : layer_in(p, l);
    float* o = down ? layer_out(p, l) : layer_buf(p, l, p.off_xmid);
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(part, (uint32_t)(ks * nr * 16) * 4u);
    for (int e = threadIdx.x; e < nr * 4; e += kThreads) {
        const int i = e >> 2, b0 = (e & 3) * 4;
        if (b0 >= B) continue;
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = buf_load16_co(prs, q < ks ? (uint32_t)(((q * nr + i) * 16 + b0) * 4) : kOOB, 0);
        float acc[4] = {__uint_as_float(v[0].x), __uint_as_float(v[0].y), __uint_as_float(v[0].z), __uint_as_float(v[0].w)};
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            if (q >= ks) continue;
            acc[0] += __uint_as_float(v[q].x);
            acc[1] += __uint_as_float(v[q].y);
            acc[2] += __uint_as_float(v[q].z);
            acc[3] += __uint_as_float(v[q].w);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (b0 + j >= B) continue;
            const int64_t idx = (int64_t)(b0 + j) * H + r0 + i;
            st_co(&o[idx], ld_act(&xm[idx]) + acc[j]);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&p.karrive[t.kgroup], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// w: the task's layer pointers, p.lw[t.layer] (the worker reads them before
// the task's event fires). pre_rows: leading rows of the task whose weights
// were preloaded into this worker's LDS slots (batch <= 2 only; 0 otherwise).
// Returns whether the task signals its event (false only for the parts of a
// K-split group that do not merge it).
template <typename WT, int NB>
__device__ __forceinline__ bool run_gemv_task(const KParams& p, const TaskRec& t, const Lds& s, const LayerPtrs& w,
                                              int pre_rows = 0) {
    // 4-bit layer matrices: VALU GEMV at batch <= 2 (in the bf16 instances),
    // matrix cores above (in instances of their own: in the bf16 batch >= 4
    // kernels that code would cost registers, and spills, when unused)
    if constexpr (std::is_same<WT, bf16_t>::value && (NB <= 2 || kW4MfmaKernels)) {
        if (p.w4 && t.op != OP_LM && t.op != OP_EMBED && t.op != OP_APPEND) {
            if constexpr (NB <= 2) run_w4_task<NB>(p, t, s, w);
            else run_w4_mfma_task<NB>(p, t, s, w);
            return true;
        }
    }
    // bf16 weights with more than two sequences run on the matrix cores
    constexpr bool kMfma = std::is_same<WT, bf16_t>::value && NB >= 4;
    const int l = t.layer, B = p.B, H = p.H;
    const int r0 = t.a0, r1 = t.a1;
    switch (t.op) {
        case OP_EMBED: embed_task<WT>(p, t); break;
        case OP_APPEND:
            if (p.D == 128) append_rows<WT, 128>(p, t, w);
            else append_rows<WT, 64>(p, t, w);
            break;
        case OP_QKV: {
            const float* x = layer_in(p, l);
            const int QD = p.QD, KD = p.KD, ld = QD + 2 * KD;
            const MatTile<WT> tq((const WT*)w.wq, H, QD, r0, r1);
            const MatTile<WT> tk((const WT*)w.wk, H, KD, r0 - QD, r1 - QD);
            const MatTile<WT> tv((const WT*)w.wv, H, KD, r0 - QD - KD, r1 - QD - KD);
            float* o = layer_buf(p, l, p.off_qkv);
            auto rowp = [&](int r, RowRef& a, RowRef& b2) {
                if (r < QD) tq.row(r, a);
                else if (r < QD + KD) tk.row(r - QD, a);
                else tv.row(r - QD - KD, a);
                b2 = a;
            };
            auto out = [&](int r, int b, float v, float) { st_co(&o[(int64_t)b * ld + r], v * s.rstd[b]); };
            if constexpr (kMfma) {
                const MSeg sg[3] = {{tq.r, tq.r, tq.n, tq.lo}, {tk.r, tk.r, tk.n, QD + tk.lo}, {tv.r, tv.r, tv.n, QD + KD + tv.lo}};
                mfma_dispatch(p, [&](auto tl) {
                    gemv_mfma<NB, false, 2, 3, decltype(out), decltype(tl)::value ? MK_TILED_NST_QG : 2, false,
                              decltype(tl)::value>(
                        sg, H, x, H, B, (const bf16_t*)w.attn_norm, p.eps, out, s, p.trace != nullptr);
                });
            } else {
                gemv_dispatch<WT, NB, false>(r0, r1, H, x, H, B, (const WT*)w.attn_norm, p.eps, rowp, out, s, p.trace != nullptr, pre_rows);
            }
            break;
        }
        case OP_O: {
            if constexpr (kMfma && !kW4MfmaKernels)
                if (t.kpart >> 8 > 1) {
                    const bool sig = run_ksplit<NB>(p, t, s, w);
                    trace_mark(p, s.marks, 2);
                    return sig;
                }
            const float* a = layer_buf(p, l, p.off_attn);
            const float* xin = layer_in(p, l);
            float* o = layer_buf(p, l, p.off_xmid);
            const int K = p.QD;
            const MatTile<WT> to((const WT*)w.wo, K, H, r0, r1);
            auto rowp = [&](int r, RowRef& a0, RowRef& b2) { to.row(r, a0); b2 = a0; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xin[i]) + v);
            };
            if constexpr (kMfma) {
                const MSeg sg[1] = {{to.r, to.r, to.n, to.lo}};
                mfma_dispatch(p, [&](auto tl) {
                    gemv_mfma<NB, false, 1, 1, decltype(out), decltype(tl)::value ? MK_TILED_NST_OD : 3, false,
                              decltype(tl)::value>(
                        sg, K, a, K, B, (const bf16_t*)nullptr, p.eps, out, s, p.trace != nullptr);
                });
            } else {
                gemv_dispatch<WT, NB, false>(r0, r1, K, a, K, B, (const WT*)nullptr, p.eps, rowp, out, s, p.trace != nullptr, pre_rows);
            }
            break;
        }
        case OP_GATEUP: {
            const float* x = layer_buf(p, l, p.off_xmid);
            float* o = layer_buf(p, l, p.off_h);
            const int F = p.F;
            const MatTile<WT> tg((const WT*)w.w_gate, H, F, r0, r1);
            const MatTile<WT> tu((const WT*)w.w_up, H, F, r0, r1);
            auto rowp = [&](int r, RowRef& a0, RowRef& b2) {
                tg.row(r, a0);
                tu.row(r, b2);
            };
            auto out = [&](int r, int b, float g, float u) {
                const float rs = s.rstd[b];
                const float gg = g * rs, uu = u * rs;
                st_co(&o[(int64_t)b * F + r], (gg / (1.0f + __expf(-gg))) * uu);
            };
            if constexpr (kMfma) {
                const MSeg sg[1] = {{tg.r, tu.r, tg.n, tg.lo}};
                mfma_dispatch(p, [&](auto tl) {
                    gemv_mfma<NB, true, 3, 1, decltype(out), decltype(tl)::value ? MK_TILED_NST_QG : 2, false,
                              decltype(tl)::value>(
                        sg, H, x, H, B, (const bf16_t*)w.mlp_norm, p.eps, out, s, p.trace != nullptr);
                });
            } else {
                gemv_dispatch<WT, NB, true>(r0, r1, H, x, H, B, (const WT*)w.mlp_norm, p.eps, rowp, out, s, p.trace != nullptr, pre_rows);
            }
            break;
        }
        case OP_DOWN: {
            if constexpr (kMfma && !kW4MfmaKernels)
                if (t.kpart >> 8 > 1) {
                    const bool sig = run_ksplit<NB>(p, t, s, w);
                    trace_mark(p, s.marks, 2);
                    return sig;
                }
            const float* h = layer_buf(p, l, p.off_h);
            const float* xm = layer_buf(p, l, p.off_xmid);
            float* o = layer_out(p, l);
            const int F = p.F;
            const MatTile<WT> td((const WT*)w.w_down, F, H, r0, r1);
            auto rowp = [&](int r, RowRef& a0, RowRef& b2) { td.row(r, a0); b2 = a0; };
            auto out = [&](int r, int b, float v, float) {
                const int64_t i = (int64_t)b * H + r;
                st_co(&o[i], ld_act(&xm[i]) + v);
            };
            if constexpr (kMfma) {
                const MSeg sg[1] = {{td.r, td.r, td.n, td.lo}};
                mfma_dispatch(p, [&](auto tl) {
                    gemv_mfma<NB, false, 1, 1, decltype(out), decltype(tl)::value ? MK_TILED_NST_OD : 3, false,
                              decltype(tl)::value>(
                        sg, F, h, F, B, (const bf16_t*)nullptr, p.eps, out, s, p.trace != nullptr);
                });
            } else {
                gemv_dispatch<WT, NB, false>(r0, r1, F, h, F, B, (const WT*)nullptr, p.eps, rowp, out, s, p.trace != nullptr, pre_rows);
            }
            break;
        }
        case OP_LM: {
            const float* x = p.x_final;
            float* o = p.logits;
            const int V = p.V;
            const MatTile<WT> tl((const WT*)p.lm_head, H, V, r0, r1);
            auto rowp = [&](int r, RowRef& a0, RowRef& b2) { tl.row(r, a0); b2 = a0; };
            auto out = [&](int r, int b, float v, float) { o[(int64_t)b * V + r] = v * s.rstd[b]; };  // read after the launch
            if constexpr (kMfma) {
                const MSeg sg[1] = {{tl.r, tl.r, tl.n, tl.lo}};
                mfma_dispatch(p, [&](auto tl) {
                    gemv_mfma<NB, false, 8, 1, decltype(out), 2, false, decltype(tl)::value>(
                        sg, H, x, H, B, (const bf16_t*)p.final_norm, p.eps, out, s, p.trace != nullptr);
                });
            } else {
                gemv_dispatch<WT, NB, false>(r0, r1, H, x, H, B, (const WT*)p.final_norm, p.eps, rowp, out, s, p.trace != nullptr, pre_rows);
            }
            if (p.greedy_tokens) lm_greedy(p, r0, r1);
            break;
        }
        default: break;
    }
    trace_mark(p, s.marks, 2);
    return true;
}

// ---------------------------------------------------------------- signalling

// Make this workgroup's writes visible device-wide, then count one
// arrival on event e (MPK article §2.1: trigger_count / required_count), in
// partial-count plane `plane` (below the waiters' plane count).
// The arrival that completes a JIT-triggering event posts a message to the
// scheduler mailbox (§2.2: the data-dependent successor is launched JIT).
// Expand layer `layer`'s JIT attention tasks (b, g, split) for every
// sequence, in sequence order, from seq_lens and the step's split length,
// and deal task i to eligible worker (start + i) mod n_elig's inbox (the
// MPK article, §2.2). `lane` of `nlanes` cooperating threads takes tasks
// lane, lane + nlanes, ...; `start` continues the previous expansion's
// round-robin position (the caller reserved `total` positions).
__device__ __forceinline__ int jit_total(const KParams& p, int chunk) {
    int total = 0;
    for (int b = 0; b < p.B; ++b) {
        const int pos = p.seq_lens[b];
        const bool ovf = pos < 0 || pos + 1 > p.cap;
        total += (ovf ? 1 : (pos + 1 + chunk - 1) / chunk) * p.Hkv;
    }
    return total;
}
__device__ __forceinline__ void jit_expand(const KParams& p, int layer, int chunk, int total, int64_t start, int lane,
                                           int nlanes) {
    for (int i = lane; i < total; i += nlanes) {
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

// signal_event of a GEMV task in a plan whose JIT attention is expanded by
// the completing QKV arrival (batch >= 8 instances, all threads): the
// arrival that completes a QKV event then expands that layer's attention
// tasks into the inboxes with the whole workgroup.
__device__ __forceinline__ void signal_gemv_jit_inline(const KParams& p, int e, const Lds& s, int plane) {
    wait_stores();  // this thread's agent-coherent stores have completed
    trace_mark(p, s.marks, 3);
    __syncthreads();
    if (threadIdx.x == 0) {
        int expand = 0;
        if (e >= 0) {
            const EventRec er = p.evrec[e];
            if (er.jit_layer < 0) {
                __hip_atomic_fetch_add(&p.ev[plane * p.ev_stride + e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                // the completing arrival must see the whole count: plane 0 only
                const uint32_t old = __hip_atomic_fetch_add(&p.ev[e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (old + 1u == er.required * (p.epoch + 1u)) expand = er.jit_layer + 1;
            }
        }
        s.cmd[14] = expand;
    }
    __syncthreads();
    const int jl = s.cmd[14] - 1;
    if (jl < 0) return;  // uniform: read after the barrier
    // every wave finds the split length; the whole workgroup deals the
    // tasks, one per thread per round
    const int chunk = attn_chunk(p), total = jit_total(p, chunk);
    if (threadIdx.x == 0) {
        const int64_t st = __hip_atomic_fetch_add(&p.ctrl->rr, (int64_t)total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.cmd[10] = (int)(uint32_t)st;
        s.cmd[11] = (int)(uint32_t)((uint64_t)st >> 32);
    }
    __syncthreads();
    const int64_t start = (int64_t)(((uint64_t)(uint32_t)s.cmd[11] << 32) | (uint32_t)s.cmd[10]);
    jit_expand(p, jl, chunk, total, start, threadIdx.x, kThreads);
}

__device__ __forceinline__ void signal_event(const KParams& p, int e, const Lds& s, int plane = 0) {
    wait_stores();  // this thread's agent-coherent stores have completed
    trace_mark(p, s.marks, 3);
    __syncthreads();
    if (threadIdx.x == 0 && e >= 0) {
        const EventRec er = p.evrec[e];
        if (er.jit_layer < 0) {
            // no one acts on the count here: the add needs no return trip
            __hip_atomic_fetch_add(&p.ev[plane * p.ev_stride + e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // the completing arrival must see the whole count: plane 0 only
        const uint32_t old = __hip_atomic_fetch_add(&p.ev[e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1u == er.required * (p.epoch + 1u)) {
            // the completing arrival posts "expand attention of this layer"
            const int64_t pos = __hip_atomic_fetch_add(&p.ctrl->mb_tail, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            RingSlot* sl = &p.mb[pos & p.mb_mask];
            st_co(&sl->p0, er.jit_layer);
            st_co(&sl->p1, 0);
            wait_stores();
            __hip_atomic_store(&sl->tag, pos + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- LDS preload (batch <= 2 GEMV)
// While a worker waits for a GEMV task's event it copies the task's first
// rows into its LDS preload slots with direct-to-LDS loads: wave w issues
// exactly the loads its own part of the task would issue (row r, matrix m,
// segment j: 16 bytes per lane at k = (w + 4 j) * SEG + lane * E), one slot
// per load, in the task's order. The task then reads those rows from LDS.
// Whole rows only, so every wave preloads the same rows.
// The cursor of each wave lives in LDS (s.pst), not in registers: the
// worker loop holds little state across the large task bodies, and a
// cursor in registers spilled to scratch, whose reloads inside the poll
// loop would wait for every load in flight. Layout (ints): next, end, r, m,
// j, nm, nsw, nseg, K, rowbytes, lim0, lim1, then three 64-bit matrix bases
// (rows [0, lim0), [lim0, lim1), [lim1, ..); QKV q, k, v; gate/up: gate, up).
enum { PS_NEXT, PS_END, PS_R, PS_M, PS_J, PS_NM, PS_NSW, PS_NSEG, PS_K, PS_ROWB, PS_LIM0, PS_LIM1, PS_B0, PS_B1 = PS_B0 + 2,
       PS_B2 = PS_B1 + 2 };
static_assert(PS_B2 + 2 <= kPstInts, "preload cursor size");

__device__ __forceinline__ bool preload_op(int op) {
    return op == OP_QKV || op == OP_O || op == OP_GATEUP || op == OP_DOWN || op == OP_LM;
}

// inputs per row of a GEMV op's matrix
__device__ __forceinline__ int gemv_k(const KParams& p, int op) {
    return op == OP_O ? p.QD : (op == OP_DOWN ? p.F : p.H);
}

// rows of task t that the preload covers (0 if it does not apply: the plan
// sets pre_slots only for batch <= 2 with ahead-of-time queues)
template <typename WT>
__device__ __forceinline__ int preload_rows(const KParams& p, const TaskRec& t) {
    if (p.pre_slots <= 0 || !preload_op(t.op) || t.wait_ev < 0) return 0;
    const int nm = t.op == OP_GATEUP ? 2 : 1;
    const int per_row = nm * ksplit_nsw<WT>(gemv_k(p, t.op));
    return min(t.a1 - t.a0, p.pre_slots / per_row);
}

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char* ps_ptr(const int* st, int i) {
    const uint32_t lo = (uint32_t)rfl(st[i]), hi = (uint32_t)rfl(st[i + 1]);
    return (const char*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void ps_put_ptr(int* st, int i, const void* v) {
    st[i] = (int)(uint32_t)(uint64_t)v;
    st[i + 1] = (int)(uint32_t)((uint64_t)v >> 32);
}

// Set this wave's cursor for task t (an empty cursor for tasks the preload
// does not cover). Lane 0 writes; the wave reads it back in order.
template <typename WT>
__device__ __forceinline__ void preload_setup(const KParams& p, const TaskRec& t, const Lds& s) {
    const int wave = threadIdx.x >> 6;
    int* st = s.pst + wave * kPstInts;
    const int rows = preload_rows<WT>(p, t);
    if ((threadIdx.x & 63) != 0) return;
    st[PS_NEXT] = 0;
    if (rows <= 0) {
        st[PS_END] = 0;
        return;
    }
    const int K = gemv_k(p, t.op), nm = t.op == OP_GATEUP ? 2 : 1, nsw = ksplit_nsw<WT>(K);
    const uint32_t rowbytes = (uint32_t)K * (uint32_t)sizeof(WT);
    st[PS_END] = rows * nm * nsw;
    st[PS_R] = t.a0;
    st[PS_M] = 0;
    st[PS_J] = 0;
    st[PS_NM] = nm;
    st[PS_NSW] = nsw;
    st[PS_NSEG] = (K + 64 * Vec16<WT>::N - 1) / (64 * Vec16<WT>::N);
    st[PS_K] = K;
    st[PS_ROWB] = (int)rowbytes;
    st[PS_LIM0] = st[PS_LIM1] = 1 << 30;
    const LayerPtrs& w = p.lw[t.layer];
    const char *b0 = nullptr, *b1 = nullptr, *b2 = nullptr;
    switch (t.op) {
        case OP_QKV:
            b0 = (const char*)w.wq;
            b1 = (const char*)w.wk - (int64_t)p.QD * rowbytes;
            b2 = (const char*)w.wv - (int64_t)(p.QD + p.KD) * rowbytes;
            st[PS_LIM0] = p.QD;
            st[PS_LIM1] = p.QD + p.KD;
            break;
        case OP_O: b0 = (const char*)w.wo; break;
        case OP_GATEUP:
            b0 = (const char*)w.w_gate;
            b1 = (const char*)w.w_up;
            break;
        case OP_DOWN: b0 = (const char*)w.w_down; break;
        default: b0 = (const char*)p.lm_head; break;
    }
    ps_put_ptr(st, PS_B0, b0);
    ps_put_ptr(st, PS_B1, b1);
    ps_put_ptr(st, PS_B2, b2);
}

constexpr int kPreSlice = 6;  // slots per wave issued between two polls

template <typename WT>
__device__ __forceinline__ void preload_step(const Lds& s) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int* st = s.pst + wave * kPstInts;
    int next = rfl(st[PS_NEXT]);
    const int end = rfl(st[PS_END]);
    if (next >= end) return;
    constexpr int E = Vec16<WT>::N;
    int r = rfl(st[PS_R]), m = rfl(st[PS_M]), j = rfl(st[PS_J]);
    const int nm = rfl(st[PS_NM]), nsw = rfl(st[PS_NSW]), nseg = rfl(st[PS_NSEG]), K = rfl(st[PS_K]);
    const uint32_t rowbytes = (uint32_t)rfl(st[PS_ROWB]);
    const int lim0 = rfl(st[PS_LIM0]), lim1 = rfl(st[PS_LIM1]);
    const char *b0 = ps_ptr(st, PS_B0), *b1 = ps_ptr(st, PS_B1), *b2 = ps_ptr(st, PS_B2);
    uint4* slots = s.pre + wave * (kPreSlots * 64);
    for (int k = 0; k < kPreSlice && next < end; ++k) {
        const int seg = wave + kWaves * j;
        if (seg < nseg) {  // past the last segment the task loads zeros itself
            const int kk = seg * 64 * E + lane * E;
            const uint32_t voff = kk < K ? (uint32_t)kk * (uint32_t)sizeof(WT) : kOOB;
            // gate/up: matrix m; QKV: the matrix holding row r
            const char* b = nm == 2 ? (m ? b1 : b0) : (r < lim0 ? b0 : (r < lim1 ? b1 : b2));
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(b + (int64_t)r * rowbytes, rowbytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(slots + next * 64),
                                                     16, voff, 0, 0, 0);
        }
        next++;
        if (++j == nsw) {
            j = 0;
            if (++m == nm) {
                m = 0;
                r++;
            }
        }
    }
    if (lane == 0) {
        st[PS_NEXT] = next;
        st[PS_R] = r;
        st[PS_M] = m;
        st[PS_J] = j;
    }
}

// rows of the task whose slots every wave has issued
__device__ __forceinline__ int preload_done_rows(const Lds& s) {
    const int* st = s.pst + (threadIdx.x >> 6) * kPstInts;
    const int end = rfl(st[PS_END]);
    return end > 0 ? rfl(st[PS_NEXT]) / (rfl(st[PS_NM]) * rfl(st[PS_NSW])) : 0;
}

// ---------------------------------------------------------------- next-task prefetch
// The weights are static, so a worker can pull its next GEMV task's rows
// toward the chip before that task's event fires (the MPK article's
// preload phase, section 3.2): HBM stays busy across level boundaries and
// the task body's own loads then hit L2 or the memory-side cache. Loads go
// direct-to-LDS into a scratch slot that is never read, so they hold no
// registers. They are issued in slices (kPrefetchSlice KB per wave) between
// polls of the event, never as one burst, so that the poll loop is not held
// up by a full load queue.
__shared__ __attribute__((aligned(16))) uint4 mk_prefetch_sink[kWaves][64];
constexpr int kPrefetchSlice = 6;

struct Prefetch {
    __amdgpu_buffer_rsrc_t a, b;  // one or two weight segments (gate and up interleave)
    uint32_t kb_a, kb_b;          // segment sizes in KB (rounded up)
    uint32_t next, end;           // next KB index to issue, total KB to issue
    uint32_t chunk_kb, stride;    // strided segment a (K-split tasks): chunks of chunk_kb KB, stride bytes apart; 0: contiguous
};

__device__ __forceinline__ void prefetch_segment(const void* m, int K, int es, int rows, int r0, int r1,
                                                 __amdgpu_buffer_rsrc_t& rs, uint32_t& kb) {
    r0 = max(0, min(r0, rows));
    r1 = max(r0, min(r1, rows));
    const uint32_t bytes = (uint32_t)(r1 - r0) * (uint32_t)K * (uint32_t)es;
    rs = make_rsrc((const char*)m + (int64_t)r0 * K * es, bytes);
    kb = (bytes + 1023u) / 1024u;
}

// Cursor over the next task's weights (empty for attention / embedding or
// when prefetching is off).
template <typename WT>
__device__ __forceinline__ Prefetch prefetch_setup(const KParams& p, const TaskRec& t) {
    Prefetch f;
    f.kb_a = f.kb_b = 0;
    f.next = f.end = 0;
    f.chunk_kb = f.stride = 0;
    f.a = f.b = make_rsrc(p.zero, 0);
    if (p.prefetch_kb <= 0) return f;
#if defined(MK_NB) && MK_NB >= 4
    // K-split tasks exist on the matrix-core path only: the branch is left out
    // of the batch <= 2 instances (there it measured 1% slower at batch 1 even
    // though it never ran: it changes their register allocation)
    if ((t.op == OP_DOWN || t.op == OP_O) && (t.kpart >> 8) > 1) {
        // a K part of the O or down projection reads columns [k0, k0 + kw)
        // of its rows: per row kw * 2 bytes, F * 2 apart (row-major), or per
        // 8-row unit kw * 16 bytes, 16 F apart (tiled; F: the row length);
        // whole KB chunks only
        const int ks = t.kpart >> 8, kp = t.kpart & 0xFF, F = t.op == OP_DOWN ? p.F : p.QD;
        const int kw = F / ks, k0 = kp * kw, nr = t.a1 - t.a0;
        const char* m = (const char*)(t.op == OP_DOWN ? p.lw[t.layer].w_down : p.lw[t.layer].wo);
        uint32_t chunk, n;
        if (p.wtiled) {
            m += (int64_t)t.a0 * F * 2 + (int64_t)(k0 / 32) * 512;
            chunk = (uint32_t)kw * 16u;
            f.stride = (uint32_t)F * 16u;
            n = (uint32_t)(nr / 8);
        } else {
            m += ((int64_t)t.a0 * F + k0) * 2;
            chunk = (uint32_t)kw * 2u;
            f.stride = (uint32_t)F * 2u;
            n = (uint32_t)nr;
        }
        if (chunk % 1024u || n == 0) return f;
        f.chunk_kb = chunk / 1024u;
        f.a = make_rsrc(m, (n - 1) * f.stride + chunk);
        f.kb_a = n * f.chunk_kb;
        f.end = min(f.kb_a, (uint32_t)p.prefetch_kb);
        return f;
    }
#endif
    // a W4 layer matrix streams K / 2 bytes of codes per row (its scales,
    // 1/64 of that, are not prefetched): the same cursor with halved K
    const bool w4m = p.w4 && t.op != OP_LM && t.op != OP_EMBED;
    const int es = w4m ? 1 : (int)sizeof(WT), l = t.layer, H = p.H;
    const int kh = w4m ? p.H / 2 : p.H, kq = w4m ? p.QD / 2 : p.QD, kf = w4m ? p.F / 2 : p.F;  // row lengths in elements of size es
    switch (t.op) {
        case OP_QKV: {
            const LayerPtrs& w = p.lw[l];
            if (t.a0 < p.QD) prefetch_segment(w.wq, kh, es, p.QD, t.a0, t.a1, f.a, f.kb_a);
            else if (t.a0 < p.QD + p.KD) prefetch_segment(w.wk, kh, es, p.KD, t.a0 - p.QD, t.a1 - p.QD, f.a, f.kb_a);
            else prefetch_segment(w.wv, kh, es, p.KD, t.a0 - p.QD - p.KD, t.a1 - p.QD - p.KD, f.a, f.kb_a);
            break;
        }
        case OP_O: prefetch_segment(p.lw[l].wo, kq, es, H, t.a0, t.a1, f.a, f.kb_a); break;
        case OP_GATEUP:
            prefetch_segment(p.lw[l].w_gate, kh, es, p.F, t.a0, t.a1, f.a, f.kb_a);
            prefetch_segment(p.lw[l].w_up, kh, es, p.F, t.a0, t.a1, f.b, f.kb_b);
            break;
        case OP_DOWN: prefetch_segment(p.lw[l].w_down, kf, es, H, t.a0, t.a1, f.a, f.kb_a); break;
        case OP_LM: prefetch_segment(p.lm_head, H, es, p.V, t.a0, t.a1, f.a, f.kb_a); break;
        default: break;
    }
    f.end = min(f.kb_a + f.kb_b, (uint32_t)p.prefetch_kb);
    // rows going to the LDS preload slots are not pulled into L2 as well
    // (KB i of the stream is KB i/2 of segment i & 1 when there are two)
    const int lds_rows = preload_rows<WT>(p, t);
    if (lds_rows > 0) {
        const uint32_t kb = (uint32_t)lds_rows * (uint32_t)gemv_k(p, t.op) * (uint32_t)es / 1024u * (f.kb_b ? 2u : 1u);
        f.next = min(kb, f.end);
    }
    return f;
}

// Cursor over the cached K and V rows of an attention split (contiguous
// cache only): the rows before position pos are fixed for the step, so a slot
// can pull them toward the chip while it waits for the layer's QKV event.
// Row pos is appended by this step and never read from memory by it.
template <typename WT>
__device__ __forceinline__ Prefetch attn_prefetch_setup(const KParams& p, int l, int bg, int split, int C) {
    Prefetch f;
    f.kb_a = f.kb_b = 0;
    f.next = f.end = 0;
    f.chunk_kb = f.stride = 0;
    f.a = f.b = make_rsrc(p.zero, 0);
    // prefill: rows of this launch's chunk are stored by the append level,
    // so nothing before the event may pull their lines into a cache
    if (p.prefetch_kb <= 0 || p.paged || p.prefill) return f;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int pos = p.seq_lens[b];
    if (pos < 0 || pos + 1 > p.cap) return f;
    const int j0 = split * C, j1 = min(j0 + C, pos);
    if (j1 <= j0) return f;
    const int64_t off = (int64_t)l * p.kv_layer_stride + ((int64_t)(b * p.Hkv + g) * p.cap + j0) * p.D;
    const uint32_t bytes = (uint32_t)(j1 - j0) * (uint32_t)p.D * (uint32_t)sizeof(WT);
    f.a = make_rsrc((const WT*)p.kv_k + off, bytes);
    f.b = make_rsrc((const WT*)p.kv_v + off, bytes);
    f.kb_a = f.kb_b = (bytes + 1023u) / 1024u;
    f.end = min(f.kb_a + f.kb_b, (uint32_t)p.prefetch_kb);
    return f;
}

// Issue the next slice: each wave takes every kWaves-th KB. With two
// segments, KB i of the stream is KB i/2 of segment (i & 1). Offsets past a
// segment are out of range for its resource and fetch nothing.
__device__ __forceinline__ void prefetch_step(Prefetch& f) {
    if (f.next >= f.end) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    auto* sink = (__attribute__((address_space(3))) void*)&mk_prefetch_sink[wave][0];
#pragma unroll
    for (int k = 0; k < kPrefetchSlice; ++k) {
        const uint32_t i = f.next + (uint32_t)(k * kWaves + wave);
        if (i >= f.end) break;
        if (f.chunk_kb) {
            const uint32_t o = (i / f.chunk_kb) * f.stride + (i % f.chunk_kb) * 1024u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(f.a, sink, 16, lane * 16, o, 0, kPfAux);
        } else if (f.kb_b == 0) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(f.a, sink, 16, lane * 16, i * 1024u, 0, kPfAux);
        } else {
            const uint32_t o = (i >> 1) * 1024u;
            if (i & 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(f.b, sink, 16, lane * 16, o, 0, kPfAux);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(f.a, sink, 16, lane * 16, o, 0, kPfAux);
        }
    }
    f.next += (uint32_t)(kPrefetchSlice * kWaves);
}

// ---------------------------------------------------------------- attention

// One split of the split-KV decode attention for (layer, b, g, split):
// positions [split*C, min((split+1)*C, pos+1)). Writes the split's partial
// (acc, m, l) and, if it is the last to arrive for (b, g), merges all
// splits in split order and (persistent mode) signals the layer's
// attention event. The split that holds position pos first normalises,
// rotates and appends the new k and v (rounded to the cache type).
// Partial record: acc[G*D], m[h] at G*D + h, l[h] at G*D + 8 + h.
// D (head size) and GP (query heads per KV head rounded up to a power of
// two) are compile-time so that every lane loop and reduction unrolls;
// heads G..GP-1 are computed on zeros and never stored.
__host__ __device__ constexpr int attn_rec(int G, int D) { return G * D + 16; }
__host__ __device__ constexpr int attn_gp(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

template <typename WT, int D, int GP>
__device__ __forceinline__ void attention_body(const KParams& p, int l, int bg, int split, int C, const Lds& s,
                                               int ev_plane) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hkv = p.Hkv, G = p.Hq / p.Hkv;
    const int b = bg / Hkv, g = bg % Hkv;
    // prefill plans: every row is a position of sequence 0 (shared K/V), and
    // the row's own key and value were stored by the append level
    const int bkv = p.prefill ? 0 : b;
    const bool own_lds = !p.prefill;
    const float* qkv = layer_buf(p, l, p.off_qkv) + (int64_t)b * (p.QD + 2 * p.KD);
    const LayerPtrs& lw = p.lw[l];
    // 0. this wave's query heads, the new k (wave 0) and v (wave 1), and the
    // norm gains are requested first: their addresses do not depend on the
    // sequence length, so they are in flight while it is read
    constexpr int QPW = (GP + kWaves - 1) / kWaves;  // query heads per wave
    float qv[QPW][2];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
        const int hh = wave + i * kWaves;
        qv[i][0] = qv[i][1] = 0.f;
        if (hh < G) {
            qv[i][0] = ld_act(&qkv[(int64_t)(g * G + hh) * D + lane]);
            if constexpr (D > 64) qv[i][1] = ld_act(&qkv[(int64_t)(g * G + hh) * D + lane + 64]);
        }
    }
    float nv[2] = {0.f, 0.f};
    if (wave < 2) {
        const int64_t base = wave == 0 ? (int64_t)p.QD + (int64_t)g * D : (int64_t)p.QD + p.KD + (int64_t)g * D;
        nv[0] = ld_act(&qkv[base + lane]);
        if constexpr (D > 64) nv[1] = ld_act(&qkv[base + lane + 64]);
    }
    const bool qkn = p.qk_norm != 0;
    float gq[2] = {1.f, 1.f}, gk[2] = {1.f, 1.f};
    if (qkn) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            gq[i] = load_scalar<WT>((const WT*)lw.q_norm, lane + 64 * i);
            gk[i] = load_scalar<WT>((const WT*)lw.k_norm, lane + 64 * i);
        }
    }

    const int pos = p.seq_lens[b];
    const bool overflow = pos < 0 || pos + 1 > p.cap;
    const int keys = pos + 1;
    const int ns = overflow ? 1 : (keys + C - 1) / C;
    if (split >= ns) return;  // reserved AOT slot beyond this sequence's length
    float* out = layer_buf(p, l, p.off_attn) + (int64_t)b * p.QD + (int64_t)g * G * D;

    if (overflow) {
        for (int i = tid; i < G * D; i += kThreads) st_co(&out[i], 0.f);
        if (tid == 0) raise_error(p.ctrl, MK_ERR_KV_OVERFLOW);
        if (p.persistent) signal_event(p, ev_attn(l), s, ev_plane);
        return;
    }
    const int j0 = split * C, j1 = min(j0 + C, keys);
    const bool owner = (j1 == keys);
    const int n = j1 - j0;
    const bool appender = own_lds && owner && wave < 2;
    // this lane's RoPE factors at position pos
    const float2 cs = p.rope[(int64_t)pos * (D / 2) + (D == 128 ? lane : (lane & 31))];
    asm volatile("" ::: "memory");

    // K/V rows of this split. V (and, for an fp32 cache, K) is held in the
    // lane layout of the P.V update: lane (rr, cc) holds 16 bytes (column
    // segment cc) of one row per load. With a bf16 cache the scores run on the
    // 16x16x32 matrix cores and K is loaded in their operand layout instead:
    // for k-step q, lane l holds dims 32 q + 8 (l/16) .. + 7 of row l % 16 of
    // a 16-row tile, so one load covers 64 contiguous bytes of each row.
    using VK = Vec16<WT>;
    constexpr int E = VK::N;
    constexpr int LPR = D / E;             // lanes per row in the P.V layout
    constexpr int PPW = 64 / LPR;          // rows per wave per load
    constexpr int PER_IT = kWaves * PPW;   // rows per workgroup iteration
    constexpr bool kMf = std::is_same<WT, bf16_t>::value;
    constexpr int WR = 16;                 // rows per wave per batch in the matrix-core layout (16-row tiles)
    constexpr int NT = WR / 16;            // tiles per wave per batch
    constexpr int KS = D / 32;             // MFMA k-steps per row
    constexpr int NIT = kMf ? WR / PPW : (GP >= 8 ? 16 : 32) / kWaves;  // V loads per lane per batch
    constexpr int NK = kMf ? NT * KS : NIT;                             // K loads per lane per batch
    constexpr int SUB = kMf ? kWaves * WR : PER_IT * NIT;               // rows per batch
    const int rr = lane / LPR, cc = lane % LPR;
    const int li = lane & 15, lg = lane >> 4;  // matrix-core row and k group
    // K/V of this (layer, b, g) through buffer resources; rows past the split
    // (or the new row, which comes from LDS) load through an out-of-range
    // offset: no branches around loads
    constexpr int es = (int)sizeof(WT);
    const int64_t lbase = (int64_t)l * p.kv_layer_stride;
    __amdgpu_buffer_rsrc_t krs, vrs;
    if (!p.paged) {
        const int64_t seq = lbase + (int64_t)(bkv * Hkv + g) * p.cap * D;
        krs = make_rsrc((const WT*)p.kv_k + seq, (uint32_t)p.cap * (uint32_t)(D * es));
        vrs = make_rsrc((const WT*)p.kv_v + seq, (uint32_t)p.cap * (uint32_t)(D * es));
    } else {
        krs = make_rsrc((const WT*)p.kv_k + lbase, (uint32_t)(p.kv_layer_stride * es));
        vrs = make_rsrc((const WT*)p.kv_v + lbase, (uint32_t)(p.kv_layer_stride * es));
    }
    const int32_t* btab = p.paged ? p.block_table + (int64_t)bkv * p.max_blocks : nullptr;
    // the split's block-table entries are staged in LDS for the batches after
    // the first (visible after the prologue barrier), so that a batch's K/V
    // requests never wait behind a block-table load
    const int blk0 = p.paged ? j0 / p.kv_block : 0;
    if (p.paged) {
        const int nblk = (j1 - 1) / p.kv_block - blk0 + 1;
        for (int i = tid; i < nblk; i += kThreads) {
            const int e = btab[blk0 + i];
            // an entry outside the pool reads zeros (and is reported)
            if ((unsigned)e >= (unsigned)p.n_pool_blocks) raise_error(p.ctrl, MK_ERR_BLOCK_TABLE);
            s.btab[i] = e;
        }
    }
    // byte offset of row j of the split (plus `add`), or out of range for
    // rows past the split, for the new row and for blocks outside the pool.
    // In range, every offset is below 2^31 bytes (the plan and the step
    // check that a sequence's contiguous span, or a paged layer, is smaller).
    auto row_off = [&](int j, uint32_t add, bool staged) -> uint32_t {
        const int jj = j0 + j;
        if (j >= n || (own_lds && jj == pos)) return kOOB;
        uint32_t o;
        if (p.paged) {
            const int bi = jj / p.kv_block;
            const int blk = staged ? s.btab[bi - blk0] : btab[bi];
            if ((unsigned)blk >= (unsigned)p.n_pool_blocks) return kOOB;
            o = (uint32_t)(((blk * Hkv + g) * p.kv_block + jj % p.kv_block) * D * es);
        } else {
            o = (uint32_t)(jj * D * es);
        }
        return o + add;
    };
    // row of the split that V load `it` of this lane holds in a batch at `base`
    auto vrow = [&](int base, int it) {
        return kMf ? base + wave * WR + it * PPW + rr : base + it * PER_IT + wave * PPW + rr;
    };
    // Matrix-core layout (bf16 cache): a wave's K and V rows of a batch are
    // the 16 rows tb .. tb + 15 (tb = base + 16 wave, a multiple of 16, as is
    // j0). A paged bf16 cache has blocks of a multiple of 16 positions (the
    // plan checks it), so the 16 rows share one block: its entry and the
    // tile's offset are found once per batch and wave, not per row.
    static_assert(!kMf || (NT == 1 && WR == 16 && NIT * PPW == 16), "one 16-row tile per wave and batch");
    // K and V rows of a batch into registers (rows at or past n fetch nothing)
    auto load_kv = [&](uint4 (&kd)[NK], uint4 (&vd)[NIT], int base, bool staged) {
        if constexpr (kMf) {
            {
                const int tb = base + wave * WR;
                uint32_t tile = kOOB;
                if (tb < n) {
                    const int jt = j0 + tb;
                    if (!p.paged) {
                        tile = (uint32_t)(jt * D * es);
                    } else {
                        const int bi = jt / p.kv_block;
                        const int blk = staged ? s.btab[bi - blk0] : btab[bi];
                        if ((unsigned)blk < (unsigned)p.n_pool_blocks)
                            tile = (uint32_t)(((blk * Hkv + g) * p.kv_block + jt % p.kv_block) * D * es);
                    }
                }
                // row tb + d of the tile, or out of range
                auto off = [&](int d, uint32_t add) -> uint32_t {
                    const int j = tb + d;
                    if (tile == kOOB || j >= n || (own_lds && j0 + j == pos)) return kOOB;
                    return tile + (uint32_t)(d * D * es) + add;
                };
#pragma unroll
                for (int q = 0; q < NK; ++q) kd[q] = buf_load16_kv(krs, off(li, (uint32_t)(16 * (4 * (q % KS) + lg))), 0);
#pragma unroll
                for (int it = 0; it < NIT; ++it) vd[it] = buf_load16_kv(vrs, off(it * PPW + rr, (uint32_t)(cc * 16)), 0);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NK; ++q) kd[q] = buf_load16_kv(krs, row_off(vrow(base, q), (uint32_t)(cc * 16), staged), 0);
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                vd[it] = buf_load16_kv(vrs, row_off(vrow(base, it), (uint32_t)(cc * 16), staged), 0);
        }
    };
    // the first batch of K and V rows is requested before the prologue's math
    const bool one_batch = n <= SUB;
    uint4 kr[NK], vr[NIT];
    load_kv(kr, vr, 0, false);

    // 1. query heads of this group: norm + RoPE into LDS
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
        const int hh = wave + i * kWaves;
        if (hh < G) {
            head_norm_rope<D>(qv[i], gq, qkn, p.eps, cs);
            s.q[hh * D + lane] = qv[i][0];
            if constexpr (D > 64) s.q[hh * D + lane + 64] = qv[i][1];
        }
    }
    // 2. owner: new k (norm + RoPE) and v, rounded to the cache type, appended
    if (appender) {
        if (wave == 0) head_norm_rope<D>(nv, gk, qkn, p.eps, cs);
        const int64_t off = kv_offset(p, l, b, g, pos);
        if (off < 0 && lane == 0 && wave == 0) raise_error(p.ctrl, MK_ERR_BLOCK_TABLE);
        WT* dst = (WT*)(wave == 0 ? p.kv_k : p.kv_v) + (off < 0 ? 0 : off);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const WT c = from_float<WT>(nv[i]);
            // agent-coherent: a later step of the same launch may read the row on
            // another CU (a bad block-table entry: nothing is written)
            if (off >= 0) st_co(&dst[lane + 64 * i], c);
            s.kn[wave * 128 + lane + 64 * i] = to_float<WT>(c);
        }
    }
    __syncthreads();
    trace_mark(p, s.marks, 0);

    // 3. one pass over the split's keys with a running (max, sum, acc) per
    // head in each wave: the K and V rows of a batch are requested together,
    // one batch ahead of the one in use. The running max of a head is the
    // same in every lane of the wave, which keeps every lane's acc on one
    // scale; the four waves merge at the end.
    float acc[GP][E], lsum[GP], mrun[GP];
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) {
        lsum[hh] = 0.f;
        mrun[hh] = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
    }
    // fp32 cache: lanes (rr, cc) of row group rr hold the full score of their
    // row after the group sum, which is the probability their P.V update needs
    auto process_valu = [&](const uint4 (&kk)[NK], const uint4 (&vv)[NIT], int base) {
        float d[NIT][GP];
        float bm[GP];
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) bm[hh] = -INFINITY;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int j = base + it * PER_IT + wave * PPW + rr;
            const bool valid = j < n;
            float kf[E];
            if (own_lds && valid && j0 + j == pos) {
#pragma unroll
                for (int e = 0; e < E; ++e) kf[e] = s.kn[cc * E + e];
            } else {
                VK::widen(kk[it], kf);
            }
#pragma unroll
            for (int hh = 0; hh < GP; ++hh) {
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) t = fmaf(s.q[hh * D + cc * E + e], kf[e], t);
                t = group_sum<LPR>(t) * p.scale;
                d[it][hh] = valid ? t : -INFINITY;
                bm[hh] = fmaxf(bm[hh], d[it][hh]);
            }
        }
        float mz[GP], corr[GP];
        bool grew = false;  // some head's running max rose (uniform over the wave)
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
            const float mn = fmaxf(mrun[hh], column_max<LPR>(bm[hh]));
            // mn is -inf only while this wave has seen no key: nothing to scale
            corr[hh] = mn == -INFINITY ? 1.f : __expf(mrun[hh] - mn);
            mz[hh] = mn == -INFINITY ? 0.f : mn;
            grew |= mn != mrun[hh];
            mrun[hh] = mn;
        }
        // an unchanged max scales by exactly e^0 = 1: skipping it keeps the bits
        if (grew) {
#pragma unroll
            for (int hh = 0; hh < GP; ++hh) {
                lsum[hh] *= corr[hh];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[hh][e] *= corr[hh];
            }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int j = base + it * PER_IT + wave * PPW + rr;
            float vf[E];
            if (own_lds && j < n && j0 + j == pos) {
#pragma unroll
                for (int e = 0; e < E; ++e) vf[e] = s.kn[128 + cc * E + e];
            } else {
                VK::widen(vv[it], vf);  // rows past the split loaded zeros
            }
#pragma unroll
            for (int hh = 0; hh < GP; ++hh) {
                const float pj = __expf(d[it][hh] - mz[hh]);  // exp(-inf) = 0 past the split
                lsum[hh] += pj;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[hh][e] = fmaf(pj, vf[e], acc[hh][e]);
            }
        }
    };
    // bf16 cache: scores on the matrix cores. Query heads are the 16 columns
    // (heads past G are zeros), split hi + lo into bf16 like the GEMV
    // activations; each wave scores its 16-row tiles, keeps the online
    // softmax on the result tiles (lane l: rows 4*(l/16) + r, head l % 16)
    // and hands the probabilities to its P.V lanes through LDS.
    mk_bf16x8 qh[KS], ql[KS];
    if constexpr (kMf) {
#pragma unroll
        for (int q = 0; q < KS; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = li < G ? s.q[li * D + 32 * q + 8 * lg + e] : 0.f;
                const __bf16 h = (__bf16)v;
                qh[q][e] = h;
                ql[q][e] = (__bf16)(v - (float)h);
            }
    }
    float* pw = s.pt + wave * (WR * 8);  // this wave's probabilities [row][head]
    float mlane = -INFINITY;             // running max of head li, as mrun[li]
    auto process_mf = [&](const uint4 (&kk)[NK], const uint4 (&vv)[NIT], int base) {
        mk_f32x4 sc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // the hi and lo query terms accumulate in two independent chains
            mk_f32x4 sh = mk_f32x4{0.f, 0.f, 0.f, 0.f}, sl = sh;
            const int j = base + wave * WR + 16 * t + li;
            const bool nw = own_lds && j < n && j0 + j == pos;  // the new row's k comes from LDS
#pragma unroll
            for (int q = 0; q < KS; ++q) {
                uint4 a = kk[t * KS + q];
                if (nw) {
                    mk_bf16x8 kb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) kb[e] = (__bf16)s.kn[32 * q + 8 * lg + e];
                    a = __builtin_bit_cast(uint4, kb);
                }
                sh = mfma_bf16(a, qh[q], sh);
                sl = mfma_bf16(a, ql[q], sl);
            }
            sc[t] = sh + sl;
        }
        // scale, mask rows past the split, batch max of head li
        float bm = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = base + wave * WR + 16 * t + 4 * lg + r;
                sc[t][r] = j < n ? sc[t][r] * p.scale : -INFINITY;
                bm = fmaxf(bm, sc[t][r]);
            }
        bm = column_max<16>(bm);
        float mz[GP], corr[GP];
        bool grew = false;  // some head's running max rose (uniform over the wave)
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
            const float mn = fmaxf(mrun[hh], read_lane(bm, hh));
            // mn is -inf only while this wave has seen no key: nothing to scale
            corr[hh] = mn == -INFINITY ? 1.f : __expf(mrun[hh] - mn);
            mz[hh] = mn == -INFINITY ? 0.f : mn;
            grew |= mn != mrun[hh];
            mrun[hh] = mn;
        }
        // an unchanged max scales by exactly e^0 = 1: skipping it keeps the bits
        if (grew) {
#pragma unroll
            for (int hh = 0; hh < GP; ++hh) {
                lsum[hh] *= corr[hh];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[hh][e] *= corr[hh];
            }
        }
        mlane = fmaxf(mlane, bm);
        const float mzl = mlane == -INFINITY ? 0.f : mlane;
        if (li < GP) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) pw[(16 * t + 4 * lg + r) * 8 + li] = __expf(sc[t][r] - mzl);  // 0 past the split
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int jw = it * PPW + rr;  // row within the wave's WR
            const int j = base + wave * WR + jw;
            float vf[E];
            if (own_lds && j < n && j0 + j == pos) {
#pragma unroll
                for (int e = 0; e < E; ++e) vf[e] = s.kn[128 + cc * E + e];
            } else {
                VK::widen(vv[it], vf);  // rows past the split loaded zeros
            }
#pragma unroll
            for (int hh = 0; hh < GP; ++hh) {
                const float pj = pw[jw * 8 + hh];
                lsum[hh] += pj;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[hh][e] = fmaf(pj, vf[e], acc[hh][e]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    };
    auto process = [&](const uint4 (&kk)[NK], const uint4 (&vv)[NIT], int base) {
        if constexpr (kMf) process_mf(kk, vv, base);
        else process_valu(kk, vv, base);
    };
    if (one_batch) {
        process(kr, vr, 0);
    } else {
        uint4 kb[NK], vb[NIT];
        for (int base = 0; base < n; base += 2 * SUB) {
            load_kv(kb, vb, base + SUB, true);
            process(kr, vr, base);
            load_kv(kr, vr, base + 2 * SUB, true);
            if (base + SUB < n) process(kb, vb, base + SUB);
        }
    }
    trace_mark(p, s.marks, 1);
    // 4. this wave's (m, l, acc): sums over its row groups (lanes with equal cc)
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) {
        lsum[hh] = column_sum<LPR>(lsum[hh]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = column_sum<LPR>(acc[hh][e]);
    }
    if (rr == 0) {
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
            if (hh >= G) continue;
#pragma unroll
            for (int e = 0; e < E; ++e) s.acc[(wave * 8 + hh) * 128 + cc * E + e] = acc[hh][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
            if (hh >= G) continue;
            s.wml[wave * 16 + hh] = mrun[hh];
            s.wml[wave * 16 + 8 + hh] = lsum[hh];
        }
    }
    __syncthreads();

    trace_mark(p, s.marks, 2);
    // 5. partial record: the waves merged in wave order on the split's max
    const int rec = attn_rec(G, D);
    float* part = p.partials + ((int64_t)bg * p.max_splits + split) * rec;
    auto wave_scale = [&](int w, int hh, float M) {
        const float m = s.wml[w * 16 + hh];
        return m == -INFINITY ? 0.f : __expf(m - M);
    };
    auto split_max = [&](int hh) {
        float M = s.wml[hh];
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s.wml[w * 16 + hh]);
        return M;  // finite: the split holds at least one key
    };
    if (tid < G) {
        const float M = split_max(tid);
        float L = s.wml[8 + tid] * wave_scale(0, tid, M);
        for (int w = 1; w < kWaves; ++w) L = fmaf(s.wml[w * 16 + 8 + tid], wave_scale(w, tid, M), L);
        s.ml[2 * tid] = M;
        s.ml[2 * tid + 1] = L;
        if (ns > 1) {
            st_co(&part[G * D + tid], M);
            st_co(&part[G * D + 8 + tid], L);
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kThreads) {
        const int hh = i / D, d = i % D;
        const float M = s.ml[2 * hh];
        float a = s.acc[hh * 128 + d] * wave_scale(0, hh, M);
        for (int w = 1; w < kWaves; ++w) a = fmaf(s.acc[(w * 8 + hh) * 128 + d], wave_scale(w, hh, M), a);
        // a sequence of one split is its own combine: the merge below would
        // compute a * e^0 / (l * e^0), the same bits
        if (ns == 1) st_co(&out[i], a / s.ml[2 * hh + 1]);
        else st_co(&part[i], a);
    }
    if (ns == 1) {
        if (p.persistent) signal_event(p, ev_attn(l), s, ev_plane);
        return;
    }

    // 6. last arrival merges the splits in split order
    wait_stores();
    trace_mark(p, s.marks, 3);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.arrive[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.cmd[8] = (old + 1u == (uint32_t)ns) ? 1 : 0;
    }
    __syncthreads();
    const bool last = s.cmd[8] != 0;
    __syncthreads();
    if (!last) return;
    const float* part0 = p.partials + (int64_t)bg * p.max_splits * rec;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(part0, (uint32_t)(ns * rec) * 4u);
    const int q4 = rec / 4;  // 16-byte chunks per record
    // running (M, num, den) per output element, merged split by split:
    //   M' = max(M, m_s); num = num e^{M-M'} + acc_s e^{m_s-M'}; den likewise with l_s
    float M[4], num[4], den[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        M[k] = -INFINITY;
        num[k] = 0.f;
        den[k] = 0.f;
    }
    for (int c0 = 0; c0 < ns; c0 += kCmbSplits) {
        const int nc = min(kCmbSplits, ns - c0);
        // up to 8 loads of a thread in flight before its LDS stores
        for (int i0 = tid; i0 < nc * q4; i0 += 8 * kThreads) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kThreads;
                v[u] = buf_load16_co(prs, i < nc * q4 ? (uint32_t)((c0 * q4 + i) * 16) : kOOB, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kThreads;
                if (i < nc * q4) *(uint4*)(s.cmb + i * 4) = v[u];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = tid + k * kThreads;
            if (i >= G * D) continue;
            const int hh = i / D;
            for (int sp = 0; sp < nc; ++sp) {
                const float* r = s.cmb + sp * rec;
                const float ms = r[G * D + hh], ls = r[G * D + 8 + hh], as = r[i];
                const float Mn = fmaxf(M[k], ms);
                const float co = __expf(M[k] - Mn), cn = __expf(ms - Mn);
                num[k] = num[k] * co + as * cn;
                den[k] = den[k] * co + ls * cn;
                M[k] = Mn;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = tid + k * kThreads;
        if (i < G * D) st_co(&out[i], num[k] / den[k]);
    }
    if (tid == 0) __hip_atomic_store(&p.arrive[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.persistent) signal_event(p, ev_attn(l), s, ev_plane);
}

template <typename WT, int D>
__device__ __forceinline__ void attention_task_d(const KParams& p, int l, int bg, int split, int C, const Lds& s,
                                                 int ev_plane) {
    switch (attn_gp(p.Hq / p.Hkv)) {
        case 1: attention_body<WT, D, 1>(p, l, bg, split, C, s, ev_plane); break;
        case 2: attention_body<WT, D, 2>(p, l, bg, split, C, s, ev_plane); break;
        case 4: attention_body<WT, D, 4>(p, l, bg, split, C, s, ev_plane); break;
        default: attention_body<WT, D, 8>(p, l, bg, split, C, s, ev_plane); break;
    }
}
// C: the step's chunk, attn_chunk(p); ev_plane: the attention-done count
// plane this workgroup adds to
template <typename WT>
__device__ __forceinline__ void attention_task(const KParams& p, int l, int bg, int split, int C, const Lds& s,
                                               int ev_plane = 0) {
    if (p.D == 128) attention_task_d<WT, 128>(p, l, bg, split, C, s, ev_plane);
    else attention_task_d<WT, 64>(p, l, bg, split, C, s, ev_plane);
}

}  // namespace mk
