// Device-side helpers and the kernel parameter block shared by the
// persistent megakernel and the kernel-per-operator launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

using bf16_t = uint16_t;

constexpr int kThreads = 256;  // one workgroup = 4 wave64 (one per SIMD)
constexpr int kWaves = kThreads / 64;

// Per-layer weight pointers (same layout as mk_layer_weights).
struct LayerPtrs {
    const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
};
static_assert(sizeof(LayerPtrs) == sizeof(mk_layer_weights), "LayerPtrs layout");

// Each event counter is kept as up to kEvPlanesMax partial counts, one
// 128-byte aligned plane each; its value is the sum of the planes (mod 2^32).
// A kernel instance for batch NB uses ev_planes(NB) of them: GEMV and
// attention producers spread their arrivals over those planes, so that the
// arrivals of one event do not all queue on one address, and a waiter sums
// them. At batch
// 8 and 16 that is faster; at smaller batches the waiters' extra polling
// loads cost more than it saves, and one plane is used.
constexpr int kEvPlanesMax = 8;
__host__ __device__ constexpr int ev_planes(int nb) { return nb >= 8 ? kEvPlanesMax : 1; }
__host__ __device__ constexpr int ev_plane_stride(int n_events) { return (n_events + 31) / 32 * 32; }

// Everything a task body needs; passed by value to every kernel.
struct KParams {
    // task graph
    const TaskRec* tasks;
    const int32_t* qoff;
    const int32_t* queue;
    const EventRec* evrec;
    uint32_t* ev;      // [kEvPlanesMax][ev_stride] partial counts
    int ev_stride;
    uint32_t* arrive;  // [B * Hkv] last-arrival counters (self-resetting)
    RingSlot* inbox;         // [workers][inbox_mask + 1] JIT tasks dealt to each worker
    int64_t* inbox_tail;     // [workers] producer positions
    int64_t* inbox_head;     // [workers] consumer positions (kept across launches)
    const int32_t* elig;     // workers that receive JIT tasks
    RingSlot* mb;
    Ctrl* ctrl;
    const float2* rope;  // [cap][D/2] (cos, sin)
    float* partials;     // [B * Hkv][max_splits][G * D + 2 G]
    // activations (fp32)
    const float* x0;  // layer-0 input [B, H]
    float* x0_w;      // writable view of x0 (token mode: the embedding gather writes it)
    float* act;       // per-layer blocks
    int64_t act_stride;
    int64_t off_qkv, off_attn, off_xmid, off_h, off_xnext;
    float* x_final;  // output of the last layer's down projection
    float* logits;
    // weights
    const LayerPtrs* lw;
    const void* zero;  // zero-filled buffer of at least the largest K (stays cached)
    const void* embed;
    const void* final_norm;
    const void* lm_head;
    // KV cache
    void* kv_k;
    void* kv_v;
    int64_t kv_layer_stride;
    const int32_t* block_table;
    int n_pool_blocks;  // paged: physical blocks per layer (layer_stride / (Hkv * kv_block * D))
    // step inputs
    const int32_t* tokens;
    const int32_t* seq_lens;
    // shape
    int B, H, Hq, Hkv, D, F, V, L, QD, KD, cap, chunk, max_splits, qk_norm, paged, kv_block, max_blocks;
    int chunk_max, attn_target;  // per-step attention chunk rule (attn_chunk_for)
    float eps, scale;
    // schedule
    uint32_t epoch;
    int n_workers;
    int jit_on;  // 0 AOT, 1 JIT through scheduler waves, 2 JIT expanded by the completing QKV arrival
    int persistent;  // 1: events are signalled (persistent mode)
    int inbox_mask;
    int n_elig;
    int mb_mask;
    uint64_t watchdog_ticks;  // 100 MHz ticks
    int prefetch_kb;          // next-task weight bytes pulled into L2 per worker (KB)
    int pre_slots;            // LDS preload slots per wave for the awaited GEMV task (0: off)
    int w4;                   // 1: the layer matrices are W4 buffers (batch <= 2); gains, embedding, LM head bf16
    int wtiled;               // 1: layer matrices and LM head in the tiled layout (matrix-core instances)
    float* kpart;             // K-split down projection: partial tiles [rows][parts][16]
    uint32_t* karrive;        // K-split down projection: arrivals per row group (self-resetting)
    int prefill;              // 1: the batch rows are consecutive positions of sequence 0 (prompt chunk)
    int32_t* greedy_tokens;   // greedy step: next token of each sequence written here (else null)
    int32_t* greedy_lens;     // greedy step: each sequence's length advanced here
    int32_t* out_tokens;      // greedy steps: step s's tokens at [s * B, s * B + B) (or null)
    int n_steps;              // greedy decode steps this launch runs (1 unless multi-step)
    unsigned long long* amax; // [B] packed (value, index) argmax keys; zero between steps
    uint32_t* lm_done;        // kernel-per-op greedy step: LM-head tasks finished (reset by the last)
    uint32_t* exit_cnt;       // persistent greedy step: workers that left their queue (reset by the last)
    int n_lm_tasks;
    // optional task trace: per worker `trace_cap` records, count in trace_n
    mk_trace_rec* trace;
    int32_t* trace_n;
    int trace_cap;
};


// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (bf16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (bf16_t)(b >> 16);
}

// 16 bytes of weights widened to floats: 8 bf16 or 4 f32
template <typename WT>
struct Vec16;
template <>
struct Vec16<bf16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void widen(const uint4& w, float* f) {
        f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
        f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
        f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    }
};
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void widen(const uint4& w, float* f) {
        f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
    }
};

template <typename WT>
__device__ __forceinline__ float load_scalar(const WT* p, int64_t i);
template <>
__device__ __forceinline__ float load_scalar<bf16_t>(const bf16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ __forceinline__ float load_scalar<float>(const float* p, int64_t i) {
    return p[i];
}

template <typename WT>
__device__ __forceinline__ float to_float(WT v);
template <>
__device__ __forceinline__ float to_float<bf16_t>(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <>
__device__ __forceinline__ float to_float<float>(float v) { return v; }

template <typename WT>
__device__ __forceinline__ WT from_float(float f);
template <>
__device__ __forceinline__ bf16_t from_float<bf16_t>(float f) { return f32_to_bf16(f); }
template <>
__device__ __forceinline__ float from_float<float>(float f) { return f; }

// ---------------------------------------------------------------- lane reductions
// Sums and maxima over aligned groups of N lanes through DPP lane selects,
// which stay inside the VALU (no LDS crossbar round trip): two quad_perm
// swaps reduce groups of 4, the half-row mirror (lane i <-> 7 - i) and the
// row mirror (i <-> 15 - i) extend that to 8 and 16 lanes. The four rows of
// a wave meet through readlane. The pairing is symmetric, so every lane of
// a group ends with the bitwise-same value. Call with all lanes active.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp_sel(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float read_lane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sums across the rows of 16 lanes through the gfx950 row-swap instructions
// (VALU, no LDS crossbar): with both operands equal, permlane16_swap returns
// the even rows in its first result and the odd rows in its second, so their
// sum is v[l] + v[l ^ 16] in every lane, added in the same order in both
// lanes; permlane32_swap does the same for the two halves (l ^ 32).
__device__ __forceinline__ float rows_sum16(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float halves_sum32(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// the value of lane l ^ 32
__device__ __forceinline__ float halves_partner(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N >= 2) v += dpp_sel<kDppXor1>(v);
    if constexpr (N >= 4) v += dpp_sel<kDppXor2>(v);
    if constexpr (N >= 8) v += dpp_sel<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_sel<kDppMirror>(v);
    if constexpr (N == 32) v = rows_sum16(v);
    if constexpr (N == 64) v = (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
    return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N >= 2) v = fmaxf(v, dpp_sel<kDppXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_sel<kDppXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_sel<kDppHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_sel<kDppMirror>(v));
    if constexpr (N == 32) {
        const unsigned u = __builtin_bit_cast(unsigned, v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
    }
    if constexpr (N == 64) v = fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
    return v;
}
constexpr int kDppRor8 = 0x128;  // row_ror:8 (lane l <- l ^ 8 inside a row of 16)

// Sum over the lanes l' with l' % N == l % N (N = 8, 16 or 32): the lanes
// that hold the same column position in each group of N.
template <int N>
__device__ __forceinline__ float column_sum(float v) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N == 8) v += dpp_sel<kDppRor8>(v);
    if constexpr (N <= 16) v = rows_sum16(v);
    if constexpr (N <= 32) v = halves_sum32(v);
    return v;
}

// Maximum over the same lanes as column_sum.
template <int N>
__device__ __forceinline__ float column_max(float v) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N == 8) v = fmaxf(v, dpp_sel<kDppRor8>(v));
    if constexpr (N <= 16) {
        const unsigned u = __builtin_bit_cast(unsigned, v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
    }
    if constexpr (N <= 32) {
        const unsigned u = __builtin_bit_cast(unsigned, v);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// ---------------------------------------------------------------- memory model

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int64_t ld_acquire64(const int64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int64_t ld_relaxed64(const int64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Coherence between workgroups without L2-wide fences. On this part an
// agent-scope release fence writes back the whole L2 and an acquire
// invalidates it (several microseconds each), so data that one workgroup
// hands to another within a step moves with agent-coherent (sc1) accesses
// instead: the producer stores with st_co, waits for its stores to
// complete (wait_stores), then bumps the event counter with a relaxed
// atomic; the consumer polls the counter, then reads with ld_co / sc1
// buffer loads, which do not hit stale cache lines. Weights and the KV
// cache positions read within a step were written before the launch and
// use ordinary cached loads.
constexpr int kSC1 = 16;  // cache-policy bit of agent-coherent buffer accesses
__device__ __forceinline__ float ld_co(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_co(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_co(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_co(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_co(uint16_t* p, uint16_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// phase marks for the task trace: thread 0 keeps them in shared memory
__device__ __forceinline__ void trace_mark(const KParams& p, uint64_t* marks, int i) {
    if (p.trace && threadIdx.x == 0) marks[i] = now_ticks();
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources (base, size) in SGPRs with 32-bit lane offsets: a
// load whose offset is past `size` returns zero and touches no memory, which
// pads tails and unused rows for free.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Cache policy of the once-per-step streams, chosen per kernel instance
// (each batch tile is its own compilation unit, MK_NB). At batch <= 2 a
// wave's weight load covers whole 128-byte lines that nothing reads again,
// so weights stream with the non-temporal policy: a plain read of a large
// buffer measured 6.1 TB/s, a non-temporal one 6.6-6.7 TB/s, and the batch-1
// step went 3.744 -> 3.514 ms. Cached K/V keeps the plain policy there (its
// rows were pulled into L2 while the attention slot waited; non-temporal:
// 3.525 ms). In the matrix-core instances (batch >= 4) each load reads half
// of a line and the next k-step the other half: non-temporal weights made
// the batch-16 step 9% slower (5.81 -> 6.36 ms), so everything stays plain.
// The prefetch loads must stay plain: their lines are meant to be kept.
#ifndef MK_STREAM_AUX_SMALL
#define MK_STREAM_AUX_SMALL 2
#endif
#ifndef MK_KV_AUX_SMALL
#define MK_KV_AUX_SMALL 0
#endif
#ifndef MK_STREAM_AUX_LARGE
#define MK_STREAM_AUX_LARGE 0
#endif
#ifndef MK_KV_AUX_LARGE
#define MK_KV_AUX_LARGE 0
#endif
#if defined(MK_NB) && MK_NB >= 4
#ifndef MK_STREAM_AUX
#define MK_STREAM_AUX MK_STREAM_AUX_LARGE
#endif
#ifndef MK_KV_AUX
#define MK_KV_AUX MK_KV_AUX_LARGE
#endif
#else
#ifndef MK_STREAM_AUX
#define MK_STREAM_AUX MK_STREAM_AUX_SMALL
#endif
#ifndef MK_KV_AUX
#define MK_KV_AUX MK_KV_AUX_SMALL
#endif
#endif
#ifndef MK_PF_AUX
#define MK_PF_AUX 0
#endif
// Tiled weights (MK_WEIGHTS_TILED): a matrix-core load reads 512-byte runs
// of consecutive bytes, whole lines that nothing reads again, so they stream
// non-temporally. A stream probe on one MI355X (all CUs, four blocks in
// flight per wave) measured 4.4-5.1 TB/s for the row-major operand pattern,
// 5.6-5.9 TB/s for the same bytes in tile order with plain loads and
// 6.2-6.5 TB/s with non-temporal ones.
#ifndef MK_TILED_AUX
#define MK_TILED_AUX 2
#endif
constexpr int kStreamAux = MK_STREAM_AUX;  // cache policy of weight loads (0 plain, 2 non-temporal)
constexpr int kTiledAux = MK_TILED_AUX;    // cache policy of tiled weight loads
constexpr int kKvAux = MK_KV_AUX;          // cache policy of cached K/V loads
constexpr int kPfAux = MK_PF_AUX;          // cache policy of the prefetch loads (they must stay in L2)
__device__ __forceinline__ uint4 buf_load16_w(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamAux);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 buf_load16_wt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kTiledAux);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 buf_load16_kv(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kKvAux);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// agent-coherent variant for data written earlier in the same step
__device__ __forceinline__ uint4 buf_load16_co(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kSC1);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Activations (per-layer buffers written exactly once per step by other
// workgroups, before the event their readers wait on) are read with plain,
// L2-cacheable loads. This is safe because (1) the producers write them with
// agent-coherent stores, which reach memory past every L2, (2) no workgroup
// touches such a buffer before its event fires, so no L2 holds a line of it
// from earlier in the step, and (3) each step starts with an agent-scope
// acquire that drops every line cached in an earlier step. The other
// workgroups of the same XCD then hit in the shared L2 instead of going to
// memory, which matters when every worker reads the whole input vector.
// Buffers reused within a step (attention partials, rings) keep coherent loads.
__device__ __forceinline__ uint4 buf_load16_act(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return buf_load16(r, voff, soff);
}
__device__ __forceinline__ float ld_act(const float* p) { return *p; }

// One weight row as seen by a GEMV: resource of its matrix tile and the
// byte offset of the row inside it.
struct RowRef {
    __amdgpu_buffer_rsrc_t r;
    uint32_t soff;
};

__device__ __forceinline__ void raise_error(Ctrl* c, uint32_t bits) {
    __hip_atomic_fetch_or(&c->error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void raise_abort(Ctrl* c) {
    raise_error(c, MK_ERR_TIMEOUT);
    __hip_atomic_store(&c->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool aborted(Ctrl* c) { return ld_relaxed(&c->abort) != 0; }

}  // namespace mk
