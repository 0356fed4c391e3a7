// Persistent megakernel, kernel-per-operator launches and the C ABI.
//
// Persistent mode (MPK article, devpress.csdn.net, §2.1 "Mega-Kernel执行模型"):
// one cooperative launch of (workers + scheduler) workgroups, one per CU.
//  - Worker workgroups walk their ahead-of-time queue. Before a task they
//    wait for its event counter to reach required * (epoch + 1); while
//    waiting they pop just-in-time attention tasks from the ready ring
//    (§2.2: attention is JIT, GEMVs AOT).
//  - Scheduler workgroups run four independent waves each (16 waves with
//    the default four scheduler CUs, §5.1). A wave pops "layer l finished
//    its QKV" messages from the mailbox, reads seq_lens on the device and
//    publishes one attention task per (sequence, KV head, KV split).
//  - Every spin wait is bounded by a watchdog on the 100 MHz real-time
//    counter; on expiry the error word gets MK_ERR_TIMEOUT and every
//    workgroup leaves its loops.
// Kernel-per-operator mode (§1, the execution model MPK replaces) launches
// one kernel per task-graph level running the same task bodies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tasks.h"
#include "kernels.h"

namespace mk {

// argmax over each logits row, lowest index on ties. grid (kArgBlocks, B):
// every block reduces a contiguous slice; the last block of a row to finish
// (arrival counter, self-resetting) reduces the slice winners in order.
constexpr int kArgBlocks = 64;

__device__ __forceinline__ void argmax_merge(float& best, int& bi, float ov, int oi) {
    if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
    }
}

// Winner (value, index) of slice blockIdx.x of row b; valid in thread 0.
// best = -inf with index V when the slice holds no number.
__device__ __forceinline__ void argmax_slice(const float* logits, int V, int b, float& best, int& bi) {
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    const float* row = logits + (int64_t)b * V;
    const int per = (V + kArgBlocks - 1) / kArgBlocks;
    const int i0 = blockIdx.x * per, i1 = min(V, i0 + per);
    best = -INFINITY;
    bi = V;
    for (int i = i0 + (int)threadIdx.x; i < i1; i += kThreads) {
        const float v = row[i];
        if (v > best) {  // strict: lowest index wins ties; NaN never wins
            best = v;
            bi = i;
        }
    }
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = best;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0)
        for (int w = 1; w < kWaves; ++w) argmax_merge(best, bi, sv[w], si[w]);
}

__global__ __launch_bounds__(kThreads) void k_argmax(const float* logits, int V, int32_t* out, float* pv, int32_t* pi,
                                                     uint32_t* cnt) {
    __shared__ int last;
    const int b = blockIdx.y;
    float best;
    int bi;
    argmax_slice(logits, V, b, best, bi);
    if (threadIdx.x == 0) {
        st_co(&pv[b * kArgBlocks + blockIdx.x], best);
        st_co(&pi[b * kArgBlocks + blockIdx.x], bi);
        wait_stores();
        const uint32_t old = __hip_atomic_fetch_add(&cnt[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old + 1u == (uint32_t)kArgBlocks);
    }
    __syncthreads();
    if (!last || threadIdx.x != 0) return;
    best = -INFINITY;
    bi = V;
    for (int k = 0; k < kArgBlocks; ++k) argmax_merge(best, bi, ld_co(&pv[b * kArgBlocks + k]), ld_co(&pi[b * kArgBlocks + k]));
    out[b] = bi < V ? bi : 0;
    __hip_atomic_store(&cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- argmax without allocation
// The slice winners of mk_argmax_noalloc live in this fixed array: one per
// device, for callers that cannot allocate. It is written by k_argmax_part
// and read by k_argmax_final, in stream order, so nothing in it has to start
// at zero. Host code never passes `scratch` itself to a kernel (in host code
// the name is a stand-in, not a device address): it passes the address that
// hipGetSymbolAddress returned for the current device.
constexpr int kNoAllocMaxRows = 256;
struct ArgmaxScratch {
    float v[kNoAllocMaxRows * kArgBlocks];
    int32_t i[kNoAllocMaxRows * kArgBlocks];
};
static __device__ __align__(256) ArgmaxScratch scratch;

__global__ __launch_bounds__(kThreads) void k_argmax_part(const float* logits, int V, ArgmaxScratch* sc) {
    const int b = blockIdx.y;
    float best;
    int bi;
    argmax_slice(logits, V, b, best, bi);
    if (threadIdx.x == 0) {
        sc->v[b * kArgBlocks + blockIdx.x] = best;
        sc->i[b * kArgBlocks + blockIdx.x] = bi;
    }
}

// one wave per row: the slice winners in slice order, lowest index on ties
__global__ __launch_bounds__(64) void k_argmax_final(const ArgmaxScratch* sc, int V, int32_t* out) {
    const int b = blockIdx.x, lane = threadIdx.x;
    float best = sc->v[b * kArgBlocks + lane];
    int bi = sc->i[b * kArgBlocks + lane];
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
    if (lane == 0) out[b] = bi < V ? bi : 0;
}
static_assert(kArgBlocks == 64, "k_argmax_final reduces one slice winner per lane");

// Tiled copy of a row-major bf16 matrix (mk_pack_tiled): one thread per
// 16-byte piece of the destination. Piece j of unit u (8 rows) is 32-column
// step j / 32 and, inside it, (column group, row) = ((j % 32) / 8, j % 8):
// the piece a matrix-core lane (row i, group jj) loads for that step.
__global__ __launch_bounds__(256) void k_pack_tiled(const uint4* src, uint4* dst, int64_t rows, int64_t cols) {
    const int64_t n = rows * cols / 8;  // 16-byte pieces
    const int64_t cp = cols / 8;        // pieces per row
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t u = q / cols, j = q % cols;  // a unit holds 8 * cols elements = cols pieces
        const int64_t step = j / 32, grp = (j % 32) / 8, row = j % 8;
        dst[q] = src[(u * 8 + row) * cp + step * 4 + grp];
    }
}

// prefill chunk: row i takes prompt position min(i, n - 1) of the chunk
__global__ void k_prefill_rows(const int32_t* tokens, int n, int pos, int B, int32_t* ptok, int32_t* plen) {
    const int i = threadIdx.x;
    if (i >= B) return;
    const int j = i < n ? i : n - 1;
    ptok[i] = tokens[j];
    plen[i] = pos + j;
}

}  // namespace mk

// ============================================================================
// host side

using namespace mk;

struct mk_plan {
    HostPlan hp;
    int device = 0;
    int cus = 0;
    bool host_only = false;
    // device memory
    char* dmem = nullptr;
    size_t dbytes = 0;
    TaskRec* d_tasks = nullptr;
    int32_t* d_qoff = nullptr;
    int32_t* d_queue = nullptr;
    int32_t* d_level_tasks = nullptr;
    EventRec* d_evrec = nullptr;
    uint32_t* d_ev = nullptr;
    uint32_t* d_arrive = nullptr;
    float* d_kpart = nullptr;       // K-split down projection: partial tiles
    uint32_t* d_karrive = nullptr;  // K-split down projection: row-group arrivals
    unsigned long long* d_amax = nullptr;  // greedy step: per-sequence argmax keys
    uint32_t* d_lm_done = nullptr;         // greedy step: LM tasks finished (kernel-per-op)
    uint32_t* d_exit_cnt = nullptr;        // greedy step: workers done (persistent)
    RingSlot* d_inbox = nullptr;
    int64_t* d_inbox_tail = nullptr;
    int64_t* d_inbox_head = nullptr;
    int32_t* d_elig = nullptr;
    void* d_zero = nullptr;
    RingSlot* d_mb = nullptr;
    Ctrl* d_ctrl = nullptr;
    float2* d_rope = nullptr;
    float* d_partials = nullptr;
    float* d_act = nullptr;
    float* d_x0 = nullptr;
    float* d_xfinal = nullptr;
    LayerPtrs* d_lw = nullptr;
    float* d_argv = nullptr;
    int32_t* d_argi = nullptr;
    uint32_t* d_argc = nullptr;
    mk_trace_rec* d_trace = nullptr;
    int32_t* d_ptok = nullptr;   // prefill plans: the chunk's tokens
    int32_t* d_plen = nullptr;   // prefill plans: the chunk's positions
    float* d_plogits = nullptr;  // prefill plans: the chunk's logits [batch, vocab]
    int32_t* d_trace_n = nullptr;
    int trace_cap = 0;
    int64_t act_stride = 0, off_qkv = 0, off_attn = 0, off_xmid = 0, off_h = 0, off_xnext = 0;
    size_t ctrl_off = 0, ev_off = 0, arrive_off = 0, jit_off = 0, mb_off = 0, ctrl_bytes = 0;
    // state
    std::vector<LayerPtrs> cached_lw;
    LayerPtrs* h_lw_pinned = nullptr;
    uint32_t epoch = 0;
    int lds_bytes = 0;
    int lds_bytes_persistent = 0;
    int lds_bytes_level = 0;  // kernel-per-op GEMV levels
};

namespace {

thread_local std::string g_err;

void set_err(const std::string& s) { g_err = s; }

bool hip_ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    set_err(std::string(what) + ": " + hipGetErrorString(e));
    return false;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMaxStepsPerLaunch = 4096;

int nb_for(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

void* kernel_for(const mk_plan* pl, int kind) {
    const int nb = nb_for(pl->hp.desc.batch);
    if (pl->hp.desc.weight_dtype == MK_W4 && nb >= 4) {
        switch (nb) {
            case 4: return mk_kernels_bf16_4w(kind);
            case 8: return mk_kernels_bf16_8w(kind);
            default: return mk_kernels_bf16_16w(kind);
        }
    }
    if (pl->hp.desc.weight_dtype == MK_BF16 || pl->hp.desc.weight_dtype == MK_W4) {
        switch (nb) {
            case 1: return pl->hp.desc.opts.lds_stream == 1 ? mk_kernels_bf16_1s(kind) : mk_kernels_bf16_1(kind);
            case 2: return mk_kernels_bf16_2(kind);
            case 4: return mk_kernels_bf16_4(kind);
            case 8: return mk_kernels_bf16_8(kind);
            default: return mk_kernels_bf16_16(kind);
        }
    }
    switch (nb) {
        case 1: return mk_kernels_f32_1(kind);
        case 2: return mk_kernels_f32_2(kind);
        default: return mk_kernels_f32_4(kind);
    }
}
void* persistent_kernel(const mk_plan* pl) { return kernel_for(pl, KK_PERSISTENT); }
void* level_kernel(const mk_plan* pl) { return kernel_for(pl, KK_LEVEL_GEMV); }
void* attn_kernel(const mk_plan* pl) { return kernel_for(pl, KK_LEVEL_ATTN); }

// LDS preload of the awaited GEMV task's first rows (opts.lds_preload = 1):
// persistent mode with ahead-of-time queues (no JIT task may run in the
// wait), the batch <= 2 GEMV, not the LDS-ring variant
bool lds_preload_on(const mk_plan* pl) {
    const mk_model_desc& d = pl->hp.desc;
    return d.opts.mode == MK_PERSISTENT && !pl->hp.jit && nb_for(d.batch) <= 2 && d.opts.lds_stream != 1 &&
           d.opts.lds_preload == 1 && d.weight_dtype != MK_W4;
}

bool upload_plan(mk_plan* pl) {
    const HostPlan& hp = pl->hp;
    const mk_model_desc& d = hp.desc;
    const int L = d.n_layers, B = d.batch, H = d.hidden, F = d.ffn, Hkv = d.n_kv_heads, D = d.head_dim;
    const int G = d.n_heads / Hkv;
    const int64_t QD = (int64_t)d.n_heads * D, KD = (int64_t)Hkv * D;
    // activation layout per layer (floats, 64-float aligned blocks)
    auto a64 = [](int64_t v) { return (v + 63) / 64 * 64; };
    pl->off_qkv = 0;
    pl->off_attn = pl->off_qkv + a64(B * (QD + 2 * KD));
    pl->off_xmid = pl->off_attn + a64(B * QD);
    pl->off_h = pl->off_xmid + a64((int64_t)B * H);
    pl->off_xnext = pl->off_h + a64((int64_t)B * F);
    pl->act_stride = pl->off_xnext + a64((int64_t)B * H);

    struct Region { size_t off, bytes; };
    size_t at = 0;
    auto take = [&](size_t bytes) {
        Region r{align_up(at, 256), bytes};
        at = r.off + bytes;
        return r;
    };
    Region r_tasks = take(sizeof(TaskRec) * std::max<size_t>(1, hp.tasks.size()));
    Region r_qoff = take(sizeof(int32_t) * hp.queue_off.size());
    Region r_queue = take(sizeof(int32_t) * std::max<size_t>(1, hp.queue.size()));
    Region r_lvl = take(sizeof(int32_t) * std::max<size_t>(1, hp.level_tasks.size()));
    Region r_evrec = take(sizeof(EventRec) * hp.events.size());
    // zero-initialised control area: events, arrivals, rings, ctrl
    Region r_ev = take(sizeof(uint32_t) * (size_t)ev_plane_stride((int)hp.events.size()) * kEvPlanesMax);
    Region r_arr = take(sizeof(uint32_t) * (size_t)B * Hkv);
    // K-split levels (O, down: hidden rows each) share the partial tiles and
    // counters: a level's merges all complete before its event fires, and the
    // next split level waits (through the events) on that one
    const int kmax = std::max(hp.down_ks, hp.o_ks);
    Region r_karr = take(sizeof(uint32_t) * (size_t)std::max(1, hp.ksplit_groups));
    Region r_kpart = take(kmax > 1 ? sizeof(float) * (size_t)H * kmax * 16 : 0);
    Region r_amax = take(sizeof(unsigned long long) * (size_t)B);
    Region r_lmd = take(sizeof(uint32_t));
    Region r_exit = take(sizeof(uint32_t));
    Region r_inbox = take(sizeof(RingSlot) * (size_t)hp.workers * hp.inbox_cap);
    Region r_itail = take(sizeof(int64_t) * (size_t)hp.workers);
    Region r_ihead = take(sizeof(int64_t) * (size_t)hp.workers);
    Region r_mb = take(sizeof(RingSlot) * (size_t)hp.mb_cap);
    Region r_ctrl = take(sizeof(Ctrl));
    Region r_rope = take(sizeof(float2) * (size_t)hp.cap * (D / 2));
    Region r_part = take(sizeof(float) * (size_t)B * Hkv * hp.max_splits * attn_rec(G, D));
    Region r_act = take(sizeof(float) * (size_t)L * pl->act_stride);
    Region r_x0 = take(sizeof(float) * (size_t)B * H);
    Region r_xf = take(sizeof(float) * (size_t)B * H);
    Region r_lw = take(sizeof(LayerPtrs) * L);
    Region r_zero = take(64 * 1024);
    Region r_elig = take(sizeof(int32_t) * std::max<size_t>(1, hp.jit_elig.size()));
    Region r_argv = take(sizeof(float) * (size_t)B * kArgBlocks);
    Region r_argi = take(sizeof(int32_t) * (size_t)B * kArgBlocks);
    Region r_argc = take(sizeof(uint32_t) * (size_t)B);
    pl->trace_cap = d.opts.trace > 0 ? d.opts.trace : 0;
    Region r_tr = take(sizeof(mk_trace_rec) * (size_t)hp.workers * pl->trace_cap);
    Region r_trn = take(sizeof(int32_t) * (size_t)hp.workers);
    Region r_ptok = take(hp.prefill ? sizeof(int32_t) * (size_t)B : 0);
    Region r_plen = take(hp.prefill ? sizeof(int32_t) * (size_t)B : 0);
    Region r_plog = take(hp.prefill ? sizeof(float) * (size_t)B * d.vocab : 0);
    pl->dbytes = align_up(at, 256);
    if (!hip_ok(hipSetDevice(pl->device), "hipSetDevice")) return false;
    if (!hip_ok(hipMalloc((void**)&pl->dmem, pl->dbytes), "hipMalloc(plan)")) return false;
    if (!hip_ok(hipMemset(pl->dmem, 0, pl->dbytes), "hipMemset(plan)")) return false;
    char* m = pl->dmem;
    pl->d_tasks = (TaskRec*)(m + r_tasks.off);
    pl->d_qoff = (int32_t*)(m + r_qoff.off);
    pl->d_queue = (int32_t*)(m + r_queue.off);
    pl->d_level_tasks = (int32_t*)(m + r_lvl.off);
    pl->d_evrec = (EventRec*)(m + r_evrec.off);
    pl->d_ev = (uint32_t*)(m + r_ev.off);
    pl->d_arrive = (uint32_t*)(m + r_arr.off);
    pl->d_karrive = (uint32_t*)(m + r_karr.off);
    pl->d_kpart = kmax > 1 ? (float*)(m + r_kpart.off) : nullptr;
    pl->d_amax = (unsigned long long*)(m + r_amax.off);
    pl->d_lm_done = (uint32_t*)(m + r_lmd.off);
    pl->d_exit_cnt = (uint32_t*)(m + r_exit.off);
    pl->d_inbox = (RingSlot*)(m + r_inbox.off);
    pl->d_inbox_tail = (int64_t*)(m + r_itail.off);
    pl->d_inbox_head = (int64_t*)(m + r_ihead.off);
    pl->d_mb = (RingSlot*)(m + r_mb.off);
    pl->d_ctrl = (Ctrl*)(m + r_ctrl.off);
    pl->d_rope = (float2*)(m + r_rope.off);
    pl->d_partials = (float*)(m + r_part.off);
    pl->d_act = (float*)(m + r_act.off);
    pl->d_x0 = (float*)(m + r_x0.off);
    pl->d_xfinal = (float*)(m + r_xf.off);
    pl->d_lw = (LayerPtrs*)(m + r_lw.off);
    pl->d_elig = (int32_t*)(m + r_elig.off);
    pl->d_zero = m + r_zero.off;
    pl->d_argv = (float*)(m + r_argv.off);
    pl->d_argi = (int32_t*)(m + r_argi.off);
    pl->d_argc = (uint32_t*)(m + r_argc.off);
    pl->d_trace = pl->trace_cap ? (mk_trace_rec*)(m + r_tr.off) : nullptr;
    pl->d_trace_n = (int32_t*)(m + r_trn.off);
    if (hp.prefill) {
        pl->d_ptok = (int32_t*)(m + r_ptok.off);
        pl->d_plen = (int32_t*)(m + r_plen.off);
        pl->d_plogits = (float*)(m + r_plog.off);
    }
    pl->ctrl_off = r_ev.off;
    pl->ctrl_bytes = r_ctrl.off + r_ctrl.bytes - r_ev.off;
    auto up = [&](void* dst, const void* src, size_t n) {
        return n == 0 || hip_ok(hipMemcpy(dst, src, n, hipMemcpyHostToDevice), "hipMemcpy(plan tables)");
    };
    if (!up(pl->d_tasks, hp.tasks.data(), sizeof(TaskRec) * hp.tasks.size())) return false;
    if (!up(pl->d_qoff, hp.queue_off.data(), sizeof(int32_t) * hp.queue_off.size())) return false;
    if (!up(pl->d_queue, hp.queue.data(), sizeof(int32_t) * hp.queue.size())) return false;
    if (!up(pl->d_level_tasks, hp.level_tasks.data(), sizeof(int32_t) * hp.level_tasks.size())) return false;
    if (!up(pl->d_evrec, hp.events.data(), sizeof(EventRec) * hp.events.size())) return false;
    if (!up(pl->d_elig, hp.jit_elig.data(), sizeof(int32_t) * hp.jit_elig.size())) return false;
    // RoPE table: theta_i = pos * base^(-2i/D), cos/sin in double, stored as float
    std::vector<float2> rope((size_t)hp.cap * (D / 2));
    for (int pos = 0; pos < hp.cap; ++pos)
        for (int i = 0; i < D / 2; ++i) {
            const double th = (double)pos * std::pow((double)d.rope_base, -2.0 * (double)i / (double)D);
            rope[(size_t)pos * (D / 2) + i] = make_float2((float)std::cos(th), (float)std::sin(th));
        }
    if (!up(pl->d_rope, rope.data(), sizeof(float2) * rope.size())) return false;
    if (!hip_ok(hipHostMalloc((void**)&pl->h_lw_pinned, sizeof(LayerPtrs) * L, hipHostMallocDefault), "hipHostMalloc"))
        return false;
    pl->lds_bytes = lds_bytes_for(hp.kv_chunk_max, d.kv_layout == MK_KV_PAGED ? d.kv_block : 1, d.kv_layout == MK_KV_PAGED);
    // one workgroup per CU: the LDS-ring variant's static page ring already
    // takes more than half of the CU's LDS; other kernels reserve it dynamically
    const bool ring = nb_for(d.batch) == 1 && d.weight_dtype != MK_F32 && d.opts.lds_stream == 1;
    pl->lds_bytes_persistent = ring ? pl->lds_bytes : std::max(pl->lds_bytes, 82 * 1024);
    if (lds_preload_on(pl)) pl->lds_bytes_persistent = std::max(pl->lds_bytes_persistent, lds_bytes_preload());
    // a W4 matrix-core GEMV (batch >= 3) stages a pass's scales after the partial sums
    pl->lds_bytes_level = lds_bytes_gemv();
    if (d.weight_dtype == MK_W4 && nb_for(d.batch) >= 4) {
        pl->lds_bytes_level = lds_bytes_gemv() + kW4ScaleLdsBytes;
        pl->lds_bytes_persistent = std::max(pl->lds_bytes_persistent, pl->lds_bytes_level);
    }
    // 160 KB per CU, less the statically declared prefetch sink (4 KB)
    if (pl->lds_bytes_persistent > 156 * 1024) {
        set_err("LDS need exceeds 156 KB of dynamic LDS (reduce kv_chunk_max)");
        return false;
    }
    void* kp = persistent_kernel(pl);
    void* kl = level_kernel(pl);
    void* ka = attn_kernel(pl);
    if (!hip_ok(hipFuncSetAttribute(kp, hipFuncAttributeMaxDynamicSharedMemorySize, pl->lds_bytes_persistent),
                "hipFuncSetAttribute(persistent)"))
        return false;
    if (!hip_ok(hipFuncSetAttribute(kl, hipFuncAttributeMaxDynamicSharedMemorySize, pl->lds_bytes_level), "hipFuncSetAttribute"))
        return false;
    if (!hip_ok(hipFuncSetAttribute(ka, hipFuncAttributeMaxDynamicSharedMemorySize, pl->lds_bytes), "hipFuncSetAttribute"))
        return false;
    // every persistent workgroup must be co-resident
    int per_cu = 0;
    if (!hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kp, kThreads, pl->lds_bytes_persistent),
                "hipOccupancyMaxActiveBlocksPerMultiprocessor"))
        return false;
    if (per_cu < 1 || (int64_t)per_cu * pl->cus < hp.workers + hp.sched_wgs) {
        set_err("persistent grid cannot be co-resident on this device");
        return false;
    }
    return true;
}

KParams make_params(const mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const int32_t* tokens,
                    const int32_t* seq_lens, const float* x_in, float* out) {
    const HostPlan& hp = pl->hp;
    const mk_model_desc& d = hp.desc;
    KParams p{};
    p.n_steps = 1;
    p.tasks = pl->d_tasks;
    p.qoff = pl->d_qoff;
    p.queue = pl->d_queue;
    p.evrec = pl->d_evrec;
    p.ev = pl->d_ev;
    p.ev_stride = ev_plane_stride((int)hp.events.size());
    p.arrive = pl->d_arrive;
    p.kpart = pl->d_kpart;
    p.karrive = pl->d_karrive;
    p.amax = pl->d_amax;
    p.lm_done = pl->d_lm_done;
    p.exit_cnt = pl->d_exit_cnt;
    p.n_lm_tasks = hp.tasks_per_op[OP_LM];
    p.inbox = pl->d_inbox;
    p.inbox_tail = pl->d_inbox_tail;
    p.inbox_head = pl->d_inbox_head;
    p.elig = pl->d_elig;
    p.mb = pl->d_mb;
    p.ctrl = pl->d_ctrl;
    p.rope = pl->d_rope;
    p.partials = pl->d_partials;
    p.act = pl->d_act;
    p.act_stride = pl->act_stride;
    p.off_qkv = pl->off_qkv;
    p.off_attn = pl->off_attn;
    p.off_xmid = pl->off_xmid;
    p.off_h = pl->off_h;
    p.off_xnext = pl->off_xnext;
    if (d.hidden_io) {
        p.x0 = x_in;
        p.x0_w = nullptr;
        p.x_final = out;
        p.logits = nullptr;
    } else {
        p.x0 = pl->d_x0;
        p.x0_w = pl->d_x0;
        p.x_final = pl->d_xfinal;
        p.logits = out;
    }
    p.lw = pl->d_lw;
    p.zero = pl->d_zero;
    p.embed = w->embed;
    p.final_norm = w->final_norm;
    p.lm_head = w->lm_head;
    p.kv_k = kv->k;
    p.kv_v = kv->v;
    p.kv_layer_stride = kv->layer_stride;
    p.block_table = kv->block_table;
    p.n_pool_blocks = d.kv_layout == MK_KV_PAGED
                          ? (int)(kv->layer_stride / ((int64_t)d.n_kv_heads * d.kv_block * d.head_dim))
                          : 0;
    p.tokens = tokens;
    p.seq_lens = seq_lens;
    p.B = d.batch;
    p.H = d.hidden;
    p.Hq = d.n_heads;
    p.Hkv = d.n_kv_heads;
    p.D = d.head_dim;
    p.F = d.ffn;
    p.V = d.vocab;
    p.L = d.n_layers;
    p.QD = d.n_heads * d.head_dim;
    p.KD = d.n_kv_heads * d.head_dim;
    p.cap = hp.cap;
    p.chunk = hp.kv_chunk;
    p.chunk_max = hp.kv_chunk_max;
    p.attn_target = hp.attn_target;
    p.max_splits = hp.max_splits;
    p.qk_norm = d.qk_norm;
    p.paged = d.kv_layout == MK_KV_PAGED;
    p.kv_block = d.kv_layout == MK_KV_PAGED ? d.kv_block : 1;
    p.max_blocks = d.max_blocks_per_seq;
    p.eps = d.rms_eps;
    p.scale = (float)(1.0 / std::sqrt((double)d.head_dim));
    p.epoch = pl->epoch;
    p.n_workers = hp.workers;
    p.jit_on = hp.jit ? (hp.jit_inline ? 2 : 1) : 0;
    p.persistent = d.opts.mode == MK_PERSISTENT ? 1 : 0;
    p.inbox_mask = hp.inbox_cap - 1;
    p.n_elig = (int)hp.jit_elig.size();
    p.mb_mask = hp.mb_cap - 1;
    const int wd = d.opts.watchdog_ms > 0 ? d.opts.watchdog_ms : 2000;
    p.watchdog_ticks = (uint64_t)wd * 100000ull;
    // default: on for the batch <= 2 instances (batch 1: 3.76 -> 3.55 ms/step),
    // off for the matrix-core ones, whose non-temporal streams lost to the
    // L2 prefetch (batch 16 4.60 -> 4.44, paged batch 8 6.20 -> 6.11, W4 batch
    // 16 6.58 -> 6.16 ms/step with it off)
    p.prefetch_kb = d.opts.prefetch_kb == 0 ? (nb_for(d.batch) <= 2 ? 256 : 0)
                                            : (d.opts.prefetch_kb < 0 ? 0 : d.opts.prefetch_kb);
    p.pre_slots = lds_preload_on(pl) ? kPreSlots : 0;
    p.w4 = d.weight_dtype == MK_W4 ? 1 : 0;
    p.wtiled = d.weight_layout == MK_WEIGHTS_TILED ? 1 : 0;
    p.prefill = hp.prefill;
    p.trace = pl->d_trace;
    p.trace_n = pl->d_trace_n;
    p.trace_cap = pl->trace_cap;
    return p;
}

// Arguments are checked before the plan's state, so that a host-only plan
// reports a bad argument the same way a device plan does.
int check_step_args(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const int32_t* seq_lens, const void* in,
                    const void* out) {
    if (!pl) return set_err("null plan"), MK_ERR_ARG;
    const mk_model_desc& d = pl->hp.desc;
    if (!w || !kv || !seq_lens || !in || !out) return set_err("null argument"), MK_ERR_ARG;
    if (w->n_layers != d.n_layers || !w->layers) return set_err("weights.n_layers does not match the plan"), MK_ERR_ARG;
    if (!kv->k || !kv->v) return set_err("null KV cache pointer"), MK_ERR_ARG;
    if (d.kv_layout == MK_KV_PAGED && !kv->block_table) return set_err("paged plan needs a block table"), MK_ERR_ARG;
    {
        // attention reads K/V through buffer resources with 32-bit byte
        // offsets: a contiguous sequence span (checked at build) or a paged
        // layer must stay below 2^31 bytes
        const int64_t es = d.kv_dtype == MK_BF16 ? 2 : 4;
        const int64_t blk = (int64_t)d.n_kv_heads * d.kv_block * d.head_dim;
        if (d.kv_layout == MK_KV_PAGED) {
            if (kv->layer_stride < blk || kv->layer_stride % blk)
                return set_err("paged KV: layer_stride must be a positive multiple of n_kv_heads * kv_block * head_dim"),
                       MK_ERR_ARG;
            if (kv->layer_stride * es >= ((int64_t)1 << 31))
                return set_err("paged KV: one layer's pool must be smaller than 2 GiB (32-bit buffer offsets)"), MK_ERR_ARG;
        } else if (kv->layer_stride < (int64_t)(pl->hp.prefill ? 1 : d.batch) * d.n_kv_heads * d.max_seq_len * d.head_dim) {
            // a prefill plan's rows all use sequence 0
            return set_err("contiguous KV: layer_stride is smaller than sequences * n_kv_heads * max_seq_len * head_dim"),
                   MK_ERR_ARG;
        }
    }
    if (!d.hidden_io && (!w->embed || !w->lm_head || !w->final_norm))
        return set_err("embed, lm_head and final_norm are required"), MK_ERR_ARG;
    for (int l = 0; l < d.n_layers; ++l) {
        const mk_layer_weights& lw = w->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.mlp_norm || !lw.w_gate || !lw.w_up || !lw.w_down)
            return set_err("null weight pointer in layer " + std::to_string(l)), MK_ERR_ARG;
        if (d.qk_norm && (!lw.q_norm || !lw.k_norm)) return set_err("qk_norm needs q_norm and k_norm"), MK_ERR_ARG;
    }
    if (pl->host_only) return set_err("host-only plan cannot run steps"), MK_ERR_STATE;
    return MK_OK;
}

// pointer table re-upload only when a pointer changed (a captured or cached
// launch must never run with stale pointers)
int sync_pointer_table(mk_plan* pl, const mk_weights* w, hipStream_t st) {
    const int L = pl->hp.desc.n_layers;
    bool same = (int)pl->cached_lw.size() == L &&
                std::memcmp(pl->cached_lw.data(), w->layers, sizeof(LayerPtrs) * L) == 0;
    if (same) return MK_OK;
    if (!hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize")) return MK_ERR_HIP;
    std::memcpy(pl->h_lw_pinned, w->layers, sizeof(LayerPtrs) * L);
    if (!hip_ok(hipMemcpyAsync(pl->d_lw, pl->h_lw_pinned, sizeof(LayerPtrs) * L, hipMemcpyHostToDevice, st),
                "hipMemcpyAsync(pointer table)"))
        return MK_ERR_HIP;
    pl->cached_lw.assign((const LayerPtrs*)w->layers, (const LayerPtrs*)w->layers + L);
    return MK_OK;
}

// One step (n_steps = 1) or, with the greedy choice, n_steps greedy steps:
// one persistent launch, or n_steps rounds of kernel-per-op level launches.
int launch_step(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const int32_t* tokens, const int32_t* seq_lens,
                const float* x_in, float* out, hipStream_t st, int32_t* greedy_tokens = nullptr,
                int32_t* greedy_lens = nullptr, int n_steps = 1, int32_t* out_tokens = nullptr) {
    if (!hip_ok(hipSetDevice(pl->device), "hipSetDevice")) return MK_ERR_HIP;
    int rc = sync_pointer_table(pl, w, st);
    if (rc) return rc;
    KParams p = make_params(pl, w, kv, tokens, seq_lens, x_in, out);
    p.greedy_tokens = greedy_tokens;
    p.greedy_lens = greedy_lens;
    p.out_tokens = out_tokens;
    p.n_steps = n_steps;
    const HostPlan& hp = pl->hp;
    if (hp.desc.opts.mode == MK_PERSISTENT) {
        void* args[] = {&p};
        if (!hip_ok(hipLaunchCooperativeKernel(persistent_kernel(pl), dim3(hp.workers + hp.sched_wgs), dim3(kThreads), args,
                                               pl->lds_bytes_persistent, st),
                    "hipLaunchCooperativeKernel"))
            return MK_ERR_HIP;
        pl->epoch += (uint32_t)n_steps;
        return MK_OK;
    }
    p.n_steps = 1;
    for (int step = 0; step < n_steps; ++step) {
    p.out_tokens = out_tokens ? out_tokens + (int64_t)step * hp.desc.batch : nullptr;
    for (int lv = 0; lv < hp.n_levels; ++lv) {
        const int op = hp.level_op[lv];
        if (op == OP_ATTN) {
            int layer = hp.level_layer[lv];
            void* args[] = {&p, &layer};
            const int grid = hp.desc.batch * hp.desc.n_kv_heads * hp.max_splits;
            if (!hip_ok(hipLaunchKernel(attn_kernel(pl), dim3(grid), dim3(kThreads), args, pl->lds_bytes, st),
                        "hipLaunchKernel(attention level)"))
                return MK_ERR_HIP;
        } else {
            const int n = hp.level_off[lv + 1] - hp.level_off[lv];
            if (n == 0) continue;
            const int32_t* ids = pl->d_level_tasks + hp.level_off[lv];
            void* args[] = {&p, (void*)&ids};
            if (!hip_ok(hipLaunchKernel(level_kernel(pl), dim3(n), dim3(kThreads), args, pl->lds_bytes_level, st),
                        "hipLaunchKernel(level)"))
                return MK_ERR_HIP;
        }
    }
    }  // step
    return MK_OK;
}

}  // namespace

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

mk_plan* mk_build_graph(const mk_model_desc* desc) {
    if (!desc) {
        set_err("null desc");
        return nullptr;
    }
    mk_plan* pl = new mk_plan();
    pl->host_only = desc->opts.host_only != 0;
    int cus = desc->opts.device_cus > 0 ? desc->opts.device_cus : 256;
    if (!pl->host_only) {
        hipDeviceProp_t prop;
        if (!hip_ok(hipGetDevice(&pl->device), "hipGetDevice") ||
            !hip_ok(hipGetDeviceProperties(&prop, pl->device), "hipGetDeviceProperties")) {
            delete pl;
            return nullptr;
        }
        cus = prop.multiProcessorCount;
        if (!prop.cooperativeLaunch && desc->opts.mode == MK_PERSISTENT) {
            set_err("device does not support cooperative launch");
            delete pl;
            return nullptr;
        }
    }
    pl->cus = cus;
    std::string err;
    if (!build_host_plan(*desc, cus, pl->hp, err) || !verify_plan(pl->hp, err)) {
        set_err(err);
        delete pl;
        return nullptr;
    }
    if (pl->host_only) return pl;
    if (!upload_plan(pl)) {
        mk_destroy_plan(pl);
        return nullptr;
    }
    return pl;
}

void mk_destroy_plan(mk_plan* pl) {
    if (!pl) return;
    if (!pl->host_only) {
        (void)hipSetDevice(pl->device);
        (void)hipDeviceSynchronize();
        if (pl->dmem) (void)hipFree(pl->dmem);
        if (pl->h_lw_pinned) (void)hipHostFree(pl->h_lw_pinned);
    }
    delete pl;
}

int mk_plan_query(const mk_plan* pl, mk_plan_info* info) {
    if (!pl || !info) return set_err("null argument"), MK_ERR_ARG;
    const HostPlan& hp = pl->hp;
    std::memset(info, 0, sizeof(*info));
    info->workers = hp.workers;
    info->sched_waves = hp.sched_wgs * 4;
    info->n_aot_tasks = (int32_t)hp.tasks.size();
    info->n_events = (int32_t)hp.events.size();
    info->n_levels = hp.n_levels;
    info->max_jit_tasks = hp.max_jit_tasks;
    info->kv_chunk = hp.kv_chunk;
    info->max_splits = hp.max_splits;
    for (int i = 0; i < 12 && i < kNumOps; ++i) info->tasks_per_op[i] = hp.tasks_per_op[i];
    info->weight_bytes_per_step = hp.weight_bytes;
    info->kv_bytes_per_token = hp.kv_bytes_per_token;
    info->device_bytes = (int64_t)pl->dbytes;
    info->jit = hp.jit_inline ? 3 : hp.jit;
    info->mode = hp.desc.opts.mode;
    info->host_only = pl->host_only ? 1 : 0;
    info->schedule = hp.schedule;
    info->predicted_layer_us = hp.predicted_layer_us;
    return MK_OK;
}

int mk_decode_step(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const int32_t* tokens,
                   const int32_t* seq_lens, float* logits, void* stream) {
    int rc = check_step_args(pl, w, kv, seq_lens, tokens, logits);
    if (rc) return rc;
    if (pl->hp.desc.hidden_io) return set_err("hidden_io plan: use mk_decode_step_hidden"), MK_ERR_STATE;
    if (pl->hp.prefill) return set_err("prefill plan: use mk_prefill"), MK_ERR_STATE;
    return launch_step(pl, w, kv, tokens, seq_lens, nullptr, logits, (hipStream_t)stream);
}

int mk_decode_step_greedy(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, int32_t* tokens,
                          int32_t* seq_lens, float* logits, void* stream) {
    int rc = check_step_args(pl, w, kv, seq_lens, tokens, logits);
    if (rc) return rc;
    if (pl->hp.desc.hidden_io) return set_err("hidden_io plan has no logits"), MK_ERR_STATE;
    if (pl->hp.prefill) return set_err("prefill plan: use mk_prefill"), MK_ERR_STATE;
    return launch_step(pl, w, kv, tokens, seq_lens, nullptr, logits, (hipStream_t)stream, tokens, seq_lens);
}

int mk_decode_steps_greedy(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, int32_t* tokens,
                           int32_t* seq_lens, float* logits, int32_t n_steps, int32_t* out_tokens, void* stream) {
    int rc = check_step_args(pl, w, kv, seq_lens, tokens, logits);
    if (rc) return rc;
    if (pl->hp.desc.hidden_io) return set_err("hidden_io plan has no logits"), MK_ERR_STATE;
    if (pl->hp.prefill) return set_err("prefill plan: use mk_prefill"), MK_ERR_STATE;
    if (n_steps < 1 || n_steps > kMaxStepsPerLaunch)
        return set_err("n_steps must be in [1, " + std::to_string(kMaxStepsPerLaunch) + "]"), MK_ERR_ARG;
    if (pl->hp.desc.opts.mode == MK_PERSISTENT && n_steps > 1 && (pl->hp.jit || pl->hp.desc.opts.lds_stream == 1))
        return set_err("several steps per launch need ahead-of-time attention (opts.jit 0 or 2, no lds_stream)"),
               MK_ERR_UNSUPPORTED;
    return launch_step(pl, w, kv, tokens, seq_lens, nullptr, logits, (hipStream_t)stream, tokens, seq_lens, n_steps,
                       out_tokens);
}

int mk_prefill(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const int32_t* tokens, int32_t pos0, int32_t T,
               float* logits, void* stream) {
    if (!pl) return set_err("null plan"), MK_ERR_ARG;
    if (!tokens || !logits) return set_err("null argument"), MK_ERR_ARG;
    const mk_model_desc& d = pl->hp.desc;
    if (T < 1 || pos0 < 0 || (int64_t)pos0 + T > d.max_seq_len)
        return set_err("prefill needs T >= 1, pos0 >= 0 and pos0 + T <= max_seq_len"), MK_ERR_ARG;
    int rc = check_step_args(pl, w, kv, tokens, tokens, logits);
    if (rc) return rc;
    if (!pl->hp.prefill) return set_err("mk_prefill needs a plan built with opts.prefill = 1"), MK_ERR_STATE;
    hipStream_t st = (hipStream_t)stream;
    const int B = d.batch;
    int n = 0;
    for (int c = 0; c < T; c += B) {
        n = std::min(B, T - c);
        hipLaunchKernelGGL(k_prefill_rows, dim3(1), dim3(64), 0, st, tokens + c, n, pos0 + c, B, pl->d_ptok, pl->d_plen);
        if (!hip_ok(hipGetLastError(), "k_prefill_rows launch")) return MK_ERR_HIP;
        rc = launch_step(pl, w, kv, pl->d_ptok, pl->d_plen, nullptr, pl->d_plogits, st);
        if (rc) return rc;
    }
    if (!hip_ok(hipMemcpyAsync(logits, pl->d_plogits + (size_t)(n - 1) * d.vocab, sizeof(float) * d.vocab,
                               hipMemcpyDeviceToDevice, st),
                "hipMemcpyAsync(prefill logits)"))
        return MK_ERR_HIP;
    return MK_OK;
}

int mk_decode_step_hidden(mk_plan* pl, const mk_weights* w, const mk_kv_cache* kv, const float* x_in,
                          const int32_t* seq_lens, float* x_out, void* stream) {
    int rc = check_step_args(pl, w, kv, seq_lens, x_in, x_out);
    if (rc) return rc;
    if (!pl->hp.desc.hidden_io) return set_err("token plan: use mk_decode_step"), MK_ERR_STATE;
    if ((const void*)x_in == (const void*)x_out) return set_err("x_in and x_out must not alias"), MK_ERR_ARG;
    return launch_step(pl, w, kv, nullptr, seq_lens, x_in, x_out, (hipStream_t)stream);
}

int mk_get_device_error(mk_plan* pl, void* stream) {
    if (!pl) return set_err("null plan"), MK_ERR_ARG;
    if (pl->host_only) return set_err("host-only plan"), MK_ERR_STATE;
    hipStream_t st = (hipStream_t)stream;
    if (!hip_ok(hipSetDevice(pl->device), "hipSetDevice") || !hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize"))
        return MK_ERR_HIP;
    Ctrl c;
    if (!hip_ok(hipMemcpy(&c, pl->d_ctrl, sizeof(Ctrl), hipMemcpyDeviceToHost), "hipMemcpy(error word)")) return MK_ERR_HIP;
    const int bits = (int)c.error;
    if (bits) {
        if (bits & MK_ERR_TIMEOUT) {
            // counters are inconsistent after an aborted step: restart from epoch 0
            if (!hip_ok(hipMemset(pl->dmem + pl->ctrl_off, 0, pl->ctrl_bytes), "hipMemset(reset)")) return MK_ERR_HIP;
            pl->epoch = 0;
        } else {
            uint32_t z = 0;
            if (!hip_ok(hipMemcpy(&pl->d_ctrl->error, &z, sizeof(z), hipMemcpyHostToDevice), "hipMemcpy(clear)"))
                return MK_ERR_HIP;
        }
    }
    return bits;
}

int mk_argmax(const mk_plan* pl, const float* logits, int32_t* out_tokens, void* stream) {
    if (!pl || !logits || !out_tokens) return set_err("null argument"), MK_ERR_ARG;
    if (pl->host_only) return set_err("host-only plan"), MK_ERR_STATE;
    if (pl->hp.desc.hidden_io) return set_err("hidden_io plan has no logits"), MK_ERR_STATE;
    hipLaunchKernelGGL(k_argmax, dim3(kArgBlocks, pl->hp.desc.batch), dim3(kThreads), 0, (hipStream_t)stream, logits,
                       pl->hp.desc.vocab, out_tokens, pl->d_argv, pl->d_argi, pl->d_argc);
    if (!hip_ok(hipGetLastError(), "k_argmax launch")) return MK_ERR_HIP;
    return MK_OK;
}

int mk_argmax_noalloc(const float* logits, int32_t batch, int32_t vocab, int32_t* out_tokens, void* stream) {
    if (!logits || !out_tokens) return set_err("null argument"), MK_ERR_ARG;
    if (batch < 1 || batch > kNoAllocMaxRows)
        return set_err("mk_argmax_noalloc: batch must be in [1, " + std::to_string(kNoAllocMaxRows) + "]"), MK_ERR_ARG;
    if (vocab < 1) return set_err("mk_argmax_noalloc: vocab must be positive"), MK_ERR_ARG;
    // the array's address on the current device, looked up once per device
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev), "hipGetDevice")) return MK_ERR_HIP;
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> g(mu);
        if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
        if (!addr[dev]) {
            void* a = nullptr;
            if (!hip_ok(hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return MK_ERR_HIP;
            addr[dev] = a;
        }
        ptr = addr[dev];
    }
    ArgmaxScratch* sc = (ArgmaxScratch*)ptr;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k_argmax_part, dim3(kArgBlocks, batch), dim3(kThreads), 0, st, logits, vocab, sc);
    if (!hip_ok(hipGetLastError(), "k_argmax_part launch")) return MK_ERR_HIP;
    hipLaunchKernelGGL(k_argmax_final, dim3(batch), dim3(64), 0, st, (const ArgmaxScratch*)sc, vocab, out_tokens);
    if (!hip_ok(hipGetLastError(), "k_argmax_final launch")) return MK_ERR_HIP;
    return MK_OK;
}

int mk_pack_tiled(const void* src, void* dst, int64_t rows, int64_t cols, void* stream) {
    if (!src || !dst) return set_err("mk_pack_tiled: null pointer"), MK_ERR_ARG;
    if (rows < 8 || rows % 8 || cols < 64 || cols % 64)
        return set_err("mk_pack_tiled: rows must be a positive multiple of 8 and cols of 64"), MK_ERR_ARG;
    const int64_t pieces = rows * cols / 8;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, nb = (uintptr_t)pieces * 16u;
    if (a < b + nb && b < a + nb) return set_err("mk_pack_tiled: src and dst must not overlap"), MK_ERR_ARG;
    const int blocks = (int)std::min<int64_t>((pieces + 255) / 256, 65536);
    hipLaunchKernelGGL(k_pack_tiled, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                       rows, cols);
    if (!hip_ok(hipGetLastError(), "k_pack_tiled launch")) return MK_ERR_HIP;
    return MK_OK;
}

int mk_plan_trace(const mk_plan* pl, mk_trace_rec* out, int64_t max_records, void* stream) {
    if (!pl || (!out && max_records > 0)) return set_err("null argument"), MK_ERR_ARG;
    if (pl->host_only || !pl->d_trace) return set_err("plan built without trace"), MK_ERR_STATE;
    if (!hip_ok(hipSetDevice(pl->device), "hipSetDevice") ||
        !hip_ok(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize"))
        return MK_ERR_HIP;
    const int W = pl->hp.workers;
    std::vector<int32_t> n(W);
    std::vector<mk_trace_rec> all((size_t)W * pl->trace_cap);
    if (!hip_ok(hipMemcpy(n.data(), pl->d_trace_n, sizeof(int32_t) * W, hipMemcpyDeviceToHost), "hipMemcpy(trace)") ||
        !hip_ok(hipMemcpy(all.data(), pl->d_trace, sizeof(mk_trace_rec) * all.size(), hipMemcpyDeviceToHost),
                "hipMemcpy(trace)"))
        return MK_ERR_HIP;
    int64_t k = 0;
    for (int w = 0; w < W; ++w)
        for (int i = 0; i < std::min(n[w], pl->trace_cap) && k < max_records; ++i) out[k++] = all[(size_t)w * pl->trace_cap + i];
    return (int)k;
}

int mk_plan_verify(const mk_plan* pl) {
    if (!pl) return set_err("null plan"), MK_ERR_ARG;
    std::string err;
    if (!verify_plan(pl->hp, err)) return set_err(err), MK_ERR_STATE;
    return MK_OK;
}

int mk_plan_dry_run(const mk_plan* pl, int n_threads, uint64_t seed, int drop_task, int timeout_ms,
                    const int32_t* seq_lens_host) {
    if (!pl) return set_err("null plan"), MK_ERR_ARG;
    std::string err;
    if (!dry_run(pl->hp, n_threads, seed, drop_task, timeout_ms, seq_lens_host, err)) return set_err(err), MK_ERR_STATE;
    return MK_OK;
}

}  // extern "C"
