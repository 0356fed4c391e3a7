// Internal records shared by the host planner (plan.cpp) and the device
// runtime (runtime.hip). Plain C++ types only; no HIP headers here.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"

namespace mk {

// Operator of a task. The numbering is also the index into
// mk_plan_info::tasks_per_op.
enum Op : uint8_t {
    OP_NONE = 0,
    OP_QKV = 1,     // [q|k|v] = W_qkv . RMSNorm(x)            (AOT GEMV)
    OP_O = 2,       // x_mid = x + W_o . attn                  (AOT GEMV)
    OP_GATEUP = 3,  // h = silu(W_g . RMSNorm(x_mid)) * (W_u . RMSNorm(x_mid))
    OP_DOWN = 4,    // x_next = x_mid + W_d . h                (AOT GEMV)
    OP_LM = 5,      // logits = W_lm . RMSNorm(x_final)        (AOT GEMV)
    OP_ATTN = 6,    // split-KV attention + last-arrival combine (JIT, or AOT fallback)
    OP_EMBED = 7,   // x_0 = E[token] (AOT row copy)
    OP_APPEND = 8,  // prefill plans: QK-norm + RoPE + K/V store of rows (b, g), before attention
};

constexpr int kNumOps = 9;

// Task record, 32 bytes (the MPK article's TaskDesc, §2.1, as our own
// fixed-size record: operator, tile, the one event it waits on and the one
// it signals).
struct TaskRec {
    uint8_t op;
    uint8_t flags;
    uint16_t layer;
    int32_t a0;       // GEMV/EMBED: first row; ATTN: b * n_kv_heads + g
    int32_t a1;       // GEMV/EMBED: end row;   ATTN: split index
    int32_t wait_ev;  // event to wait on, -1 = none
    int32_t sig_ev;   // event to signal on completion, -1 = none
    int32_t level;    // task-graph level (kernel-per-op grouping, queue order)
    int32_t kpart;    // K-split GEMV: part index | (parts << 8); 0 = whole K
    int32_t kgroup;   // K-split GEMV: the row group (its arrival counter)
};
static_assert(sizeof(TaskRec) == 32, "TaskRec size");
// TaskRec.flags: an attention task of the static schedule, fixed to
// (b * n_kv_heads + g = a0, split = a1)
constexpr uint8_t kTaskStaticAttn = 1;

// Event record (the article's Event, §2.1): the counter itself lives in a
// separate uint32 array and only grows; step e is complete for this event
// when counter - required * (e + 1) >= 0 (wrap-safe signed difference).
struct EventRec {
    uint32_t required;  // producer tasks per step
    int32_t jit_layer;  // >= 0: the completing arrival posts "expand attention of this layer"
};

// One slot of the JIT ready ring or the scheduler mailbox. `tag` is
// position + 1 once the payload is published (monotonic positions).
struct RingSlot {
    int64_t tag;
    int32_t p0;
    int32_t p1;
};

// Device control block (one per plan, zeroed at build).
struct Ctrl {
    uint32_t error;      // sticky mk_device_error bits
    uint32_t abort;      // set when any wait times out; all loops exit
    uint32_t pad00[14];
    uint32_t step_done;  // greedy steps: epoch + 1 of the last step whose tokens and lengths are written
    uint32_t pad0[15];
    int64_t rr;          // round-robin position for dealing JIT tasks to worker inboxes
    int64_t pad1[7];
    int64_t pad2[8];
    int64_t mb_tail;     // mailbox reserve position
    int64_t pad3[7];
    int64_t mb_head;     // mailbox pop position
    int64_t pad4[7];
};

// Host-side plan (task graph) produced by the planner. Device buffers are
// added by the runtime.
struct HostPlan {
    mk_model_desc desc;
    int workers = 0;
    int sched_wgs = 0;
    int jit = 1;  // 1 JIT, 0 AOT attention
    int jit_inline = 0;  // JIT expanded by the completing QKV arrival (no scheduler workgroups)
    int schedule = 0;  // 0 event runtime, 1 static (searched) schedule
    int prefill = 0;   // 1: the batch rows are consecutive positions of one sequence (prompt chunks)
    int down_ks = 1;   // K parts of the down projection (1: whole K)
    int o_ks = 1;      // K parts of the O projection
    int ksplit_groups = 0;  // most row groups of a K-split level (arrival counters)
    double predicted_layer_us = 0;  // static schedule: cost-model time of one layer
    int kv_chunk = 256;     // base keys per split (sizes the partial records)
    int kv_chunk_max = 4096; // largest per-step chunk
    int attn_target = 0;    // split tasks per step above which the chunk doubles
    int max_splits = 0;
    int n_levels = 0;
    int cap = 0;  // KV positions per sequence
    std::vector<TaskRec> tasks;
    std::vector<EventRec> events;
    std::vector<int32_t> queue_off;  // workers + 1
    std::vector<int32_t> queue;      // task ids
    std::vector<int32_t> level_off;  // n_levels + 1 (kernel-per-op)
    std::vector<int32_t> level_tasks;
    std::vector<uint8_t> level_op;   // op of each level
    std::vector<uint16_t> level_layer;
    int inbox_cap = 0;  // JIT inbox slots per worker (power of two)
    int mb_cap = 0;     // power of two
    std::vector<int32_t> jit_elig;  // workers that may receive JIT tasks
    int max_jit_tasks = 0;
    int tasks_per_op[kNumOps] = {0};
    int64_t weight_bytes = 0;
    int64_t kv_bytes_per_token = 0;
};

// Build / validate on the host. Returns false with `err` set on failure.
bool build_host_plan(const mk_model_desc& desc, int device_cus, HostPlan& out, std::string& err);
bool verify_plan(const HostPlan& p, std::string& err);
// Dry run (see mk_plan_dry_run).
bool dry_run(const HostPlan& p, int n_threads, uint64_t seed, int drop_task, int timeout_ms,
             const int32_t* seq_lens, std::string& err);

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

// event id helpers: five events per layer, plus the embedding event
MK_HD inline int ev_qkv(int l) { return 5 * l + 0; }
MK_HD inline int ev_attn(int l) { return 5 * l + 1; }
MK_HD inline int ev_o(int l) { return 5 * l + 2; }
MK_HD inline int ev_gateup(int l) { return 5 * l + 3; }
MK_HD inline int ev_down(int l) { return 5 * l + 4; }
MK_HD inline int ev_embed(int n_layers) { return 5 * n_layers; }
// prefill plans: layer l's appends done
MK_HD inline int ev_append(int l, int n_layers) { return 5 * n_layers + 1 + l; }

MK_HD inline int n_splits_for(int keys, int chunk) { return (keys + chunk - 1) / chunk; }

// Split tasks per step that the attention chunk is sized for: one per
// worker of a 256-CU device, so that a step's split tasks run in one round
// (batch 16, log-uniform lengths: 240 -> 256 took the step from 4.44 to
// 4.40 ms; 272 or 320, a second round for some workers, 5.0 ms). A constant
// (not the worker count), so that results do not depend on how many workers
// a plan uses.
constexpr int kAttnSplitTarget = 256;

// Keys per attention split in one step: the smallest multiple of 16 in
// [c0, cmax] for which the step's split tasks, total(c) = sum over b of
// Hkv * ceil(keys_b / c), number at most `target` (cmax if none does).
// total(c) never grows with c, so a bisection finds it. It depends only on
// the sequence lengths, so every execution mode and every task of the step
// derives the same splits, and hence the same bits. c0 and cmax are
// multiples of 16.
template <typename TotalFn>
MK_HD inline int attn_chunk_search(TotalFn total, int c0, int cmax, int target) {
    if (cmax <= c0 || total(c0) <= (long long)target) return c0;
    if (total(cmax) > (long long)target) return cmax;
    int lo = c0, hi = cmax;  // total(lo) > target >= total(hi)
    while (hi - lo > 16) {
        const int mid = lo + ((hi - lo) / 32) * 16;
        if (total(mid) <= (long long)target) hi = mid;
        else lo = mid;
    }
    return hi;
}
// AOT attention slots per layer, one per split task a step can have: a
// step's chunk gives at most kAttnSplitTarget tasks unless it is capped at
// kv_chunk_max, where a sequence has at most ceil(cap / kv_chunk_max) splits
template <typename Plan>
inline int aot_attn_slots(const Plan& p) {
    const long long bg = (long long)p.desc.batch * p.desc.n_kv_heads;
    const long long most = bg * p.max_splits;
    const long long capped = bg * ((p.cap + p.kv_chunk_max - 1) / p.kv_chunk_max);
    const long long target = most < kAttnSplitTarget ? most : kAttnSplitTarget;
    return (int)(capped > target ? capped : target);
}
// keys counted for sequence length L (tokens cached before the step)
MK_HD inline int attn_keys(int L) { return L < 0 ? 1 : L + 1; }

}  // namespace mk
