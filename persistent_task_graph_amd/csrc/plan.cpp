// Host task-graph builder, verifier and dry-run executor.
//
// The builder turns one decode step into output-tile tasks linked by
// event counters (MPK article, devpress.csdn.net, §2.1 TaskDesc / Event),
// classifies each operator as JIT or AOT (§2.2 classify_task: the
// attention, whose split count depends on the sequence lengths held on
// the device, is JIT; every GEMV consumes a full vector produced by all
// tiles of the previous operator, i.e. AOT_AFTER_BARRIER, expressed as an
// event whose required count is the producer count), and places AOT
// tasks in per-worker queues sorted by level (§5.1: workers = CUs - 4).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>

#include "mk_internal.h"

namespace mk {

static int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

static bool fail(std::string& err, const std::string& m) {
    err = m;
    return false;
}

static int64_t op_rows(const mk_model_desc& d, int op) {
    const int64_t QD = (int64_t)d.n_heads * d.head_dim, KD = (int64_t)d.n_kv_heads * d.head_dim;
    switch (op) {
        case OP_QKV: return QD + 2 * KD;
        case OP_O: return d.hidden;
        case OP_GATEUP: return d.ffn;
        case OP_DOWN: return d.hidden;
        case OP_LM: return d.vocab;
        case OP_EMBED: return d.hidden;
        case OP_APPEND: return (int64_t)d.batch * d.n_kv_heads;
        default: return 0;
    }
}

// ---------------------------------------------------------------------------
// Static schedule (opts.schedule = 1): an offline search fixes the tiling and
// the per-worker task order before any step runs (the Ada-MK articles,
// gist.science "Methodik" 1 and zingnex.cn 技术二: a DAG-level offline search
// with pruning, searched layer by layer under a cost model, whose result is
// frozen so that no runtime scheduling decision remains). Here the searched
// variables are the number of tasks of each GEMV operator (their rows are cut
// evenly, in 16-row tiles on the matrix-core path) and the attention split
// length, which must cover the plan's whole KV capacity because the split
// tasks are placed before any sequence length is known; tasks are placed on
// workers longest first onto the least-loaded worker (LPT). The task bodies
// are the event runtime's, so the two give the same bits at the same split
// length.
//
// Cost model (microseconds; calibrated on the per-operator trace of the 8B
// model on one MI355X): a GEMV task costs a fixed kLamGemv (event seen,
// operands issued, cross-wave reduction, stores, completion signal) plus its
// weight bytes at kRateW per worker plus the activation bytes it reads at
// kRateAct (once per pass of its matrix-core tiles); an attention split task
// costs kLamAttn plus its K/V bytes at kRateKV; every level adds one event
// hop kHop. A level lasts as long as its most loaded worker.
namespace {
constexpr double kLamGemv = 4.5, kRateW = 28000.0, kRateAct = 60000.0;  // us, bytes/us
constexpr double kLamAttn = 9.0, kRateKV = 20000.0, kHop = 2.0;

struct StaticChoice {
    int tasks[kNumOps] = {0};  // tasks per GEMV operator
    int chunk = 0;             // attention split length
    double predicted_us = 0;   // cost-model time of one layer
};

// cost of the most loaded worker when `costs` are placed longest first
double lpt_span(std::vector<double> costs, int W) {
    std::sort(costs.begin(), costs.end(), [](double a, double b) { return a > b; });
    std::vector<double> load(W, 0.0);
    double span = 0;
    for (double c : costs) {
        int best = 0;
        for (int w = 1; w < W; ++w)
            if (load[w] < load[best]) best = w;
        load[best] += c;
        span = std::max(span, load[best]);
    }
    return span;
}

// rows cut evenly into n tasks; on the matrix-core path (batch >= 3, bf16)
// the cuts fall on 16-row tile boundaries
std::vector<std::pair<int, int>> cut_rows(int64_t rows, int64_t n, bool tiles) {
    std::vector<std::pair<int, int>> r;
    const int64_t unit = tiles ? 16 : 1;
    const int64_t units = (rows + unit - 1) / unit;
    n = std::max<int64_t>(1, std::min(n, units));
    for (int64_t i = 0; i < n; ++i) {
        const int64_t a = std::min(rows, i * units / n * unit), b = std::min(rows, (i + 1) * units / n * unit);
        if (b > a) r.push_back({(int)a, (int)b});
    }
    return r;
}

// matrix-core tiles a task runs per pass (the task bodies' fixed counts)
int mfma_tiles_per_pass(int op) { return op == OP_QKV ? 2 : op == OP_GATEUP ? 3 : op == OP_LM ? 8 : 1; }

double gemv_level_cost(const mk_model_desc& d, int op, int n, int W) {
    const int64_t rows = op_rows(d, op);
    const int64_t K = op == OP_O ? (int64_t)d.n_heads * d.head_dim : op == OP_DOWN ? d.ffn : d.hidden;
    const int es = d.weight_dtype == MK_BF16 ? 2 : 4, nm = op == OP_GATEUP ? 2 : 1;
    const bool mf = d.weight_dtype == MK_BF16 && d.batch >= 3;
    std::vector<double> c;
    for (auto& r : cut_rows(rows, n, mf)) {
        const int64_t nr = r.second - r.first;
        const int passes = mf ? (int)(((nr + 15) / 16 + mfma_tiles_per_pass(op) - 1) / mfma_tiles_per_pass(op)) : 1;
        c.push_back(kLamGemv + (double)(nr * K * es * nm) / kRateW + (double)(passes * d.batch * K * 4) / kRateAct);
    }
    return lpt_span(c, W) + kHop;
}

double attn_level_cost(const mk_model_desc& d, int cap, int C, int W) {
    const int64_t splits = (cap + C - 1) / C;
    const int es = d.kv_dtype == MK_BF16 ? 2 : 4;
    std::vector<double> c((size_t)((int64_t)d.batch * d.n_kv_heads * splits),
                          kLamAttn + (double)C * 2 * d.head_dim * es / kRateKV);
    return lpt_span(c, W) + kHop;
}

// layered search: every layer has the same shape, so one layer's operators
// are searched (each independently, levels being separated by events) and
// the choice is used for all; a candidate whose lower bound (its bytes spread
// evenly over every worker) cannot beat the best so far is pruned
StaticChoice search_static(const mk_model_desc& d, int W, int cap, int chunk_min, int chunk_max) {
    StaticChoice ch;
    const int ops[] = {OP_QKV, OP_O, OP_GATEUP, OP_DOWN, OP_LM};
    const double frac[] = {0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 3.0};
    for (int op : ops) {
        if (op == OP_LM && d.hidden_io) continue;
        const int64_t rows = op_rows(d, op);
        double best = 1e300;
        int best_n = (int)std::min<int64_t>(W, rows);
        for (double f : frac) {
            const int n = (int)std::max<int64_t>(1, std::min<int64_t>(rows, (int64_t)(f * W)));
            const int64_t K = op == OP_O ? (int64_t)d.n_heads * d.head_dim : op == OP_DOWN ? d.ffn : d.hidden;
            const double lb = kLamGemv + (double)rows * K * (d.weight_dtype == MK_BF16 ? 2 : 4) *
                                             (op == OP_GATEUP ? 2 : 1) / W / kRateW + kHop;
            if (lb >= best) continue;  // pruned
            const double c = gemv_level_cost(d, op, n, W);
            if (c < best) {
                best = c;
                best_n = n;
            }
        }
        ch.tasks[op] = best_n;
        if (op != OP_LM) ch.predicted_us += best;
    }
    double best = 1e300;
    for (int C = chunk_min; C <= chunk_max; C *= 2) {
        const double c = attn_level_cost(d, cap, C, W);
        if (c < best) {
            best = c;
            ch.chunk = C;
        }
    }
    ch.predicted_us += best;
    return ch;
}
}  // namespace

bool build_host_plan(const mk_model_desc& d, int device_cus, HostPlan& p, std::string& err) {
    // ---- validation
    if (d.n_layers < 1 || d.n_layers > 1024) return fail(err, "n_layers must be in [1, 1024]");
    if (d.hidden < 8 || d.hidden % 8) return fail(err, "hidden must be a positive multiple of 8");
    if (d.head_dim != 64 && d.head_dim != 128) return fail(err, "head_dim must be 64 or 128");
    if (d.n_heads < 1 || d.n_kv_heads < 1 || d.n_heads % d.n_kv_heads)
        return fail(err, "n_heads must be a positive multiple of n_kv_heads");
    if (d.n_heads / d.n_kv_heads > 8) return fail(err, "at most 8 query heads per KV head");
    if (d.n_kv_heads > 64) return fail(err, "at most 64 KV heads");
    if (d.ffn < 8 || d.ffn % 8) return fail(err, "ffn must be a positive multiple of 8");
    if (!d.hidden_io && (d.vocab < 1)) return fail(err, "vocab must be positive");
    if (d.batch < 1 || d.batch > 16) return fail(err, "batch must be in [1, 16]");
    if (d.weight_dtype != MK_BF16 && d.weight_dtype != MK_F32 && d.weight_dtype != MK_W4)
        return fail(err, "weight_dtype must be MK_BF16, MK_F32 or MK_W4");
    if (d.weight_dtype == MK_W4) {
        if (d.kv_dtype != MK_BF16) return fail(err, "W4 weights need a bf16 KV cache");
        if (d.opts.lds_stream == 1) return fail(err, "W4 weights do not support lds_stream");
        const int64_t ks[3] = {d.hidden, d.ffn, (int64_t)d.n_heads * d.head_dim};
        for (int64_t k : ks)
            if (k % 1024 || k > 12288) return fail(err, "W4: hidden, ffn and n_heads*head_dim must be multiples of 1024, at most 12288");
    } else if (d.kv_dtype != d.weight_dtype) {
        return fail(err, "kv_dtype must equal weight_dtype (bf16/bf16 or f32/f32)");
    }
    if (d.weight_dtype == MK_F32 && d.batch > 4) return fail(err, "f32 weights support batch <= 4");
    if (d.weight_layout != MK_WEIGHTS_ROWS && d.weight_layout != MK_WEIGHTS_TILED)
        return fail(err, "weight_layout must be MK_WEIGHTS_ROWS or MK_WEIGHTS_TILED");
    const bool tiled = d.weight_layout == MK_WEIGHTS_TILED;
    if (tiled) {
        // the tiled layout is read by the matrix-core GEMV only
        if (d.weight_dtype != MK_BF16) return fail(err, "tiled weights must be bf16");
        if (d.batch < 3) return fail(err, "tiled weights need batch >= 3 (the matrix-core GEMV)");
        const int64_t QD = (int64_t)d.n_heads * d.head_dim, KD = (int64_t)d.n_kv_heads * d.head_dim;
        const int64_t rows[5] = {QD, KD, d.hidden, d.ffn, d.hidden_io ? 8 : d.vocab};
        for (int64_t r : rows)
            if (r % 8) return fail(err, "tiled weights: every matrix's row count must be a multiple of 8");
        const int64_t ks[3] = {d.hidden, d.ffn, QD};
        for (int64_t k : ks)
            if (k % 64) return fail(err, "tiled weights: hidden, ffn and n_heads*head_dim must be multiples of 64");
    }
    {
        const int64_t seg = d.weight_dtype == MK_F32 ? 256 : 512;
        const int64_t kmax = 4 * 8 * seg;  // four waves x eight 16-byte segments per lane
        if (d.hidden > kmax || d.ffn > kmax || (int64_t)d.n_heads * d.head_dim > kmax)
            return fail(err, "hidden, ffn and n_heads*head_dim must be <= " + std::to_string(kmax));
    }
    if (d.max_seq_len < 1 || d.max_seq_len > (1 << 22)) return fail(err, "max_seq_len must be in [1, 4M]");
    if (d.kv_layout == MK_KV_CONTIGUOUS &&
        (int64_t)d.max_seq_len * d.head_dim * (d.kv_dtype == MK_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
        return fail(err, "contiguous KV: one sequence's span (max_seq_len * head_dim * element size) must be "
                         "smaller than 2 GiB (32-bit buffer offsets)");
    if (!(d.rms_eps >= 0.f) || !(d.rope_base > 1.f)) return fail(err, "rms_eps must be >= 0 and rope_base > 1");
    if (d.kv_layout != MK_KV_CONTIGUOUS && d.kv_layout != MK_KV_PAGED) return fail(err, "bad kv_layout");
    if (d.kv_layout == MK_KV_PAGED) {
        if (d.kv_block < 1 || d.kv_block > 1024) return fail(err, "kv_block must be in [1, 1024]");
        // the matrix-core attention reads 16 consecutive positions of one block
        if (d.kv_dtype == MK_BF16 && d.kv_block % 16)
            return fail(err, "a paged bf16 cache needs kv_block a multiple of 16");
        if (d.max_blocks_per_seq < 1) return fail(err, "max_blocks_per_seq must be positive");
        if ((int64_t)d.max_blocks_per_seq * d.kv_block < d.max_seq_len)
            return fail(err, "max_blocks_per_seq * kv_block must cover max_seq_len");
    }
    const mk_exec_opts& o = d.opts;
    if (o.mode != MK_PERSISTENT && o.mode != MK_KERNEL_PER_OP) return fail(err, "opts.mode must be 0 or 1");
    if (device_cus < 2) return fail(err, "device has too few CUs");
    p = HostPlan();
    p.desc = d;
    if (o.jit < 0 || o.jit > 3) return fail(err, "opts.jit must be 0, 1, 2 or 3");
    const bool jit_opt = o.jit == 1 || o.jit == 3;
    if (o.schedule < 0 || o.schedule > 1) return fail(err, "opts.schedule must be 0 (event runtime) or 1 (static)");
    if (o.schedule == 1 && jit_opt) return fail(err, "the static schedule has no JIT attention (opts.jit 0 or 2)");
    p.jit = jit_opt ? 1 : 0;  // default: AOT attention slots
    p.jit_inline = o.jit == 3 ? 1 : 0;
    if (p.jit_inline && d.batch < 5)
        return fail(err, "opts.jit = 3 needs batch >= 5 (the batch >= 8 kernel instances)");
    p.schedule = o.schedule;
    if (o.prefill < 0 || o.prefill > 1) return fail(err, "opts.prefill must be 0 or 1");
    p.prefill = o.prefill;
    if (p.prefill && (jit_opt || d.hidden_io))
        return fail(err, "prefill plans need ahead-of-time attention and token input (no jit, no hidden_io)");
    // scheduler workgroups exist only to deal JIT attention; without them
    // every CU is a worker
    p.sched_wgs = (p.jit && !p.jit_inline) ? (o.sched_wgs > 0 ? o.sched_wgs : 4) : 0;
    p.workers = o.workers > 0 ? o.workers : device_cus - p.sched_wgs;
    if (p.workers < 1 || p.workers + p.sched_wgs > device_cus)
        return fail(err, "workers + sched_wgs must be in [1, CU count] (one workgroup per CU)");
    if (o.lds_stream < 0 || o.lds_stream > 1) return fail(err, "opts.lds_stream must be 0 or 1");
    if (o.lds_preload < 0 || o.lds_preload > 1) return fail(err, "opts.lds_preload must be 0 (off) or 1 (on)");
    p.kv_chunk = o.kv_chunk > 0 ? o.kv_chunk : 128;
    if (p.kv_chunk % 16 || p.kv_chunk > 4096) return fail(err, "kv_chunk must be a multiple of 16, at most 4096");
    p.cap = d.max_seq_len;
    p.max_splits = n_splits_for(p.cap, p.kv_chunk);
    {
        // the per-step chunk may grow to cmax (a paged split stages its
        // block-table entries, cmax / kv_block + 2 ints, in LDS)
        if (o.kv_chunk_max > 0 && (o.kv_chunk_max < p.kv_chunk || o.kv_chunk_max % 16 || o.kv_chunk_max > 16384))
            return fail(err, "opts.kv_chunk_max must be a multiple of 16 in [kv_chunk, 16384]");
        p.kv_chunk_max = o.kv_chunk_max > 0 ? o.kv_chunk_max : std::max(p.kv_chunk, 4096);
        p.attn_target = kAttnSplitTarget;
    }
    if (p.max_splits > 65535) return fail(err, "too many splits per sequence");
    {
        // K split of the O and down projections on the matrix-core path
        const bool mf_path = d.weight_dtype == MK_BF16 && d.batch >= 3;
        // default: 4 parts for down, none for O (measured no faster split)
        auto pick = [&](int ks, int64_t K, const char* name, int auto_parts, int& outk) {
            const std::string n(name);
            if (ks != 0 && ks != 1 && ks != 2 && ks != 4) return fail(err, "opts." + n + " must be 0, 1, 2 or 4");
            if (ks == 0) {
                ks = (mf_path && o.schedule == 0 && K % (64 * auto_parts) == 0) ? auto_parts : 1;
            } else if (ks > 1) {
                if (!mf_path) return fail(err, "opts." + n + " > 1 needs the matrix-core path (bf16 weights, batch >= 3)");
                if (o.schedule == 1) return fail(err, "opts." + n + " > 1 is not available with the static schedule");
                if (K % (64 * ks)) return fail(err, "opts." + n + ": K must be a multiple of 64 * parts");
            }
            outk = ks;
            return true;
        };
        if (!pick(o.down_ksplit, d.ffn, "down_ksplit", 4, p.down_ks)) return false;
        if (!pick(o.o_ksplit, (int64_t)d.n_heads * d.head_dim, "o_ksplit", 1, p.o_ks)) return false;
    }
    StaticChoice sc;
    if (p.schedule == 1) {
        // the split length is fixed for every step: chunk = chunk_max = the searched C
        const int cmin = std::max(64, p.kv_chunk);
        sc = search_static(d, p.workers, p.cap, cmin, std::max(cmin, std::min(p.kv_chunk_max, 4096)));
        p.kv_chunk = p.kv_chunk_max = sc.chunk;
        p.max_splits = n_splits_for(p.cap, p.kv_chunk);
        p.predicted_layer_us = sc.predicted_us;
    }

    const int L = d.n_layers, W = p.workers, B = d.batch, Hkv = d.n_kv_heads;
    p.events.assign(5 * L + 1 + (p.prefill ? L : 0), EventRec{0, -1});
    int rot = 0;
    std::vector<std::vector<int32_t>> q(W);
    int level = 0;

    auto add_level = [&](int op, int layer) {
        p.level_op.push_back((uint8_t)op);
        p.level_layer.push_back((uint16_t)layer);
        p.level_off.push_back((int32_t)p.level_tasks.size());
    };
    // static schedule: tasks placed longest first onto the least-loaded worker
    // of the level (ties to the lowest index after the rotation)
    auto lpt_place = [&](const std::vector<int>& ids, const std::vector<double>& cost) {
        std::vector<int> order(ids.size());
        for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cost[a] > cost[b]; });
        std::vector<double> load(W, 0.0);
        std::vector<std::vector<int>> per(W);
        for (int i : order) {
            int best = rot;
            for (int k = 1; k < W; ++k) {
                const int w = (rot + k) % W;
                if (load[w] < load[best]) best = w;
            }
            load[best] += cost[i];
            per[best].push_back(ids[i]);
        }
        for (int w = 0; w < W; ++w) {
            std::sort(per[w].begin(), per[w].end());
            for (int id : per[w]) q[w].push_back(id);
        }
        rot = (rot + (int)ids.size()) % W;
    };
    auto add_gemv = [&](int op, int layer, int wait, int sig, int min_rows) {
        const int64_t rows = op_rows(d, op);
        if (p.schedule == 1 && op != OP_EMBED && op != OP_APPEND) {
            const bool mf = d.weight_dtype == MK_BF16 && d.batch >= 3;
            add_level(op, layer);
            std::vector<int> ids;
            std::vector<double> cost;
            for (auto& r : cut_rows(rows, sc.tasks[op], mf)) {
                TaskRec t{};
                t.op = (uint8_t)op;
                t.layer = (uint16_t)layer;
                t.a0 = r.first;
                t.a1 = r.second;
                t.wait_ev = wait;
                t.sig_ev = sig;
                t.level = level;
                const int id = (int)p.tasks.size();
                p.tasks.push_back(t);
                p.level_tasks.push_back(id);
                ids.push_back(id);
                cost.push_back((double)(r.second - r.first));
                if (sig >= 0) p.events[sig].required++;
                p.tasks_per_op[op]++;
            }
            lpt_place(ids, cost);
            level++;
            return;
        }
        // tiled weights: tasks own whole 8-row units of the tiled layout
        const int64_t unit = (tiled && op != OP_EMBED && op != OP_APPEND) ? 8 : 1;
        const int64_t units = rows / unit;
        if ((op == OP_DOWN && p.down_ks > 1) || (op == OP_O && p.o_ks > 1)) {
            // K split: row groups of about ks 16-row tiles, each group's K
            // cut into ks parts, one task per part on consecutive workers;
            // the last part to arrive merges and signals, so the event counts
            // groups
            const int ks = op == OP_DOWN ? p.down_ks : p.o_ks;
            const int64_t groups = std::min<int64_t>(std::max(1, W / ks), units);
            add_level(op, layer);
            for (int64_t g = 0; g < groups; ++g) {
                const int32_t a0 = (int32_t)(g * units / groups * unit), a1 = (int32_t)((g + 1) * units / groups * unit);
                for (int kp = 0; kp < ks; ++kp) {
                    TaskRec t{};
                    t.op = (uint8_t)op;
                    t.layer = (uint16_t)layer;
                    t.a0 = a0;
                    t.a1 = a1;
                    t.kpart = kp | (ks << 8);
                    t.kgroup = (int32_t)g;
                    t.wait_ev = wait;
                    t.sig_ev = sig;
                    t.level = level;
                    const int id = (int)p.tasks.size();
                    p.tasks.push_back(t);
                    p.level_tasks.push_back(id);
                    q[(g * ks + kp + rot) % W].push_back(id);
                    p.tasks_per_op[op]++;
                }
                if (sig >= 0) p.events[sig].required++;
            }
            p.ksplit_groups = std::max(p.ksplit_groups, (int)groups);
            rot = (int)((rot + groups * ks) % W);
            level++;
            return;
        }
        int64_t nt = std::min<int64_t>(W, (units + min_rows - 1) / min_rows);
        add_level(op, layer);
        for (int64_t i = 0; i < nt; ++i) {
            TaskRec t{};
            t.op = (uint8_t)op;
            t.layer = (uint16_t)layer;
            t.a0 = (int32_t)(i * units / nt * unit);
            t.a1 = (int32_t)((i + 1) * units / nt * unit);
            if (t.a1 <= t.a0) continue;
            t.wait_ev = wait;
            t.sig_ev = sig;
            t.level = level;
            int id = (int)p.tasks.size();
            p.tasks.push_back(t);
            p.level_tasks.push_back(id);
            q[(i + rot) % W].push_back(id);
            if (sig >= 0) p.events[sig].required++;
            p.tasks_per_op[op]++;
        }
        rot = (int)((rot + nt) % W);
        level++;
    };

    int prev = -1;
    if (!d.hidden_io) {
        add_gemv(OP_EMBED, 0, -1, ev_embed(L), 256);
        prev = ev_embed(L);
    }
    for (int l = 0; l < L; ++l) {
        add_gemv(OP_QKV, l, prev, ev_qkv(l), 1);
        // prefill: the rows' keys and values are stored in a level of their
        // own, so that every row's attention finds the rows before it
        if (p.prefill) add_gemv(OP_APPEND, l, ev_qkv(l), ev_append(l, L), 1);
        const int attn_wait = p.prefill ? ev_append(l, L) : ev_qkv(l);
        // attention: one level; tasks exist in AOT mode only (JIT tasks are
        // created on the device by the scheduler waves)
        add_level(OP_ATTN, l);
        if (p.jit) {
            p.events[ev_qkv(l)].jit_layer = l;
        } else if (p.schedule == 1) {
            // static: one task per (sequence, KV head, split) of the capacity,
            // its identity fixed in the record; splits past a sequence's
            // length end at once
            std::vector<int> ids;
            std::vector<double> cost;
            for (int bg = 0; bg < B * Hkv; ++bg)
                for (int sp = 0; sp < p.max_splits; ++sp) {
                    TaskRec t{};
                    t.op = OP_ATTN;
                    t.flags = kTaskStaticAttn;
                    t.layer = (uint16_t)l;
                    t.a0 = bg;
                    t.a1 = sp;
                    t.wait_ev = attn_wait;
                    t.sig_ev = ev_attn(l);
                    t.level = level;
                    const int id = (int)p.tasks.size();
                    p.tasks.push_back(t);
                    p.level_tasks.push_back(id);
                    ids.push_back(id);
                    cost.push_back(1.0);
                    p.tasks_per_op[OP_ATTN]++;
                }
            lpt_place(ids, cost);
        } else {
            // AOT: slot i runs split task i of the step in (b, g, split)
            // order, found from seq_lens when it runs
            const int S = aot_attn_slots(p);
            for (int i = 0; i < S; ++i) {
                TaskRec t{};
                t.op = OP_ATTN;
                t.layer = (uint16_t)l;
                t.a0 = i;
                t.a1 = S;
                t.wait_ev = attn_wait;
                t.sig_ev = ev_attn(l);
                t.level = level;
                int id = (int)p.tasks.size();
                p.tasks.push_back(t);
                p.level_tasks.push_back(id);
                q[rot].push_back(id);
                rot = (rot + 1) % W;
                p.tasks_per_op[OP_ATTN]++;
            }
        }
        p.events[ev_attn(l)].required = (uint32_t)(B * Hkv);
        level++;
        add_gemv(OP_O, l, ev_attn(l), ev_o(l), 1);
        add_gemv(OP_GATEUP, l, ev_o(l), ev_gateup(l), 1);
        add_gemv(OP_DOWN, l, ev_gateup(l), ev_down(l), 1);
        prev = ev_down(l);
    }
    if (!d.hidden_io) add_gemv(OP_LM, 0, prev, -1, 1);
    p.n_levels = level;
    p.level_off.push_back((int32_t)p.level_tasks.size());

    p.queue_off.assign(W + 1, 0);
    for (int w = 0; w < W; ++w) p.queue_off[w + 1] = p.queue_off[w] + (int32_t)q[w].size();
    p.queue.reserve(p.queue_off[W]);
    for (int w = 0; w < W; ++w) p.queue.insert(p.queue.end(), q[w].begin(), q[w].end());

    if (o.debug_extra_required > 0) {
        if (o.debug_event < 0 || o.debug_event >= (int)p.events.size()) return fail(err, "debug_event out of range");
        p.events[o.debug_event].required += (uint32_t)o.debug_extra_required;
    }

    const int64_t per_layer_jit = (int64_t)B * Hkv * p.max_splits;
    if (per_layer_jit > (1 << 26)) return fail(err, "too many attention tasks per layer");
    p.max_jit_tasks = (int)per_layer_jit;
    // JIT tasks are dealt round-robin to workers that still have an AOT task
    // after the last attention level: such a worker is bound to wait on an
    // event that depends on the attention, and drains its inbox meanwhile
    int last_attn = -1;
    for (int lv = 0; lv < p.n_levels; ++lv)
        if (p.level_op[lv] == OP_ATTN) last_attn = lv;
    for (int w = 0; w < W; ++w) {
        bool ok = false;
        for (int i = p.queue_off[w]; i < p.queue_off[w + 1] && !ok; ++i) ok = p.tasks[p.queue[i]].level > last_attn;
        if (ok) p.jit_elig.push_back(w);
    }
    if (p.jit && p.jit_elig.empty()) return fail(err, "no worker can receive JIT tasks");
    p.inbox_cap = next_pow2((int)std::max<int64_t>(16, per_layer_jit / std::max<size_t>(1, p.jit_elig.size()) + 2));
    p.mb_cap = next_pow2(std::max(16, L));

    const int64_t es = d.weight_dtype == MK_F32 ? 4 : 2;
    const int64_t H = d.hidden, F = d.ffn, QD = (int64_t)d.n_heads * d.head_dim, KD = (int64_t)Hkv * d.head_dim;
    int64_t layer = ((QD + 2 * KD) * H + H * QD + 3 * F * H + 2 * H + (d.qk_norm ? 2 * d.head_dim : 0)) * es;
    if (d.weight_dtype == MK_W4) {
        // codes (K / 2 bytes per row) and scales (2 bytes per 128 inputs); gains bf16
        const int64_t dims[7][2] = {{QD, H}, {KD, H}, {KD, H}, {H, QD}, {F, H}, {F, H}, {H, F}};
        layer = (2 * H + (d.qk_norm ? 2 * d.head_dim : 0)) * 2;
        for (auto& rc : dims) layer += rc[0] * rc[1] / 2 + rc[0] * (rc[1] / 128) * 2;
    }
    p.weight_bytes = L * layer + (d.hidden_io ? 0 : ((int64_t)d.vocab * H + H) * es);
    p.kv_bytes_per_token = (int64_t)L * 2 * KD * (d.kv_dtype == MK_BF16 ? 2 : 4);
    return true;
}

bool verify_plan(const HostPlan& p, std::string& err) {
    const mk_model_desc& d = p.desc;
    const int nt = (int)p.tasks.size();
    // queues: every task exactly once, levels non-decreasing
    std::vector<int> seen(nt, 0);
    if ((int)p.queue_off.size() != p.workers + 1) return fail(err, "queue_off size");
    for (int w = 0; w < p.workers; ++w) {
        int last = -1;
        for (int i = p.queue_off[w]; i < p.queue_off[w + 1]; ++i) {
            int t = p.queue[i];
            if (t < 0 || t >= nt) return fail(err, "queue holds a bad task id");
            seen[t]++;
            if (p.tasks[t].level < last) return fail(err, "queue of worker " + std::to_string(w) + " not level-sorted");
            last = p.tasks[t].level;
        }
    }
    for (int t = 0; t < nt; ++t)
        if (seen[t] != 1) return fail(err, "task " + std::to_string(t) + " queued " + std::to_string(seen[t]) + " times");
    // producers per event; waits only on strictly lower levels
    std::vector<uint32_t> prod(p.events.size(), 0);
    std::vector<int> prod_level(p.events.size(), -1);
    for (const TaskRec& t : p.tasks) {
        if (t.sig_ev >= (int)p.events.size() || t.wait_ev >= (int)p.events.size()) return fail(err, "event id range");
        // a K-split task group signals once (its merging part)
        if (t.sig_ev >= 0 && t.op != OP_ATTN && (t.kpart & 0xFF) == 0) {
            prod[t.sig_ev]++;
            prod_level[t.sig_ev] = std::max(prod_level[t.sig_ev], t.level);
        }
    }
    for (int l = 0; l < d.n_layers; ++l) {
        prod[ev_attn(l)] += (uint32_t)(d.batch * d.n_kv_heads);  // combines
        prod_level[ev_attn(l)] = -2;                              // checked through levels below
    }
    for (size_t e = 0; e < p.events.size(); ++e) {
        uint32_t req = p.events[e].required;
        if ((int)e == d.opts.debug_event && d.opts.debug_extra_required > 0) req -= (uint32_t)d.opts.debug_extra_required;
        if (req != prod[e]) return fail(err, "event " + std::to_string(e) + " required " + std::to_string(req) +
                                                 " != producers " + std::to_string(prod[e]));
    }
    for (const TaskRec& t : p.tasks) {
        if (t.wait_ev < 0) continue;
        if (prod_level[t.wait_ev] >= t.level)
            return fail(err, "task waits on an event produced at its own or a later level");
    }
    // row coverage per GEMV level
    for (int lv = 0; lv < p.n_levels; ++lv) {
        int op = p.level_op[lv];
        if (op == OP_ATTN) continue;
        // every K part (0 .. ks - 1) covers the rows exactly once, in the
        // same row groups
        int ks = 1;
        for (int i = p.level_off[lv]; i < p.level_off[lv + 1]; ++i) ks = std::max(ks, p.tasks[p.level_tasks[i]].kpart >> 8);
        std::vector<std::vector<std::pair<int, int>>> parts(ks);
        std::vector<std::pair<int, int>> r;
        for (int i = p.level_off[lv]; i < p.level_off[lv + 1]; ++i) {
            const TaskRec& t = p.tasks[p.level_tasks[i]];
            if (t.op != op || t.level != lv) return fail(err, "level list mixes operators");
            const int kp = t.kpart & 0xFF, tks = t.kpart >> 8;
            if (ks > 1 && (tks != ks || kp >= ks || t.kgroup < 0)) return fail(err, "K-split task with a bad part");
            parts[kp].push_back({t.a0, t.a1});
            if (kp == 0) r.push_back({t.a0, t.a1});
        }
        for (auto& v : parts) {
            std::sort(v.begin(), v.end());
            if (v != parts[0]) return fail(err, "K parts of a level cover different rows");
        }
        std::sort(r.begin(), r.end());
        int64_t at = 0;
        // tiled weights: every matrix task starts and ends on an 8-row unit
        const bool unit8 = d.weight_layout == MK_WEIGHTS_TILED && op != OP_EMBED && op != OP_APPEND;
        for (auto& x : r) {
            if (unit8 && (x.first % 8 || x.second % 8)) return fail(err, "tiled weights: task rows not on 8-row units");
            if (x.first != at || x.second <= x.first) return fail(err, "rows not covered exactly once at level " + std::to_string(lv));
            at = x.second;
        }
        if (at != op_rows(d, op)) return fail(err, "rows not fully covered at level " + std::to_string(lv));
    }
    if (!p.jit) {
        const int want = p.schedule == 1 ? d.batch * d.n_kv_heads * p.max_splits : aot_attn_slots(p);
        for (int lv = 0; lv < p.n_levels; ++lv) {
            if (p.level_op[lv] != OP_ATTN) continue;
            int n = p.level_off[lv + 1] - p.level_off[lv];
            if (n != want) return fail(err, "AOT attention level incomplete");
        }
    }
    return true;
}

// ---------------------------------------------------------------------------
// Dry run: host threads replay the persistent protocol on integer data.

namespace {

inline uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

struct DryState {
    const HostPlan& p;
    std::vector<int> seq;
    // per level: output array
    std::vector<std::vector<std::atomic<uint64_t>>> out;
    std::vector<std::atomic<uint32_t>> ev;
    std::vector<std::atomic<uint32_t>> arrive;
    std::vector<std::atomic<uint64_t>> partial;  // [B*Hkv][max_splits]
    // K-split levels: part values [rows][ks] and row-group arrivals, per level
    std::vector<std::vector<std::atomic<uint64_t>>> kval;
    std::vector<std::vector<std::atomic<uint32_t>>> karr;
    std::vector<RingSlot> jit;                     // [workers][inbox_cap]
    std::vector<std::atomic<int64_t>> jit_tag;     // [workers][inbox_cap]
    std::vector<std::atomic<int64_t>> jit_tail;    // per worker
    std::vector<int64_t> jit_head;                 // per worker (single consumer)
    std::atomic<int64_t> rr{0};
    std::vector<std::atomic<int64_t>> mb_tag;
    std::vector<int32_t> mb_payload;
    std::atomic<int64_t> mb_tail{0}, mb_head{0};
    std::atomic<int> abort{0};
    int drop;
    std::chrono::steady_clock::time_point deadline;
    std::vector<int> level_of_event;  // producing level
    explicit DryState(const HostPlan& pl) : p(pl) {}
};

int step_chunk(const DryState& s) {
    const HostPlan& p = s.p;
    const int B = p.desc.batch, Hkv = p.desc.n_kv_heads;
    auto total = [&](int c) {
        long long t = 0;
        for (int b = 0; b < B; ++b) t += (long long)Hkv * n_splits_for(attn_keys(s.seq[b]), c);
        return t;
    };
    return attn_chunk_search(total, p.kv_chunk, p.kv_chunk_max, p.attn_target);
}

uint64_t level_input_sum(DryState& s, int lv) {
    uint64_t h = 0;
    for (auto& v : s.out[lv]) h += v.load(std::memory_order_acquire);
    return h;
}

// level whose outputs a task at `lv` consumes: the previous level (or none)
int input_level(const HostPlan& p, int lv) { return lv - 1; }

int64_t level_rows(const HostPlan& p, int lv) {
    const mk_model_desc& d = p.desc;
    if (p.level_op[lv] == OP_ATTN) return (int64_t)d.batch * d.n_kv_heads;
    return op_rows(d, p.level_op[lv]);
}

// value of K part kp of row r at level lv (a K-split row is the XOR of its parts)
uint64_t kpart_value(uint64_t sum, int lv, int64_t r, int kp) {
    return mix64(sum ^ ((uint64_t)lv << 40) ^ (uint64_t)r ^ ((uint64_t)(kp + 1) << 52));
}

// Returns whether the task signals its event: always, except the parts of a
// K-split group other than the last to arrive, which merges the group.
bool run_gemv(DryState& s, const TaskRec& t) {
    int in = input_level(s.p, t.level);
    uint64_t sum = in >= 0 ? level_input_sum(s, in) : 0x1234;
    const int ks = t.kpart >> 8;
    if (ks <= 1) {
        for (int r = t.a0; r < t.a1; ++r)
            s.out[t.level][r].store(mix64(sum ^ ((uint64_t)t.level << 40) ^ (uint64_t)r), std::memory_order_release);
        return true;
    }
    const int kp = t.kpart & 0xFF;
    auto& kv = s.kval[t.level];
    for (int r = t.a0; r < t.a1; ++r) kv[(size_t)r * ks + kp].store(kpart_value(sum, t.level, r, kp), std::memory_order_release);
    const uint32_t old = s.karr[t.level][t.kgroup].fetch_add(1, std::memory_order_acq_rel);
    if ((int)old + 1 != ks) return false;
    for (int r = t.a0; r < t.a1; ++r) {
        uint64_t v = 0;
        for (int q = 0; q < ks; ++q) v ^= kv[(size_t)r * ks + q].load(std::memory_order_acquire);
        s.out[t.level][r].store(v, std::memory_order_release);
    }
    s.karr[t.level][t.kgroup].store(0, std::memory_order_relaxed);
    return true;
}

// K parts of a level's tasks (1: whole K)
int level_ks(const HostPlan& p, int lv) {
    int ks = 1;
    for (int i = p.level_off[lv]; i < p.level_off[lv + 1]; ++i) ks = std::max(ks, p.tasks[p.level_tasks[i]].kpart >> 8);
    return ks;
}

// split task k of the step in (b, g, split) order, if the step has one
bool locate_split(const DryState& s, int C, int k, int& bg, int& split) {
    const HostPlan& p = s.p;
    for (int b = 0; b < p.desc.batch; ++b) {
        const int ns = n_splits_for(s.seq[b] + 1, C), cnt = ns * p.desc.n_kv_heads;
        if (k < cnt) {
            bg = b * p.desc.n_kv_heads + k / ns;
            split = k % ns;
            return true;
        }
        k -= cnt;
    }
    return false;
}

bool run_attn(DryState& s, int layer, int bg, int split, int lv) {
    const HostPlan& p = s.p;
    int b = bg / p.desc.n_kv_heads;
    int keys = s.seq[b] + 1;
    int ns = n_splits_for(keys, step_chunk(s));
    if (split >= ns) return false;  // reserved but unused (AOT mode)
    uint64_t sum = level_input_sum(s, lv - 1);
    s.partial[(size_t)bg * p.max_splits + split].store(mix64(sum ^ ((uint64_t)bg << 20) ^ (uint64_t)split),
                                                       std::memory_order_release);
    uint32_t old = s.arrive[bg].fetch_add(1, std::memory_order_acq_rel);
    if ((int)old + 1 == ns) {
        uint64_t c = 0;
        for (int i = 0; i < ns; ++i) c = mix64(c ^ s.partial[(size_t)bg * p.max_splits + i].load(std::memory_order_acquire));
        s.out[lv][bg].store(c, std::memory_order_release);
        s.arrive[bg].store(0, std::memory_order_relaxed);
        return true;  // completing split signals the attention event
    }
    return false;
}

}  // namespace

bool dry_run(const HostPlan& p, int n_threads, uint64_t seed, int drop_task, int timeout_ms, const int32_t* seq_lens,
             std::string& err) {
    const mk_model_desc& d = p.desc;
    DryState s(p);
    s.seq.resize(d.batch);
    for (int b = 0; b < d.batch; ++b) {
        int v = seq_lens ? seq_lens[b] : 0;
        if (v < 0 || v + 1 > p.cap) return fail(err, "seq_lens out of range for the plan");
        s.seq[b] = v;
    }
    s.drop = drop_task;
    s.out = std::vector<std::vector<std::atomic<uint64_t>>>(p.n_levels);
    for (int lv = 0; lv < p.n_levels; ++lv) {
        s.out[lv] = std::vector<std::atomic<uint64_t>>(level_rows(p, lv));
        for (auto& v : s.out[lv]) v.store(0);
    }
    s.ev = std::vector<std::atomic<uint32_t>>(p.events.size());
    for (auto& e : s.ev) e.store(0);
    s.arrive = std::vector<std::atomic<uint32_t>>(d.batch * d.n_kv_heads);
    for (auto& a : s.arrive) a.store(0);
    s.partial = std::vector<std::atomic<uint64_t>>((size_t)d.batch * d.n_kv_heads * p.max_splits);
    s.kval = std::vector<std::vector<std::atomic<uint64_t>>>(p.n_levels);
    s.karr = std::vector<std::vector<std::atomic<uint32_t>>>(p.n_levels);
    for (int lv = 0; lv < p.n_levels; ++lv) {
        const int ks = p.level_op[lv] == OP_ATTN ? 1 : level_ks(p, lv);
        if (ks <= 1) continue;
        s.kval[lv] = std::vector<std::atomic<uint64_t>>((size_t)level_rows(p, lv) * ks);
        for (auto& v : s.kval[lv]) v.store(0);
        s.karr[lv] = std::vector<std::atomic<uint32_t>>((size_t)p.workers);
        for (auto& v : s.karr[lv]) v.store(0);
    }
    s.jit.resize((size_t)p.workers * p.inbox_cap);
    s.jit_tag = std::vector<std::atomic<int64_t>>((size_t)p.workers * p.inbox_cap);
    for (auto& t : s.jit_tag) t.store(0);
    s.jit_tail = std::vector<std::atomic<int64_t>>(p.workers);
    for (auto& t : s.jit_tail) t.store(0);
    s.jit_head.assign(p.workers, 0);
    s.mb_tag = std::vector<std::atomic<int64_t>>(p.mb_cap);
    for (auto& t : s.mb_tag) t.store(0);
    s.mb_payload.assign(p.mb_cap, 0);
    s.deadline = std::chrono::steady_clock::now() + std::chrono::milliseconds(timeout_ms > 0 ? timeout_ms : 5000);

    const int W = p.workers;
    const int nthr = std::max(1, std::min(n_threads, W));

    auto timed_out = [&]() {
        if (s.abort.load()) return true;
        if (std::chrono::steady_clock::now() > s.deadline) {
            s.abort.store(1);
            return true;
        }
        return false;
    };
    // deal layer `layer`'s split tasks round-robin into the workers'
    // inboxes (the scheduler's work, or the completing producer's with
    // jit_inline)
    auto expand = [&](int layer) {
        int64_t total = 0;
        for (int b = 0; b < d.batch; ++b) total += (int64_t)d.n_kv_heads * n_splits_for(s.seq[b] + 1, step_chunk(s));
        const int64_t start = s.rr.fetch_add(total);
        int64_t i = 0;
        const int64_t ne = (int64_t)p.jit_elig.size();
        for (int b = 0; b < d.batch; ++b) {
            int ns = n_splits_for(s.seq[b] + 1, step_chunk(s));
            for (int g = 0; g < d.n_kv_heads; ++g)
                for (int sp = 0; sp < ns; ++sp, ++i) {
                    const int w = p.jit_elig[(size_t)((start + i) % ne)];
                    int64_t pos = s.jit_tail[w].fetch_add(1);
                    const size_t slot = (size_t)w * p.inbox_cap + (size_t)(pos % p.inbox_cap);
                    s.jit[slot].p0 = (layer << 16) | (b * d.n_kv_heads + g);
                    s.jit[slot].p1 = sp;
                    s.jit_tag[slot].store(pos + 1, std::memory_order_release);
                }
        }
    };
    auto signal = [&](int e) {
        if (e < 0) return;
        uint32_t old = s.ev[e].fetch_add(1, std::memory_order_acq_rel);
        if (old + 1 == p.events[e].required && p.events[e].jit_layer >= 0) {
            if (p.jit_inline) {
                expand(p.events[e].jit_layer);
                return;
            }
            int64_t pos = s.mb_tail.fetch_add(1);
            s.mb_payload[pos % p.mb_cap] = p.events[e].jit_layer;
            s.mb_tag[pos % p.mb_cap].store(pos + 1, std::memory_order_release);
        }
    };
    auto attn_level = [&](int layer) {
        for (int lv = 0; lv < p.n_levels; ++lv)
            if (p.level_op[lv] == OP_ATTN && p.level_layer[lv] == layer) return lv;
        return -1;
    };
    auto try_pop_jit = [&](int w, int& layer, int& bg, int& split) {
        const int64_t h = s.jit_head[w];
        const size_t slot = (size_t)w * p.inbox_cap + (size_t)(h % p.inbox_cap);
        if (s.jit_tag[slot].load(std::memory_order_acquire) != h + 1) return false;
        layer = s.jit[slot].p0 >> 16;
        bg = s.jit[slot].p0 & 0xFFFF;
        split = s.jit[slot].p1;
        s.jit_head[w] = h + 1;
        return true;
    };
    auto run_jit = [&](int layer, int bg, int split, std::mt19937_64& rng) {
        std::this_thread::sleep_for(std::chrono::microseconds(rng() % 40));
        int lv = attn_level(layer);
        if (run_attn(s, layer, bg, split, lv)) signal(ev_attn(layer));
    };

    // scheduler thread: pops the mailbox and expands attention tasks
    std::thread sched;
    if (p.jit && !p.jit_inline) {
        sched = std::thread([&]() {
            std::mt19937_64 rng(seed ^ 0xABCDEF);
            int64_t want = d.n_layers;
            while (s.mb_head.load() < want) {
                if (timed_out()) return;
                int64_t h = s.mb_head.load();
                if (s.mb_tag[h % p.mb_cap].load(std::memory_order_acquire) != h + 1) {
                    std::this_thread::yield();
                    continue;
                }
                int layer = s.mb_payload[h % p.mb_cap];
                if (!s.mb_head.compare_exchange_strong(h, h + 1)) continue;
                std::this_thread::sleep_for(std::chrono::microseconds(rng() % 30));
                expand(layer);
            }
        });
    }

    // worker threads: each host thread plays workers ti, ti + nthr, ...
    // round-robin, advancing one whose next task is ready, and running JIT
    // tasks while none is (as the device workers drain the JIT ring while
    // they wait)
    std::vector<std::thread> th;
    for (int ti = 0; ti < nthr; ++ti) {
        th.emplace_back([&, ti]() {
            std::mt19937_64 rng(seed * 1000003ull + ti);
            std::vector<int> mine, cur;
            for (int w = ti; w < W; w += nthr) {
                mine.push_back(w);
                cur.push_back(p.queue_off[w]);
            }
            size_t left = mine.size();
            while (left) {
                if (timed_out()) return;
                bool progressed = false;
                for (size_t k = 0; k < mine.size(); ++k) {
                    int w = mine[k];
                    if (cur[k] >= p.queue_off[w + 1]) continue;
                    const TaskRec& t = p.tasks[p.queue[cur[k]]];
                    if (t.wait_ev >= 0) {
                        uint32_t tgt = p.events[t.wait_ev].required;
                        if ((int32_t)(s.ev[t.wait_ev].load(std::memory_order_acquire) - tgt) < 0) continue;
                    }
                    if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
                    cur[k]++;
                    if (cur[k] >= p.queue_off[w + 1]) left--;
                    progressed = true;
                    if (t.op == OP_ATTN) {
                        int bg = t.a0, sp = t.a1;
                        const bool located = (t.flags & kTaskStaticAttn) || locate_split(s, step_chunk(s), t.a0, bg, sp);
                        if (located && run_attn(s, t.layer, bg, sp, t.level)) signal(t.sig_ev);
                        continue;
                    }
                    const bool sg = run_gemv(s, t);
                    if ((int)(&t - p.tasks.data()) == s.drop) continue;  // injected fault: never signals
                    if (sg) signal(t.sig_ev);
                }
                if (!progressed) {
                    bool ran = false;
                    for (size_t k = 0; k < mine.size() && p.jit; ++k) {
                        int layer, bg, sp;
                        if (try_pop_jit(mine[k], layer, bg, sp)) {
                            run_jit(layer, bg, sp, rng);
                            ran = true;
                        }
                    }
                    if (!ran) std::this_thread::yield();
                }
            }
        });
    }
    for (auto& t : th) t.join();
    if (sched.joinable()) sched.join();  // the scheduler exits once every message is popped (or on abort)
    if (!s.abort.load())
        for (int l = 0; l < d.n_layers; ++l)
            if (s.ev[ev_attn(l)].load() != p.events[ev_attn(l)].required)
                return fail(err, "attention tasks left undone when every worker finished its queue");
    if (s.abort.load()) return fail(err, "timeout: dry run did not complete (a wait never became ready)");

    // sequential reference: evaluate levels in order
    std::vector<std::vector<uint64_t>> ref(p.n_levels);
    for (int lv = 0; lv < p.n_levels; ++lv) {
        ref[lv].assign(level_rows(p, lv), 0);
        uint64_t sum = 0x1234;
        if (lv > 0) {
            sum = 0;
            for (uint64_t v : ref[lv - 1]) sum += v;
        }
        if (p.level_op[lv] == OP_ATTN) {
            for (int bg = 0; bg < d.batch * d.n_kv_heads; ++bg) {
                int ns = n_splits_for(s.seq[bg / d.n_kv_heads] + 1, step_chunk(s));
                uint64_t c = 0;
                for (int i = 0; i < ns; ++i) c = mix64(c ^ mix64(sum ^ ((uint64_t)bg << 20) ^ (uint64_t)i));
                ref[lv][bg] = c;
            }
        } else if (level_ks(p, lv) > 1) {
            const int ks = level_ks(p, lv);
            for (int64_t r = 0; r < (int64_t)ref[lv].size(); ++r) {
                uint64_t v = 0;
                for (int q = 0; q < ks; ++q) v ^= kpart_value(sum, lv, r, q);
                ref[lv][r] = v;
            }
        } else {
            for (int64_t r = 0; r < (int64_t)ref[lv].size(); ++r) ref[lv][r] = mix64(sum ^ ((uint64_t)lv << 40) ^ (uint64_t)r);
        }
    }
    for (int lv = 0; lv < p.n_levels; ++lv)
        for (size_t r = 0; r < ref[lv].size(); ++r)
            if (s.out[lv][r].load() != ref[lv][r])
                return fail(err, "checksum mismatch at level " + std::to_string(lv) + " row " + std::to_string(r));
    return true;
}

}  // namespace mk
