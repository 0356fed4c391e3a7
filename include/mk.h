/*
 * mk: one transformer-decoder decode step run as a single persistent
 * megakernel that executes a tile-level task graph on an AMD MI355X
 * (gfx950).
 *
 * The method follows the MPK article (devpress.csdn.net): the whole
 * computation graph runs in one kernel launch (§2.1 "Mega-Kernel执行模型");
 * tasks are triggered by atomic event counters (§2.1, the TaskDesc/Event
 * records); data-dependent attention tasks are launched just in time by
 * scheduler wavefronts while static GEMV tasks are queued ahead of time
 * (§2.2 "混合任务启动机制"); workers are CUs minus four scheduler CUs running
 * sixteen scheduler waves (§5.1 "参数配置建议"). The kernel-per-operator
 * mode, which the article replaces (§1), is kept as a bit-identical
 * fallback, in line with the self-scheduling essay (pgsm.cn, §5.3,
 * "rollback to eager" and "bitwise graph-vs-eager outputs").
 *
 * Conventions for every entry point:
 *  - Pointers documented "device" are HIP device pointers owned by the
 *    caller; "host" pointers are read during the call only.
 *  - Streams are passed as `void*` holding a hipStream_t (NULL = the null
 *    stream). Work is enqueued on that stream; calls return immediately.
 *  - Functions returning int return MK_OK (0) or a negative mk_status.
 *    Errors never cross the ABI as exceptions. mk_last_error() returns a
 *    thread-local message for the last failure on the calling thread.
 *  - A plan is not thread-safe; at most one step per plan may be in flight,
 *    always on the same stream.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_plan mk_plan;

enum mk_dtype { MK_F32 = 0, MK_BF16 = 1 };
enum mk_kv_layout { MK_KV_CONTIGUOUS = 0, MK_KV_PAGED = 1 };
enum mk_exec_mode { MK_PERSISTENT = 0, MK_KERNEL_PER_OP = 1 };

enum mk_status {
    MK_OK = 0,
    MK_ERR_ARG = -1,         /* invalid argument (null pointer, bad shape, mismatch with the plan) */
    MK_ERR_HIP = -2,         /* a HIP runtime call failed (message says which) */
    MK_ERR_UNSUPPORTED = -3, /* valid request this build does not support */
    MK_ERR_STATE = -4        /* plan in a state that forbids the call (e.g. host-only plan) */
};

/* Bits of the sticky device error word (mk_get_device_error). */
enum mk_device_error {
    MK_ERR_TOKEN = 1,       /* a token id outside [0, vocab): that row used token 0 */
    MK_ERR_KV_OVERFLOW = 2, /* seq_lens[b] + 1 exceeds the KV capacity: that row's attention output is zero */
    MK_ERR_TIMEOUT = 4      /* a bounded wait in the persistent kernel expired; all workgroups exited */
};

/*
 * Execution options. Zero means "default" for every field.
 *  mode          MK_PERSISTENT (default) or MK_KERNEL_PER_OP (one launch per
 *                task-graph level, same task bodies, bit-identical results).
 *  workers       worker workgroups, one per CU (default: CU count - sched_wgs).
 *  sched_wgs     scheduler workgroups of 4 waves each, JIT mode only (default
 *                4 -> 16 waves; 0 in AOT mode).
 *  jit           attention launch: 0 = default (AOT), 1 = JIT: the last QKV
 *                task of a layer posts it to a mailbox, the scheduler waves
 *                expand its split tasks from seq_lens and deal them into the
 *                workers' inboxes, 2 = AOT: each layer queues one attention
 *                slot per split task a step can have (min(240, batch *
 *                n_kv_heads * max splits), or batch * n_kv_heads *
 *                ceil(max_seq_len / kv_chunk_max) if larger) on the
 *                workers; once the layer's QKV event fires, slot i runs
 *                split task i of the step in (b, g, split) order, if any.
 *  kv_chunk      KV positions per attention split task (default 128; a
 *                multiple of 16). Each step uses the smallest multiple of 16
 *                from kv_chunk up to kv_chunk_max for which the step has at
 *                most 240 split tasks (kv_chunk_max if none does); the rule
 *                depends only on seq_lens, so every mode computes the same
 *                splits.
 *  kv_chunk_max  upper bound of that chunk (default 4096, at most 16384, a
 *                multiple of 16; set it equal to kv_chunk to keep the chunk
 *                fixed).
 *  watchdog_ms   bound on every spin wait of the persistent kernel
 *                (default 2000).
 *  host_only     1: build the task graph on the host only (no HIP calls);
 *                such a plan can be queried, verified and dry-run but not
 *                stepped. Used for CPU tests.
 *  device_cus    CU count to plan for when host_only (default 256).
 *  debug_extra_required  for fault tests: adds this many to the required
 *                count of event `debug_event` so its waiters time out.
 *  prefetch_kb   KB of the next GEMV task's weights each worker pulls toward
 *                the chip (L2 / memory-side cache) while it waits for that
 *                task's event, issued in small slices between polls
 *                (default 256; -1 = off).
 *  lds_stream    1: at batch 1 with bf16 weights, the persistent kernel streams
 *                weight pages through a per-wave LDS ring filled by
 *                direct-to-LDS buffer loads (experimental; same results).
 *  trace         records per worker kept by the in-kernel task trace (0 =
 *                off). Each record holds the task, the worker, and the
 *                real-time-clock ticks (100 MHz) at wait start, ready and
 *                done; read them with mk_plan_trace.
 */
typedef struct mk_exec_opts {
    int32_t mode;
    int32_t workers;
    int32_t sched_wgs;
    int32_t jit;
    int32_t kv_chunk;
    int32_t watchdog_ms;
    int32_t host_only;
    int32_t device_cus;
    int32_t debug_event;
    int32_t debug_extra_required;
    int32_t trace;
    int32_t prefetch_kb;
    int32_t lds_stream;
    int32_t kv_chunk_max;
    int32_t reserved[2];
} mk_exec_opts;

/*
 * Model and batch description (one plan per batch size, as in the MPK
 * article §4.2 "预编译多batch-size子图").
 *  hidden % 8 == 0; head_dim in {64, 128}; n_heads % n_kv_heads == 0;
 *  n_heads / n_kv_heads <= 8; 1 <= batch <= 16.
 *  weight_dtype, kv_dtype: MK_BF16 or MK_F32 (bf16 weights need a bf16 cache
 *  and f32 weights an f32 cache).
 *  max_seq_len: KV capacity per sequence in positions. Contiguous layout:
 *  the cache holds [layer][batch][kv_head][max_seq_len][head_dim]. Paged
 *  layout: positions are reached through a block table (see mk_kv_cache)
 *  and max_seq_len bounds seq_lens[b] + 1.
 *  hidden_io: 1 = no embedding and no LM head; steps read and write hidden
 *  states (mk_decode_step_hidden).
 */
typedef struct mk_model_desc {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
    float rms_eps;
    float rope_base;
    int32_t qk_norm;
    int32_t weight_dtype;
    int32_t kv_dtype;
    int32_t batch;
    int32_t max_seq_len;
    int32_t kv_layout;
    int32_t kv_block;           /* paged: positions per block (16) */
    int32_t max_blocks_per_seq; /* paged: row length of the block table */
    int32_t hidden_io;
    mk_exec_opts opts;
} mk_model_desc;

/* Device pointers to one layer's weights, PyTorch [out, in] row-major. */
typedef struct mk_layer_weights {
    const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} mk_layer_weights;

/*
 * Weights (device pointers; the struct itself and `layers` are host
 * memory). embed [vocab, hidden], lm_head [vocab, hidden] (may alias embed),
 * final_norm [hidden]; unused (NULL) when hidden_io.
 */
typedef struct mk_weights {
    const void* embed;
    const void* final_norm;
    const void* lm_head;
    const mk_layer_weights* layers;
    int32_t n_layers;
} mk_weights;

/*
 * KV cache (device memory, caller-owned, elements of kv_dtype).
 *  layer_stride: elements from one layer's cache to the next.
 *  Contiguous: element (l, b, h, p, d) at
 *    l*layer_stride + ((b*n_kv_heads + h)*max_seq_len + p)*head_dim + d.
 *  Paged: block_table is device int32 [batch, max_blocks_per_seq]; position
 *  p of sequence b lives in physical block blk = block_table[b][p / kv_block]
 *  at l*layer_stride + ((blk*n_kv_heads + h)*kv_block + p % kv_block)*head_dim + d.
 */
typedef struct mk_kv_cache {
    void* k;
    void* v;
    int64_t layer_stride;
    const int32_t* block_table;
} mk_kv_cache;

/* Plan summary (mk_plan_query). */
typedef struct mk_plan_info {
    int32_t workers, sched_waves, n_aot_tasks, n_events, n_levels, max_jit_tasks, kv_chunk, max_splits;
    int32_t tasks_per_op[8]; /* indexed by op: 1 QKV, 2 O, 3 gate/up, 4 down, 5 LM head, 6 attention (AOT) */
    int64_t weight_bytes_per_step; /* weight bytes one step streams (matrices, gains, LM head) */
    int64_t kv_bytes_per_token;    /* K + V bytes per cached position over all layers */
    int64_t device_bytes;          /* device memory the plan owns */
    int32_t jit, mode, host_only, reserved;
} mk_plan_info;

/*
 * Build the task graph for `desc` (MPK article §2.1: the graph becomes one
 * kernel; §2.2: classify_task; §5.1: workers = CUs - 4, 16 scheduler
 * waves) and upload its tables. Returns NULL on error (see mk_last_error).
 * The plan owns its tables, activations, partials, rings and error word.
 */
mk_plan* mk_build_graph(const mk_model_desc* desc);

/* Free a plan and its device memory (waits for the device). NULL is a no-op. */
void mk_destroy_plan(mk_plan* plan);

/* Message for the last error on the calling thread ("" if none). */
const char* mk_last_error(void);

/* Fill `info` (host). */
int mk_plan_query(const mk_plan* plan, mk_plan_info* info);

/*
 * Enqueue one decode step on `stream`.
 *  tokens   device int32 [batch]: the new token of each sequence.
 *  seq_lens device int32 [batch]: positions already cached. The step writes
 *           K/V at index seq_lens[b] and attends over seq_lens[b] + 1 keys.
 *           The library never changes seq_lens; the caller advances it.
 *  logits   device float [batch, vocab], fully overwritten.
 * Returns MK_OK or a host-detected error (MK_ERR_ARG for null pointers or
 * a weights/plan mismatch, MK_ERR_STATE for a host-only or hidden-I/O plan).
 * Device-detected errors set the sticky error word (mk_get_device_error).
 */
int mk_decode_step(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, const int32_t* tokens,
                   const int32_t* seq_lens, float* logits, void* stream);

/*
 * One decode step with the greedy choice fused into it: as mk_decode_step,
 * and then, in the same launch, tokens[b] is overwritten with the argmax of
 * logits[b] (lowest index on ties, NaN never chosen, as mk_argmax) and
 * seq_lens[b] is incremented, ready for the next step. The argmax is folded
 * into the LM-head tasks; the last of them writes tokens and seq_lens after
 * every reader of the step's lengths has finished. Not for hidden_io plans.
 */
int mk_decode_step_greedy(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, int32_t* tokens,
                          int32_t* seq_lens, float* logits, void* stream);

/*
 * Hidden-state variant for hidden_io plans: x_in, x_out are device float
 * [batch, hidden] (they may not alias); otherwise as mk_decode_step.
 */
int mk_decode_step_hidden(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, const float* x_in,
                          const int32_t* seq_lens, float* x_out, void* stream);

/*
 * Synchronise `stream`, return the sticky device error bits (0 if none) and
 * clear them. After MK_ERR_TIMEOUT the plan's event counters are reset so
 * the next step starts clean. Negative on a HIP failure.
 */
int mk_get_device_error(mk_plan* plan, void* stream);

/*
 * Greedy next token: out_tokens[b] = argmax_v logits[b, v] (lowest index on
 * ties). logits device float [batch, vocab]; out_tokens device int32 [batch].
 */
int mk_argmax(const mk_plan* plan, const float* logits, int32_t* out_tokens, void* stream);

/*
 * Host-side checks of a plan's task graph: every output row covered
 * exactly once per op, events' required counts equal their producer
 * counts, every queue sorted by level, no task waits on an event of its
 * own or a later level. Returns MK_OK or MK_ERR_STATE with a message.
 */
int mk_plan_verify(const mk_plan* plan);

/*
 * Host dry run of the persistent schedule: `n_threads` host threads play
 * the workers (AOT queues, event waits, JIT ring drained while waiting)
 * with random delays from `seed`, each task computing an integer checksum
 * of its inputs. Compares against a sequential topological evaluation.
 * drop_task >= 0 makes that task never signal (fault injection).
 * Returns MK_OK, MK_ERR_STATE on a checksum mismatch, or MK_ERR_TIMEOUT-like
 * failure as MK_ERR_STATE with "timeout" in the message.
 */
int mk_plan_dry_run(const mk_plan* plan, int n_threads, uint64_t seed, int drop_task, int timeout_ms,
                    const int32_t* seq_lens_host);

/*
 * One task-trace record (opts.trace > 0). kind: 0 AOT task (id = task
 * index in the plan), 1 JIT attention task (id = layer << 24 | (b*Hkv+g) << 12
 * | split, fields truncated). t_wait: the worker started waiting for the
 * task's event; t_ready: the event was satisfied (JIT: task popped);
 * t_done: outputs written and the completion signalled; t_a .. t_d: phase
 * marks inside the task body. Ticks of the 100 MHz device real-time clock.
 */
typedef struct mk_trace_rec {
    int32_t kind;
    int32_t id;
    int32_t worker;
    int32_t op;
    uint64_t t_wait, t_ready, t_done;
    uint64_t t_a, t_b, t_c, t_d; /* task-defined phase marks, 0 if unset. GEMV: operands
                                    ready, rows done, outputs stored, stores complete;
                                    attention: prologue done, K/V pass done, waves
                                    merged into LDS, partial stored */
} mk_trace_rec;

/*
 * Copy the trace of the last persistent step to host memory `out` (room
 * for `max_records`). Synchronises `stream`. Returns the number of records
 * written (records of workers that overflowed their share are dropped), or
 * a negative mk_status (MK_ERR_STATE if the plan was built without trace).
 */
int mk_plan_trace(const mk_plan* plan, mk_trace_rec* out, int64_t max_records, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
