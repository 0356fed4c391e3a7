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

enum mk_dtype { MK_F32 = 0, MK_BF16 = 1, MK_W4 = 2 };
enum mk_kv_layout { MK_KV_CONTIGUOUS = 0, MK_KV_PAGED = 1 };
enum mk_exec_mode { MK_PERSISTENT = 0, MK_KERNEL_PER_OP = 1 };

enum mk_status {
    MK_OK = 0,
    MK_ERR_ARG = -1,         /* invalid argument (null pointer, bad shape, mismatch with the plan) */
    MK_ERR_HIP = -2,         /* a HIP runtime call failed (message says which) */
    MK_ERR_UNSUPPORTED = -3, /* valid request this library does not support */
    MK_ERR_STATE = -4        /* plan in a state that forbids the call (e.g. host-only plan) */
};

/* Bits of the sticky device error word (mk_get_device_error). */
enum mk_device_error {
    MK_ERR_TOKEN = 1,       /* a token id outside [0, vocab): that row used token 0 */
    MK_ERR_KV_OVERFLOW = 2, /* seq_lens[b] + 1 exceeds the KV capacity: that row's attention output is zero */
    MK_ERR_TIMEOUT = 4,     /* a bounded wait in the persistent kernel expired; all workgroups exited */
    MK_ERR_BLOCK_TABLE = 8  /* a paged block-table entry outside the pool (see mk_kv_cache): those
                               positions read as zeros and the new row is not stored */
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
 *                slot per split task a step can have (min(256, batch *
 *                n_kv_heads * max splits), or batch * n_kv_heads *
 *                ceil(max_seq_len / kv_chunk_max) if larger) on the
 *                workers; once the layer's QKV event fires, slot i runs
 *                split task i of the step in (b, g, split) order, if any,
 *                3 = JIT without scheduler waves: the QKV task whose arrival
 *                completes the layer's QKV event expands the split tasks
 *                (one wave) and deals them into the workers' inboxes; every
 *                CU is a worker (the mixed launch of the MPK article, §2.2,
 *                with the expansion moved from dedicated scheduler warps
 *                into the completing producer). Batch >= 5 only.
 *  kv_chunk      KV positions per attention split task (default 128; a
 *                multiple of 16). Each step uses the smallest multiple of 16
 *                from kv_chunk up to kv_chunk_max for which the step has at
 *                most 256 split tasks (kv_chunk_max if none does); the rule
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
 *                (0: the default, 256 at batch <= 2 and off at batch >= 3,
 *                where the matrix-core GEMV's streams measured faster
 *                without it; -1 = off).
 *  lds_stream    1: at batch 1 with bf16 weights, the persistent kernel streams
 *                weight pages through a per-wave LDS ring filled by
 *                direct-to-LDS buffer loads (experimental; same results).
 *  trace         records per worker kept by the in-kernel task trace (0 =
 *                off). Each record holds the task, the worker, and the
 *                real-time-clock ticks (100 MHz) at wait start, ready and
 *                done; read them with mk_plan_trace.
 *  lds_preload   1: in persistent mode with ahead-of-time attention and
 *                batch <= 2, a worker waiting for a GEMV task's event copies
 *                the task's first rows (up to 30 KB per wave) into LDS pages
 *                with direct-to-LDS loads and the task reads them from there
 *                (the MPK article's paged shared memory, §3.1, and preload
 *                during the wait, §3.2; same results). 0 (default): off; the
 *                L2 prefetch of prefetch_kb measured faster.
 *  schedule      0 (default): the event runtime above. 1: static schedule
 *                (the Ada-MK articles, gist.science "Methodik" 1, zingnex.cn
 *                技术二: offline search, fixed execution path): the planner
 *                searches the task count of every GEMV operator and the
 *                attention split length under a cost model, layer by layer
 *                with pruning, places tasks longest first on the least-loaded
 *                worker and fixes every attention split task to its
 *                (sequence, KV head, split) of the whole capacity; kv_chunk
 *                and kv_chunk_max are replaced by the searched length. Same
 *                task bodies: the bits of the event runtime at that length.
 *                Not with jit = 1.
 *  prefill       1: a prompt-chunk plan for mk_prefill: the `batch` rows of a
 *                step are consecutive positions of one sequence, all reading
 *                and writing sequence 0's K/V; an append level (QK-norm,
 *                RoPE, K/V store) runs between QKV and attention, so each
 *                row's attention sees the rows before it. Ahead-of-time
 *                attention only (not jit = 1); token input only.
 *  down_ksplit   parts the down projection's K (the SwiGLU width) is cut
 *                into on the matrix-core path (bf16, batch >= 3, event
 *                runtime): each part is its own task over 16 * ksplit rows,
 *                writing a partial tile, and the last part of a row group
 *                to arrive adds the partials in part order (the attention
 *                combine's last-arrival rule, the MPK article §2.1) and
 *                signals; every worker then reads 1 / ksplit of the input
 *                vector instead of all of it. 0 (default): 4 where the
 *                matrix-core path runs and ffn is a multiple of 256, else
 *                1; 1: off; 2 or 4: that many parts (ffn a multiple of
 *                64 * parts). Not with schedule = 1 (its search cuts whole
 *                rows). Results differ from the unsplit sum only by
 *                rounding order; every execution mode of one plan gives the
 *                same bits.
 *  o_ksplit      the same for the O projection (K = n_heads * head_dim).
 *                0 (default) and 1: off (at batch 16 on the 8B shape, 4
 *                parts measured 4.58 ms/step against 4.57 without: the O
 *                task's activations are only twice its weight bytes); 2 or
 *                4: that many parts.
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
    int32_t lds_preload;
    int32_t schedule;
    int32_t prefill;
    int32_t down_ksplit;
    int32_t o_ksplit;
} mk_exec_opts;

/*
 * Model and batch description (one plan per batch size, as in the MPK
 * article §4.2 "预编译多batch-size子图").
 *  hidden % 8 == 0; head_dim in {64, 128}; n_heads % n_kv_heads == 0;
 *  n_heads / n_kv_heads <= 8; 1 <= batch <= 16.
 *  weight_dtype, kv_dtype: MK_BF16 or MK_F32 (bf16 weights need a bf16 cache
 *  and f32 weights an f32 cache), or weight_dtype MK_W4 with a bf16 cache:
 *  4-bit layer matrices (the Ada-MK summary's W4A16, gist.science
 *  "Hauptbeiträge" 4), any batch (VALU GEMV at batch <= 2, matrix cores
 *  with the codes dequantized in registers above), hidden, ffn and n_heads * head_dim
 *  multiples of 1024 and at most 12288. Each W4 matrix [rows, K] is one
 *  buffer: 4-bit codes in row order, two per byte (low nibble first),
 *  rows * K / 2 bytes; then, from that size rounded up to 256 bytes, one
 *  bf16 scale per 128 inputs of a row, [rows][K / 128]; the weight is
 *  (code - 8) * scale. Norm gains, embedding and LM head stay bf16.
 *  max_seq_len: KV capacity per sequence in positions. Contiguous layout:
 *  the cache holds [layer][batch][kv_head][max_seq_len][head_dim], and one
 *  sequence's span max_seq_len * head_dim * element size must be below
 *  2 GiB (attention addresses it with 32-bit byte offsets). Paged layout:
 *  positions are reached through a block table (see mk_kv_cache) and
 *  max_seq_len bounds seq_lens[b] + 1.
 *  hidden_io: 1 = no embedding and no LM head; steps read and write hidden
 *  states (mk_decode_step_hidden).
 *  weight_layout: MK_WEIGHTS_ROWS (0): every matrix [rows, K] row-major.
 *  MK_WEIGHTS_TILED (1): the seven layer matrices and the LM head are in
 *  the tiled layout that mk_pack_tiled writes (the embedding and the norm
 *  gains stay as they are); the matrix-core GEMV then reads each 16-byte
 *  lane load from 512-byte runs of consecutive bytes instead of 16 rows x
 *  64 bytes (the MPK article's GEMV tasks stream weight tiles, §2.1; the
 *  layout is this library's, chosen for the CDNA4 matrix-core operand).
 *  Needs bf16 weights, batch >= 3 (the matrix-core instances), every row
 *  count (n_heads*head_dim, n_kv_heads*head_dim, hidden, ffn, vocab) a
 *  multiple of 8 and every K (hidden, ffn, n_heads*head_dim) a multiple of
 *  64; other plans reject it (MK_ERR_ARG at mk_build_graph). Results are
 *  bit-identical to the row-major layout.
 */
enum mk_weight_layout { MK_WEIGHTS_ROWS = 0, MK_WEIGHTS_TILED = 1 };

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
    int32_t kv_block;           /* paged: positions per block (16; a multiple of 16 for a bf16 cache) */
    int32_t max_blocks_per_seq; /* paged: row length of the block table */
    int32_t hidden_io;
    mk_exec_opts opts;
    int32_t weight_layout;      /* MK_WEIGHTS_ROWS (default) or MK_WEIGHTS_TILED, below */
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
 *    l*layer_stride + ((b*n_kv_heads + h)*max_seq_len + p)*head_dim + d;
 *    layer_stride >= batch*n_kv_heads*max_seq_len*head_dim.
 *  Paged (the MPK article's paged memory, §3.1, applied to the cache):
 *    block_table is device int32 [batch, max_blocks_per_seq]; position p of
 *    sequence b lives in physical block blk = block_table[b][p / kv_block]
 *    at l*layer_stride + ((blk*n_kv_heads + h)*kv_block + p % kv_block)*head_dim + d.
 *    layer_stride is a multiple of n_kv_heads*kv_block*head_dim, so a layer
 *    holds layer_stride / (n_kv_heads*kv_block*head_dim) blocks (the pool),
 *    and layer_stride * element size must be below 2 GiB (32-bit offsets);
 *    the steps reject other strides with MK_ERR_ARG. Entries outside
 *    [0, pool) are caught on the device: MK_ERR_BLOCK_TABLE, nothing is
 *    read from or written to such a block.
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
    int32_t tasks_per_op[12]; /* indexed by op: 1 QKV, 2 O, 3 gate/up, 4 down, 5 LM head, 6 attention (AOT),
                                 7 embedding, 8 append (prefill plans) */
    int64_t weight_bytes_per_step; /* weight bytes one step streams (matrices, gains, LM head) */
    int64_t kv_bytes_per_token;    /* K + V bytes per cached position over all layers */
    int64_t device_bytes;          /* device memory the plan owns */
    int32_t jit, mode, host_only, schedule;
    double predicted_layer_us;     /* static schedule: the cost model's time of one layer (0 otherwise) */
} mk_plan_info;

/*
 * Build the task graph for `desc` and upload its tables. Defining passages:
 * the MPK article (devpress.csdn.net) §2.1 "Mega-Kernel执行模型" (each
 * operator becomes tile tasks linked by events, and the whole graph one
 * kernel), §2.2 "混合任务启动机制" (classify_task: JIT for data-dependent
 * operators, AOT otherwise), §4.2 (one pre-built graph per batch size) and
 * §5.1 "参数配置建议" (workers = CUs - 4, 16 scheduler warps).
 * Returns NULL on error (see mk_last_error). The plan owns its tables,
 * activations, partials, rings and error word (device memory allocated
 * here, once).
 */
mk_plan* mk_build_graph(const mk_model_desc* desc);

/*
 * Free a plan and its device memory. Waits for the device first. NULL is a
 * no-op. The pages define no teardown; the plan's memory is released here
 * because mk_build_graph allocated it.
 */
void mk_destroy_plan(mk_plan* plan);

/*
 * Message for the last error on the calling thread ("" if none). The pages
 * define no error reporting; errors stay inside the C ABI as status codes
 * and this thread-local text.
 */
const char* mk_last_error(void);

/*
 * Fill `info` (host memory) with the plan's task counts per operator, its
 * event and level counts and its bytes per step: the quantities of the MPK
 * article's task graph (§2.1 TaskDesc / Event) and of the decode step's
 * memory-bound cost (Ada-MK summary, gist.science, "Methodik" 2: decode is
 * IO-bound). Returns MK_OK or MK_ERR_ARG.
 */
int mk_plan_query(const mk_plan* plan, mk_plan_info* info);

/*
 * Enqueue one decode step on `stream`: embedding, every decoder layer
 * (RMSNorm, QKV, QK-norm, RoPE, KV append, attention, O, SwiGLU MLP) and
 * the final norm and LM head, as one persistent launch (the MPK article,
 * §2.1 "Mega-Kernel执行模型"; the layer as Attention then MLP, §1), or, with
 * opts.mode = MK_KERNEL_PER_OP, as one launch per task-graph level (§1, the
 * execution model the article replaces, kept as the one-switch fallback of
 * the pgsm.cn essay, §5.3 "回滚预案").
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
 * into the LM-head tasks; tokens and seq_lens are written once every reader
 * of the step's lengths has finished (persistent mode: the last worker to
 * leave its queue; kernel-per-op: the last LM-head task). Not for hidden_io
 * plans. Defining passage: the MPK article §2.1 (the next token is produced
 * inside the single launch, so the host only re-launches), §1 (per-launch
 * cost of 5-20 us).
 */
int mk_decode_step_greedy(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, int32_t* tokens,
                          int32_t* seq_lens, float* logits, void* stream);

/*
 * n_steps greedy decode steps in one persistent launch: the same as calling
 * mk_decode_step_greedy n_steps times (same tokens, lengths and, for the
 * last step, logits, bit for bit), with the next token fed to the next step
 * on the device and the events' epochs advanced there (the MPK article,
 * §2.1: the whole computation in one kernel, no per-step launch, §1).
 *  tokens, seq_lens  as mk_decode_step_greedy; on return they hold the last
 *                    step's tokens and seq_lens[b] + n_steps.
 *  logits            device float [batch, vocab]: the last step's logits.
 *  n_steps           1 .. 4096 (MK_ERR_ARG outside). Every step must fit the
 *                    KV capacity (seq_lens[b] + n_steps <= max_seq_len), else
 *                    the device reports MK_ERR_KV_OVERFLOW for those steps.
 *  out_tokens        device int32 [n_steps, batch] or NULL: step s's tokens
 *                    at out_tokens[s * batch + b].
 * Persistent mode needs ahead-of-time attention (opts.jit 0 or 2) and no
 * lds_stream for n_steps > 1 (MK_ERR_UNSUPPORTED otherwise); kernel-per-op
 * mode runs the steps as consecutive level launches. Between two steps every
 * worker waits at a device-wide step barrier released by the last worker to
 * finish the step, which writes that step's tokens and lengths.
 */
int mk_decode_steps_greedy(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, int32_t* tokens,
                           int32_t* seq_lens, float* logits, int32_t n_steps, int32_t* out_tokens, void* stream);

/*
 * Prefill of T prompt tokens of one sequence through the decode runtime, a
 * chunk of `batch` positions per persistent launch (the other half of the
 * Ada-MK hybrid engine, zingnex.cn 技术三 and gist.science "Methodik" 2,
 * here inside the same task-graph runtime): ceil(T / batch) launches of a
 * plan built with opts.prefill = 1, instead of T decode steps.
 *  tokens  device int32 [T]: the prompt, positions pos0 .. pos0 + T - 1.
 *  pos0    positions already cached for the sequence (host int, >= 0);
 *          pos0 + T <= max_seq_len.
 *  kv      the sequence's cache: contiguous (sequence 0 of the layout) or
 *          paged (row 0 of the block table).
 *  logits  device float [vocab]: the logits after the last prompt token.
 * The last chunk, if shorter, repeats its last position in the remaining
 * rows; their appends store the same bits at the same place. The plan's own
 * device memory holds the chunk's tokens, lengths and logits. Returns as
 * mk_decode_step; MK_ERR_STATE for a plan without opts.prefill.
 */
int mk_prefill(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, const int32_t* tokens, int32_t pos0,
               int32_t T, float* logits, void* stream);

/*
 * Hidden-state variant for hidden_io plans: x_in, x_out are device float
 * [batch, hidden] (they may not alias); otherwise as mk_decode_step. It runs
 * the decoder layers only (the Ada-MK summary, gist.science, "Methodik" 1:
 * the Transformer decoder, with the LM head as a separate part).
 */
int mk_decode_step_hidden(mk_plan* plan, const mk_weights* weights, const mk_kv_cache* kv, const float* x_in,
                          const int32_t* seq_lens, float* x_out, void* stream);

/*
 * Synchronise `stream`, return the sticky device error bits (0 if none) and
 * clear them. After MK_ERR_TIMEOUT the plan's event counters are reset so
 * the next step starts clean. Negative on a HIP failure. The pages define no
 * device error path; a single persistent launch cannot return one, so the
 * kernel sets bits in a word the plan owns and this call reads them (the
 * checks behind them are the caller-data checks of the pgsm.cn essay's
 * production list, §5.3, done on the device).
 */
int mk_get_device_error(mk_plan* plan, void* stream);

/*
 * Writes the tiled copy (MK_WEIGHTS_TILED) of one row-major bf16 matrix.
 * Defining passage: the MPK article's GEMV tasks, each streaming the weight
 * tile of its output rows (devpress.csdn.net, §2.1); the tile order is this
 * library's own, fitted to the operand of the CDNA4 16x16x32 matrix cores.
 *  src   device bf16 [rows, cols], row-major.
 *  dst   device bf16, rows * cols elements, caller-owned, not overlapping src.
 *        Rows are grouped in units of 8 (unit u: rows 8u .. 8u + 7), each
 *        unit is 8 * cols consecutive elements, and inside a unit the
 *        element of row 8u + i, column 32 s + 8 j + e (i, e < 8, j < 4) sits
 *        at s * 256 + (8 j + i) * 8 + e: for each 32-column step, the 16
 *        bytes of row i and column group j in the order the matrix cores'
 *        lanes load them.
 *  rows  a positive multiple of 8; cols a positive multiple of 64.
 *  Runs on the current device, stream-ordered on `stream`.
 * Returns MK_OK, MK_ERR_ARG (bad sizes or a null pointer; nothing launched)
 * or MK_ERR_HIP.
 */
int mk_pack_tiled(const void* src, void* dst, int64_t rows, int64_t cols, void* stream);

/*
 * Greedy next token: out_tokens[b] = argmax_v logits[b, v] (lowest index on
 * ties, NaN never chosen). logits device float [batch, vocab]; out_tokens
 * device int32 [batch]. Its own launch, using the plan's scratch. Defining
 * passage: greedy decoding of the next token after the LM head (the Ada-MK
 * summary, gist.science, "Methodik" 1 and "Experimentelle Ergebnisse": the
 * decode phase generates one token per step).
 */
int mk_argmax(const mk_plan* plan, const float* logits, int32_t* out_tokens, void* stream);

/*
 * mk_argmax without a plan and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same result as mk_argmax:
 * out_tokens[b] = argmax_v logits[b, v], lowest index on ties, NaN never
 * chosen (0 for a row with no number).
 *  logits     device float [batch, vocab]; out_tokens device int32 [batch].
 *  batch      1 .. 256 (larger: MK_ERR_ARG, nothing launched); vocab >= 1.
 *  Runs on the current device; `stream` must belong to it.
 * Its scratch (the 64 slice winners of each row, 128 KB at most) is a fixed
 * array in the library's device memory, one per GPU, held until the process
 * ends; its address is looked up with hipGetSymbolAddress on the first call
 * on each device. Two launches, stream-ordered; the scratch needs no
 * clearing. Calls that overlap on one GPU (different streams, or several
 * host threads) share that array and race: serialise them.
 */
int mk_argmax_noalloc(const float* logits, int32_t batch, int32_t vocab, int32_t* out_tokens, void* stream);

/*
 * Host-side checks of a plan's task graph (the MPK article §2.1: tasks,
 * events with required counts): every output row covered
 * exactly once per op, events' required counts equal their producer
 * counts, every queue sorted by level, no task waits on an event of its
 * own or a later level. Returns MK_OK or MK_ERR_STATE with a message.
 */
int mk_plan_verify(const mk_plan* plan);

/*
 * Host dry run of the persistent schedule (the MPK article §2.1-2.2: AOT
 * queues, event waits, JIT dispatch): `n_threads` host threads play
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
 * for `max_records`; the pages' timing breakdown of task phases, MPK §3.2,
 * measured per task here). Synchronises `stream`. Returns the number of records
 * written (records of workers that overflowed their share are dropped), or
 * a negative mk_status (MK_ERR_STATE if the plan was built without trace).
 */
int mk_plan_trace(const mk_plan* plan, mk_trace_rec* out, int64_t max_records, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
