/*
 * amk.h: C ABI of the MI355X batch-1 decode megakernel library (libamk.so).
 *
 * One call of amk_decode_step runs one batch-1 greedy decode step of a Llama-family
 * transformer as a single persistent launch: one workgroup per compute unit walks a static
 * task-DAG schedule, synchronised only by monotone counters, and the whole forward pass of one
 * token happens inside that one launch (AutoMegaKernel pages: page 1, author's note, "one
 * launch = one forward = one token", and "How it works"; page 3, "How it works", layer 0).
 * A schedule is validated on the CPU before anything launches; an unsafe one is refused, never
 * run (page 1, "Deadlock-free by construction"; page 2, "Statically verified schedule IR" and
 * Table 1; page 4, "De Safety Gate").
 *
 * Conventions
 *  - Every call returns an amk_status; nothing aborts, throws or exits across this ABI.
 *    Out-parameters are written only on AMK_OK (verdicts are also written on AMK_E_REJECTED).
 *  - "device" pointers are HIP device memory of the current device; "host" pointers are
 *    ordinary CPU memory. All matrices are row-major [out, in].
 *  - A context is not thread-safe; use it from one host thread and one stream at a time.
 *  - The library is silent unless the environment variable AMK_LOG=1 is set.
 */
#ifndef AMK_H
#define AMK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AMK_OK = 0,
    AMK_E_INVALID_ARG = 1,     /* null pointer, bad size, position out of range, bad struct_size */
    AMK_E_UNSUPPORTED = 2,     /* model variant the kernel does not implement (see amk_create) */
    AMK_E_REJECTED = 3,        /* the schedule failed validation; nothing was launched */
    AMK_E_OOM = 4,             /* device or host allocation failed */
    AMK_E_HIP = 5,             /* a HIP runtime call failed */
    AMK_E_NOT_RESIDENT = 6,    /* one workgroup per CU cannot be co-resident on this device */
    AMK_E_DEVICE_TIMEOUT = 7   /* a previous step hit the device watchdog (bounded spin-waits) */
} amk_status;

/* Weight format of the projection matrices (QKV, O, gate, up, down, LM head). */
typedef enum {
    AMK_F32 = 0,        /* fp32 weights; fp32 activations and KV cache when act_f32 = 1 */
    AMK_BF16 = 1,       /* bf16 weights */
    AMK_INT8_PC = 2,    /* int8, symmetric absmax per output row, fp16 scale (W8A16) */
    AMK_INT4_G128 = 3   /* int4 in [-7, 7], symmetric absmax per 128 input columns, fp16 scales */
} amk_wfmt;

/* Model shape. The decode step is the standard Llama step (RMSNorm, QKV projections, rotary
 * embedding on half-split pairs, grouped-query attention where query head h reads KV head
 * floor(h * n_kv_heads / n_heads), O projection + residual, RMSNorm, SwiGLU MLP + residual,
 * final RMSNorm, LM head, greedy argmax with the lowest index winning ties); pages: page 3,
 * "How it works" (the instruction list), page 1 "What's built". Biased projections are not
 * part of this family and cannot be expressed. */
typedef struct {
    uint32_t struct_size;     /* sizeof(amk_model_desc) */
    int32_t hidden, n_layers, n_heads, n_kv_heads, head_dim, intermediate, vocab;
    int32_t max_ctx;          /* KV cache rows per (layer, K/V, kv head) */
    int32_t tied_embeddings;  /* 1: the LM head is the embedding matrix */
    float rope_theta, rms_eps;
    int32_t wfmt;             /* amk_wfmt */
    int32_t act_f32;          /* 1: activations and KV cache fp32 (requires AMK_F32); 0: bf16 */
} amk_model_desc;

/* Canonical weights, device pointers, borrowed only for the duration of amk_create: the
 * library quantises (int formats) and repacks them into its own buffers and synchronises
 * before returning, so the caller may free them afterwards. Element type is fp32 when
 * wfmt == AMK_F32, else bf16 (the master that int formats are quantised from). Norm gains
 * and the embedding use the same element type. Per-layer entries are arrays of n_layers
 * device pointers (the arrays themselves are host memory). */
typedef struct {
    uint32_t struct_size;     /* sizeof(amk_weights) */
    const void* embed;        /* [vocab, hidden] */
    const void* final_norm;   /* [hidden] */
    const void* lm_head;      /* [vocab, hidden]; NULL when tied_embeddings */
    const void* const* attn_norm;  /* [hidden] each */
    const void* const* wq;         /* [n_heads*head_dim, hidden] */
    const void* const* wk;         /* [n_kv_heads*head_dim, hidden] */
    const void* const* wv;         /* [n_kv_heads*head_dim, hidden] */
    const void* const* wo;         /* [hidden, n_heads*head_dim] */
    const void* const* mlp_norm;   /* [hidden] */
    const void* const* wg;         /* [intermediate, hidden] */
    const void* const* wu;         /* [intermediate, hidden] */
    const void* const* wd;         /* [hidden, intermediate] */
} amk_weights;

/* ---------------------------------------------------------------- schedule IR
 * A schedule: tasks in per-CU queues; counters that tasks signal (+1 each per launch) and
 * wait on (value >= threshold, counted from the start of the launch, i.e. thresholds are
 * epoch-relative); the memory each task touches. The page-2 rule set (Table 1) decides
 * deadlock and race freedom; see amk_validate for the exact rules. */

#define AMK_ACC_WRITE 1u       /* access writes (else reads) */
#define AMK_ACC_POST 2u        /* access happens after the task's signals */
#define AMK_REGION_PLAIN 0u    /* ordinary memory */
#define AMK_REGION_LL 1u       /* flag-carrying words: written once per launch, the write is observed from the data */
#define AMK_REGION_RO 2u       /* read-only during a launch */
#define AMK_SCHED_LL_PROTOCOL 1u   /* schedule flag: waits are observed through flag-carrying reads (rule V8) */

/* opcodes of the kernel's instruction set (args in amk_task.arg[]) */
enum {
    AMK_OP_QKV = 1,      /* layer, arg0 = first row quad, arg1 = quad count: RMSNorm + QKV GEMV + RoPE + KV append */
    AMK_OP_ATTN = 2,     /* layer, arg0 = first query head, arg1 = head count, arg2 = chunk, arg3 = chunks */
    AMK_OP_MERGE = 3,    /* layer, arg0 = first query head, arg1 = head count, arg3 = chunks: split-context merge */
    AMK_OP_OPROJ = 4,    /* layer, arg0 = first row, arg1 = row count: O GEMV + residual */
    AMK_OP_GATEUP = 5,   /* layer, arg0 = first j, arg1 = count: RMSNorm + gate/up GEMV + SwiGLU */
    AMK_OP_DOWN = 6,     /* layer, arg0 = first row, arg1 = row count: down GEMV + residual */
    AMK_OP_LM = 7,       /* arg0 = first vocab row, arg1 = row count, arg2 = tile index: final RMSNorm + LM head + tile argmax */
    AMK_OP_ARGMAX = 8,   /* arg2 = number of LM tiles: greedy token */
    AMK_OP_ATTN_MERGE = 9 /* layer, arg0 = first query head, arg1 = head count, arg2 = chunk (the last),
                             arg3 = chunks: attention over the last context chunk, then the merge of
                             its state with the other chunks' states (AMK_OP_ATTN + AMK_OP_MERGE as
                             one task) */
};

typedef struct {
    uint32_t opcode, layer;
    uint32_t arg[4];
    uint32_t wait_off, wait_cnt;    /* into amk_schedule.waits */
    uint32_t sig_off, sig_cnt;      /* into amk_schedule.signals */
    uint32_t acc_off, acc_cnt;      /* into amk_schedule.accesses */
} amk_task;

typedef struct { uint32_t counter, threshold; } amk_wait;
typedef struct { uint32_t region, flags; uint64_t lo, hi; } amk_access;   /* element range [lo, hi) */
typedef struct { uint32_t region, pad; uint64_t lo, hi; } amk_range;

typedef struct {
    uint32_t struct_size;      /* sizeof(amk_schedule) */
    uint32_t flags;            /* AMK_SCHED_* */
    uint32_t n_tasks, n_queues, n_counters, n_regions;
    uint32_t n_waits, n_signals, n_accesses, n_inputs, n_outputs;
    const amk_task* tasks;             /* [n_tasks] */
    const uint32_t* queue_off;         /* [n_queues + 1]; queue q lists queue_tasks[queue_off[q] .. queue_off[q+1]) */
    const uint32_t* queue_tasks;       /* task ids in execution order */
    const amk_wait* waits;             /* [n_waits] */
    const uint32_t* signals;           /* [n_signals] counter ids */
    const amk_access* accesses;        /* [n_accesses] */
    const uint32_t* region_kind;       /* [n_regions] AMK_REGION_* */
    const amk_range* inputs;           /* [n_inputs] data defined before the launch */
    const amk_range* outputs;          /* [n_outputs] data the launch must produce */
} amk_schedule;

/* Verdict. accepted == (rule_mask == 0). Bits: 1 << k for rule Vk (k = 0..8). task, counter
 * and region name the first offender found (or -1); they are diagnostics only. */
typedef struct { int32_t accepted; uint32_t rule_mask; int32_t task, counter, region; } amk_verdict;

/* Knobs of the built-in lowering (the edit surface a schedule search varies; page 1,
 * "Two autoresearch loops", loop 2: tiling, SM assignment, pipelining depth, page allocation).
 * Zero means default. */
typedef struct {
    uint32_t struct_size;      /* sizeof(amk_schedule_config) */
    int32_t n_cu;              /* queues = workgroups; 0 = the device's CU count (amk_lower: 256) */
    int32_t tasks_qkv, tasks_o, tasks_gateup, tasks_down, tasks_lm;   /* tasks per GEMV phase (0 = min(n_cu, units)) */
    int32_t attn_chunks;       /* context chunks per attention head group (0 = auto: 1 below 256 cache
                                  rows, else the least of: CUs per head group, cache rows / 32, and
                                  the chunks whose merge states fit LDS) */
    int32_t attn_group_tasks;  /* 1: one attention task per KV group (up to 8 query heads), 2: one per
                                  query head, 0: auto (grouped when KV heads are shared and the
                                  cache holds at least 2048 positions) */
    int32_t cu_assign;         /* 0 = XCD-aware (unchunked attention of one KV group on one XCD; chunked
                                  attention round robin), 1 = plain round robin */
    int32_t prefetch_groups;   /* pipelining depth: groups of a GEMV task's weight loads (6 KiB per wave
                                  each) a wave issues as soon as the previous task's outputs are out,
                                  ahead of the task's inputs: 1 or 2, -1 for none, 0 = default (1).
                                  Used by amk_create (the kernel's launch parameters); the lowering
                                  only checks the range. */
    int32_t merge_fusion;      /* split-context attention (fusion grouping): 1 = the merge of a head
                                  group runs inside the task of its last context chunk
                                  (AMK_OP_ATTN_MERGE), which waits for the other chunks' states
                                  after its own positions; 2 = separate merge tasks (AMK_OP_MERGE)
                                  after every attention task; 0 = default (2, the faster of the two
                                  on every workload measured). 1 is refused (AMK_E_UNSUPPORTED)
                                  where the last chunk's LDS stage cannot hold every chunk state
                                  of its heads. */
} amk_schedule_config;

/* ---------------------------------------------------------------- calls */

/* Validate a schedule on the CPU: the pages' static safety gate, which refuses any schedule
 * that could deadlock or race before it runs (pages: page 1, "Deadlock-free by construction";
 * page 2, "1. Statically verified schedule IR"; page 4, "De Safety Gate"). Reentrant,
 * thread-safe, never touches a device. AMK_OK means the call ran; the verdict is in *out.
 * Rules (1 << k in rule_mask):
 *  V0 integrity: ids in range, every task in exactly one queue exactly once, lo < hi, no
 *     duplicate signal in a task, no write to a read-only region, no declared input/output
 *     and no post access on a flag-carrying region. When V0 fails nothing else is checked.
 *  V1 a wait threshold outside [1, P(c)], P(c) = number of tasks signalling counter c.
 *  V2 a partial wait (1 <= t < P(c)) on a counter with P(c) > 1.
 *  V3 the producer->waiter graph has a cycle (self-waits included).
 *  V4 the union graph (producer->waiter edges plus queue order) has a cycle although the
 *     producer->waiter graph has none: a queue is not a linear extension of the DAG.
 *  V5 (only without V3/V4) two accesses of different tasks overlap, one writes, and neither
 *     happens before the other; on flag-carrying regions any two overlapping writes.
 *  V6 a declared output is not covered by writes.
 *  V7 (only without V3/V4) a read is not covered by declared inputs plus writes that happen
 *     before it; on flag-carrying regions a write overlaps a read it does not precede.
 *  V8 (AMK_SCHED_LL_PROTOCOL only) a task waits on a counter one of whose producers writes
 *     nothing that the task reads from a flag-carrying region.
 * Happens-before is reachability in the union graph where each task is split into a pre node
 * (its waits enter, its signals leave) and a post node (AMK_ACC_POST accesses; queue order
 * leaves from it). Returns AMK_E_INVALID_ARG for null pointers or a wrong struct_size. */
amk_status amk_validate(const amk_schedule* sched, amk_verdict* out);

/* Run a schedule on the CPU under the kernel's synchronisation protocol and check it. Never
 * touches a device. One host thread per queue walks its tasks in order: a task waits until
 * every counter it waits on has reached its threshold, performs its pre accesses, increments
 * its signalled counters, then performs its post (AMK_ACC_POST) accesses. A deadlock (every
 * queue finished or blocked on a wait the counters cannot satisfy any more, at least one
 * blocked) is detected exactly when it happens; each wait is also bounded by a watchdog, whose
 * expiry is reported as a deadlock too (the device's timeout path). On either, every thread
 * stops. A seeded random
 * delay before each step varies the interleaving between runs. The declared accesses are
 * checked with vector clocks:
 *  - every queue carries a clock vector;
 *  - a counter carries the join of its signallers' clocks;
 *  - a wait that sees its threshold joins the counter's clock.
 * Two accesses of different tasks to one element, one a write, race when neither is ordered
 * before the other by queue order and waits. A wait joins every signaller seen so far, so a
 * partial wait on a multi-producer counter can hide a race but never makes one up. Reads of
 * elements nothing wrote before and no declared input covers are counted, and so are declared
 * output elements nothing wrote and flag-carrying elements written by two tasks in one launch.
 * Read-only regions are not tracked. The executor computes nothing; it checks the protocol.
 *  sched  host; must pass the structural part of V0 (ids in range, every task in exactly one
 *         queue exactly once), else AMK_E_INVALID_ARG. Borrowed for the call.
 *  opts   host; seed, the largest delay in microseconds (0 = none), the watchdog in
 *         milliseconds (0 = 2000), and the most shadow elements tracked (0 = 4M; regions past
 *         the budget are not checked and their elements are counted in `unchecked`).
 *  out    host; the outcome. */
typedef struct {
    uint32_t struct_size;      /* sizeof(amk_vm_opts) */
    uint32_t seed;
    uint32_t max_delay_us;
    uint32_t watchdog_ms;
    uint64_t max_elements;
} amk_vm_opts;

typedef struct {
    int32_t completed;          /* every queue ran to its end (no deadlock) */
    int32_t deadlocked;         /* no queue could move any more, or a wait outlived the watchdog */
    uint32_t races;             /* conflicting element accesses found unordered */
    uint32_t uncovered_reads;   /* read elements not written before and not declared inputs */
    uint32_t unwritten_outputs; /* declared output elements nothing wrote (completed runs) */
    int32_t task, other;        /* the task of the first problem found and its counterpart (or -1) */
    uint64_t unchecked;         /* accessed elements of regions past the shadow budget */
    uint32_t ll_rewrites;       /* flag-carrying elements written by a second task in the launch */
    uint32_t pad;
} amk_vm_result;

amk_status amk_vm_run(const amk_schedule* sched, const amk_vm_opts* opts, amk_vm_result* out);

/* Run the built-in lowering on the CPU (no device needed): model + config -> schedule. The
 * result is library-owned; free it with amk_schedule_free. AMK_E_UNSUPPORTED for shapes the
 * kernel does not implement (see amk_create). */
amk_status amk_lower(const amk_model_desc* desc, const amk_schedule_config* cfg, amk_schedule** out);
void amk_schedule_free(amk_schedule* sched);

typedef struct amk_ctx amk_ctx;

/* Build a context on the current device: lower (or take `sched`), validate, check that one
 * 512-thread workgroup per CU fits, quantise/repack the weights into library-owned device
 * memory, upload the task table and synchronise `stream`. This is the pages' compile step:
 * a model becomes a static per-SM (here per-CU) task program that passes the safety gate
 * before anything launches (AutoMegaKernel pages: page 2, "3. Agent-drivable compiler" and
 * "1. Statically verified schedule IR"; page 4, "De Safety Gate"; the quantised formats, page
 * 2, "Quantisation support and performance"). The device watchdog (how long any
 * single wait inside a step may last before the step gives up) is 2000 ms, or the value in
 * milliseconds of the environment variable AMK_WATCHDOG_MS when the context is created.
 *  desc      host; shape (AMK_E_UNSUPPORTED unless: head_dim in {16, 64, 128}; hidden and
 *            intermediate multiples of 16 (of 128 for AMK_INT4_G128, with n_heads * head_dim);
 *            n_heads % n_kv_heads == 0; act_f32 == 1 exactly with AMK_F32; vocab >= 2;
 *            hidden and n_heads * head_dim <= 8192; intermediate <= 16384).
 *  weights   host struct of device pointers, borrowed for this call only.
 *  kv_cache  device, caller-owned for the context's lifetime, layout
 *            [n_layers][2 (K, V)][n_kv_heads][max_ctx][head_dim] in the activation type
 *            (fp32 or bf16). K rows are stored after rotary embedding. Row `pos` is written
 *            by the step at `pos`; rows below `pos` are read; rows above are never touched.
 *  sched     host, optional: a schedule to run instead of the built-in lowering. Its tasks'
 *            access lists must equal what the kernel does for their opcodes (else V0).
 *  cfg       host, optional lowering knobs.
 *  stream    HIP stream for the set-up work (hipStream_t; NULL = default stream).
 *  verdict   host, optional: the validator's verdict (written on AMK_OK and AMK_E_REJECTED).
 * A rejected schedule returns AMK_E_REJECTED and allocates nothing. */
amk_status amk_create(const amk_model_desc* desc, const amk_weights* weights, void* kv_cache,
                      const amk_schedule* sched, const amk_schedule_config* cfg, void* stream,
                      amk_verdict* verdict, amk_ctx** out);

/* One decode step: enqueue exactly one cooperative launch on `stream` and return without
 * synchronising. One launch computes one forward pass and yields one greedy token (pages:
 * page 1, author's note and "What's built"; page 3, "How it works", layers 0 and 1).
 *  token_in   device int32[1]: the input token (read at the start of the launch).
 *  pos        host int, 0 <= pos < max_ctx (else AMK_E_INVALID_ARG and no launch).
 *  token_out  device int32[1]: the greedy token (may equal token_in: decode chains on the
 *             device with no host round trip).
 *  logits     device fp32[vocab] or NULL: the step's logits (not rounded).
 * A token outside [0, vocab) is replaced by 0 and flagged in the device status word. A
 * watchdog timeout in an earlier step (bounded spin-waits; only reachable with an invalid
 * schedule or broken hardware) is reported here as AMK_E_DEVICE_TIMEOUT without launching;
 * destroy and re-create the context to recover. A step that timed out still ends (its waits
 * give up and the launch runs to completion), but its outputs and the cache row it appends
 * at `pos` are unspecified. */
amk_status amk_decode_step(amk_ctx* ctx, const int32_t* token_in, int32_t pos, int32_t* token_out,
                           float* logits, void* stream);

/* The decode step of amk_decode_step, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): this call
 * allocates nothing. The step's scratch memory (its flag-carrying activation words: every
 * value one task publishes for another) lives in one static device array per GPU of
 * AMK_STATIC_SCRATCH_BYTES (64 MiB), set up by the first amk_create on that GPU and held until
 * the process ends. Every context on the GPU shares the array, and it keeps the last call's
 * contents: each call writes its words with a flag value no earlier call on that GPU used, so
 * nothing needs clearing between calls. Calls that overlap on one GPU (on two streams or from
 * two host threads) race on the array and give unspecified results: serialise them.
 * Arguments, effects and errors are those of amk_decode_step; in addition, a context whose step
 * needs more flag-carrying words than the array holds is refused with AMK_E_INVALID_ARG
 * (nothing launched; AMK_LOG=1 names the sizes). */
#define AMK_STATIC_SCRATCH_BYTES (64ull << 20)
amk_status amk_decode_step_static(amk_ctx* ctx, const int32_t* token_in, int32_t pos, int32_t* token_out,
                                  float* logits, void* stream);

/* Prompt prefill: run `n_tokens` prompt tokens through the model in cooperative launches of up
 * to 256 tokens each, instead of one decode launch per token (pages: page 3, "How it works",
 * layer 1, GEMM tiles among the instruction kinds). The result is the one of n_tokens chained
 * decode steps fed tokens[i] at position pos0 + i: cache rows [pos0, pos0 + n_tokens) are
 * written, rows below pos0 are read, and token_out / logits are those of the step at the last
 * position (the first generated token). The projections run as matrix-core GEMM tiles over the
 * chunk's tokens; the schedule of each chunk size is lowered, validated (amk_validate) and
 * uploaded on first use, and the first call allocates the chunk's activation buffers (about
 * 256 x (hidden + 2 x n_heads x head_dim + intermediate) activation values and a few doubles
 * per row), so it is
 * not capturable into a graph until every chunk size it uses has run once.
 *  tokens     device int32[n_tokens]; a token outside [0, vocab) is replaced by 0 and flagged
 *             in the device status word.
 *  pos0       host int, 0 <= pos0 and pos0 + n_tokens <= max_ctx (else AMK_E_INVALID_ARG).
 *  n_tokens   host int >= 1.
 *  token_out  device int32[1]: greedy token after the last prompt token.
 *  logits     device fp32[vocab] or NULL: the logits of the last prompt token.
 *  stream     HIP stream; the call enqueues its launches and returns without synchronising.
 * AMK_E_UNSUPPORTED when a weight row of the context's streams cannot be located (a user
 * schedule that splits rows) or head_dim > 128; AMK_E_DEVICE_TIMEOUT as for amk_decode_step. */
amk_status amk_prefill(amk_ctx* ctx, const int32_t* tokens, int32_t pos0, int32_t n_tokens, int32_t* token_out,
                       float* logits, void* stream);

/* The prefill schedule of one launch of n_tokens (1 .. 256) tokens for n_cu workgroups (0 =
 * 256), in the schedule IR, for inspection with amk_validate / amk_vm_run on the CPU. Phase
 * tasks over M-tiles of 64 tokens; every task of a phase waits on one counter signalled by all
 * tasks of the previous phase. Accesses are declared in tile units over these regions: 0 the
 * token ids (input), 1 the residual stream x, 2 the per-row sums of squares of x by column tile
 * (the RMSNorm inputs of the next GEMM, which fuses the norm), 3 the rotated queries,
 * 4 the attention output, 5 the SwiGLU output, 6 the LM tile results, 7 the logits (output),
 * 8 the token out (output), 9 + layer the K and V rows of the chunk in that layer's cache.
 * Caller frees with amk_schedule_free. */
amk_status amk_lower_prefill(const amk_model_desc* desc, int32_t n_cu, int32_t n_tokens, amk_schedule** out);

/* Device status word of the context (synchronises the context's last stream first):
 * 0 = fine; bit 0 = watchdog timeout; bit 1 = token out of range. */
uint32_t amk_device_status(amk_ctx* ctx);

/* The schedule the context runs (library-owned, valid until amk_destroy). */
const amk_schedule* amk_ctx_schedule(const amk_ctx* ctx);

/* Per-task timestamp trace (for critical-path and synchronisation-cost attribution of the
 * pages' per-tile sync overhead; page 2, "Performance analysis"; page 4, "Bottleneck
 * analysis"). When `trace` is non-NULL, every later amk_decode_step on this context writes,
 * for each task of the schedule, 6 uint64 values at trace[6 * k ...], where k is the task's
 * index in queue order (queue 0's tasks first; amk_ctx_schedule gives the order):
 *   [0] compute start, [1] inputs observed (all waits satisfied, prologue done),
 *   [2] rows / attention positions done (whole workgroup), [3] task end, [4] GEMV tasks: the
 *   first wave's own rows done, [5] outputs written (before the task's closing barrier),
 * in ticks of the device's constant 100 MHz realtime counter (one time base across CUs;
 * slots a task has no event for keep their old value). trace: device memory of at least
 * `capacity` uint64 values, caller-owned, borrowed until disabled; capacity must be at least
 * 6 * n_tasks (else AMK_E_INVALID_ARG). trace = NULL disables (the default). */
amk_status amk_set_trace(amk_ctx* ctx, uint64_t* trace, uint64_t capacity);

/* Per-task timestamp trace of the prefill launches (the same attribution of time to tasks and
 * to waits as amk_set_trace, for the prefill's tile tasks). When `trace` is non-NULL, every
 * later prefill launch whose schedule has at most capacity / 4 tasks writes, for each task, 4
 * uint64 values at trace[4 * k ...], k = the task's index in queue order of that launch's
 * schedule (amk_lower_prefill with the context's CU count and 64 x ceil(tokens / 64) tokens
 * gives the same schedule): [0] task start, [1] its wait satisfied, [2] its work done, [3]
 * signalled; ticks of the 100 MHz realtime counter. Launches with more tasks record nothing.
 * trace: device memory of `capacity` uint64 values, caller-owned, borrowed until disabled.
 * trace = NULL disables (the default). */
amk_status amk_set_prefill_trace(amk_ctx* ctx, uint64_t* trace, uint64_t capacity);

/* Synchronise the last stream, free every library-owned buffer; never touches caller
 * buffers. NULL-safe. (The end of the context amk_create built; the pages' runtime has the
 * same create / step / destroy life cycle, page 1, "What's built".) */
void amk_destroy(amk_ctx* ctx);

/* The library's own weight quantiser, exposed for bit-exact comparison with other
 * implementations (symmetric absmax, fp16 scales, codes decided in fp32, page 2,
 * "Quantisation support and performance"). master: device bf16 [rows, cols]. codes: device
 * int8 [rows, cols] (one code per byte, int4 codes in [-7, 7]); scales: device fp32 (the fp16
 * values widened) [rows] for AMK_INT8_PC, [rows, cols/128] for AMK_INT4_G128. Runs on
 * `stream` and synchronises it. */
amk_status amk_quantize(int32_t wfmt, const void* master, int64_t rows, int64_t cols, void* codes,
                        void* scales, void* stream);

/* Library version string. */
/* A measurement aid, not a step of the decode: read `bytes` of device memory once with the
 * same 16-byte non-temporal loads the decode kernel streams its weights with (2048 workgroups of
 * 512 threads), so that a caller timing the launch on `stream` gets the HBM read rate this GPU
 * reaches, the measured ceiling beside the specification's one for the roofline the pages
 * report (page 1, "Honesty rules"; page 3, "The results, read carefully").
 *  buf    device, 16-byte aligned, borrowed until the launch completes; `bytes` a positive
 *         multiple of 16 (else AMK_E_INVALID_ARG, nothing launched).
 *  out    device uint32[1]: written only when the xor of a thread's words equals a fixed value
 *         (it keeps the loads in the program); its content means nothing.
 * Enqueues one launch and returns without synchronising. */
amk_status amk_read_probe(const void* buf, uint64_t bytes, uint32_t* out, void* stream);

const char* amk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AMK_H */
