/*
 * mk.h - C ABI of the persistent decode megakernel for MI355X (gfx950).
 *
 * One call of mk_decode_step runs one whole low-batch decode step of a
 * Llama-style decoder - embedding lookup; per layer RMSNorm, QKV projection with
 * RoPE, GQA attention over the KV cache, O-projection with residual, SwiGLU MLP
 * or routed mixture of experts; final norm, LM head and greedy argmax - as ONE
 * persistent kernel launch with no kernel boundaries.
 *
 * Sources (no API is printed on them; they fix the behaviour):
 *  [MK]  page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞" (m.youleyou.com),
 *        section "Megakernel：从零设计的深度融合方案": the whole forward pass fused
 *        into one kernel; a per-SM plan of composite instructions whose
 *        dependencies are arranged before launch; an on-GPU interpreter with a
 *        uniform load/compute/store template; shared memory cut into pages so the
 *        next stage's weights load early; completion signals in global memory,
 *        watched by dependants instead of a grid barrier (here carried by each
 *        activation word as a tag naming its step and phase).
 *  [ROOT] same page, section "传统推理方式效率低下的根源剖析": the one-kernel-per-op
 *        design and its launch gaps (1.3-2.1 us even with graphs), the
 *        conventional path this library also provides (MK_MODE_GRAPH).
 *  [LOW] page "大模型吐一个字，显卡要启停两千四百次" (zhichai.net), sections
 *        "为什么只在低并发生效" and the reply: the path targets low concurrency,
 *        is opt-in and falls back to the normal path at high concurrency; the
 *        headline workload is Llama-3.2-1B, batch 1, 32 prompt tokens, 128
 *        greedy tokens.
 *  [MOE] same page, sections "两千四百次启停" and "AMD 先落了一子": decoders
 *        whose layers are mostly mixture-of-experts, with the expert layers
 *        (batch 4 and 8) fused into the resident kernel like the rest.
 *
 * Conventions
 *  - Every device pointer is CALLER-OWNED and borrowed until mk_destroy: weights,
 *    workspace, KV cache, token and logit buffers.  The library allocates no
 *    device memory; it owns the host-side handle, the schedule, and one small
 *    pinned host word for reporting device errors.
 *  - Every call that takes a stream enqueues on it and returns after host-side
 *    validation.  Host errors are synchronous return codes.  Device errors
 *    (watchdog expiry, NaN logits) are latched and reported by a later call as
 *    MK_E_DEVICE_TIMEOUT / MK_E_DEVICE_NAN; the handle then answers MK_E_STATE
 *    until mk_reset.
 *  - A handle is used from one host thread at a time.  No C++ exception crosses
 *    this boundary.
 *  - Weights are bf16 (bit patterns in uint16 storage), matrices row-major
 *    [out, in]; norm gains bf16 [hidden].  Tokens are int32, logits fp32 [B, V].
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MK_OK = 0,
    MK_E_INVALID = 1,        /* bad argument (NULL, size too small, B > max_batch ...) */
    MK_E_UNSUPPORTED = 2,    /* model or runtime shape outside the supported set */
    MK_E_CAPACITY = 3,       /* a sequence would exceed max_seq */
    MK_E_HIP = 4,            /* a HIP runtime call failed; see mk_last_error */
    MK_E_DEVICE_TIMEOUT = 5, /* a spin-wait on the device exceeded spin_timeout_ms */
    MK_E_STATE = 6,          /* handle is latched after a device error; call mk_reset */
    MK_E_DEVICE_NAN = 7      /* a logit was NaN */
} mk_status;

typedef enum {
    MK_MODE_MEGAKERNEL = 0, /* one persistent launch per step [MK] */
    MK_MODE_GRAPH = 1,      /* one kernel per op, replayed as a hipGraph [ROOT] */
    MK_MODE_ENV = 2         /* opt-in from the environment [LOW: the resident decode
                               kernel is off by default and enabled by an environment
                               variable]: MK_MEGAKERNEL=1 selects MK_MODE_MEGAKERNEL,
                               anything else (or unset) MK_MODE_GRAPH; read by
                               mk_query_sizes, mk_plan_inspect and mk_create */
} mk_mode;

/* GEMV arithmetic of the persistent mode.  Both read every weight once and
 * accumulate in fp32.  VALU: fp32 dot products of bf16 rows with the fp32
 * activations.  MFMA: v_mfma_f32_16x16x32_bf16 tiles of 16 rows x 32 columns
 * against the activations split into bf16 parts (3 parts at batch 1, 2 and 4,
 * 2 at batch 8: 24 or 16 mantissa bits of each fp32 activation), summed in
 * fp32.  AUTO takes VALU (faster at every supported batch on the 1B shape as
 * measured).  MK_MODE_GRAPH always computes with VALU; MK_GEMV_MFMA with it, or
 * where the parts area leaves too small a weight ring, is MK_E_UNSUPPORTED. */
typedef enum { MK_GEMV_AUTO = 0, MK_GEMV_VALU = 1, MK_GEMV_MFMA = 2 } mk_gemv_kind;

/* Model shape.  n_experts == 0 selects the dense SwiGLU FFN (ffn = its width).
 * n_experts > 0 selects a routed mixture of experts [MOE]: router logits, softmax
 * (in double, rounded to fp32), the top_k experts per sequence (ties to the lower
 * index), each a SwiGLU of width expert_ffn, plus n_shared_experts (0 or 1) with
 * weight 1; the expert outputs are added weighted by their probabilities in
 * ascending expert order.  MoE limits: n_experts <= 64, top_k <= 8, expert_ffn and
 * hidden multiples of 512 (hidden / 512 a power of two), the persistent mode and
 * the VALU GEMV only; otherwise MK_E_UNSUPPORTED. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t tied_embeddings; /* 1: the LM head is the token embedding */
    float rms_eps;
    double rope_theta;
    int32_t n_experts, top_k, n_shared_experts, expert_ffn;
} mk_model_config;

/* Device pointers of one layer (bf16).  wq [Hq*hd, d], wk/wv [Hkv*hd, d],
 * wo [d, Hq*hd], w_gate/w_up [ffn, d], w_down [d, ffn], norms [d].  A dense model
 * leaves the MoE fields NULL; an MoE model leaves w_gate/w_up/w_down NULL. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
    const void* router;                                     /* MoE [n_experts, d] */
    const void *const *e_gate, *const *e_up, *const *e_down; /* MoE: HOST arrays [n_experts] of device
                                                                pointers ([Fe, d], [Fe, d], [d, Fe]) */
    const void *s_gate, *s_up, *s_down;                     /* MoE shared expert (if any) */
} mk_layer_weights;

typedef struct {
    const void* tok_embedding; /* [V, d] */
    const void* lm_head;       /* [V, d]; NULL (or tok_embedding) when tied */
    const void* final_norm;    /* [d] */
    const mk_layer_weights* layers; /* HOST array [n_layers] */
} mk_weights;

typedef struct {
    int32_t max_batch;        /* 1..8 sequences per step */
    int32_t max_seq;          /* KV capacity per sequence */
    mk_mode mode;
    int32_t num_cus;          /* 0 = every compute unit of the device; the persistent
                                 mode needs num_cus <= the device's compute units (one
                                 resident workgroup each), else mk_create answers
                                 MK_E_UNSUPPORTED */
    int32_t gemv_kind;        /* mk_gemv_kind: how the weight-streaming GEMVs compute */
    uint32_t spin_timeout_ms; /* watchdog of every device spin-wait; 0 = 2000 ms */
    int32_t trace;            /* 1: record a per-instruction timeline (mk_read_trace) */
    int32_t attn_splits;      /* KV splits per (sequence, KV head); 0 = automatic */
    int32_t down_split;       /* dense down projection split by columns (per-part partial
                                 outputs from a transposed copy of Wdown that the workspace
                                 holds, then a per-row sum): 0 = automatic (batch 4 and 8,
                                 VALU GEMV, hidden <= 2048), 1 = on where supported, -1 = off.
                                 mk_create_static never splits. */
} mk_runtime_config;

typedef struct mk_handle mk_handle;

/* Bytes of caller-provided device memory that mk_create needs for this model and
 * runtime: the workspace (schedule, tickets, tagged activations, RoPE table) and the
 * KV cache [2][n_layers][max_batch][n_kv_heads][max_seq][head_dim] bf16.
 * Host only; MK_E_UNSUPPORTED for shapes this build does not run. */
mk_status mk_query_sizes(const mk_model_config* cfg, const mk_runtime_config* rt, size_t* workspace_bytes,
                         size_t* kv_bytes);

/* Validate, build and verify the static schedule [MK: per-SM plan, dependencies
 * arranged before launch], lay out the workspace, upload the schedule and the
 * RoPE table on `stream`, and return a handle.  `stream` is a hipStream_t (NULL =
 * the default stream).  The KV cache is zero-filled; every context length is 0. */
mk_status mk_create(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt, void* d_workspace,
                    size_t workspace_bytes, void* d_kv, size_t kv_bytes, void* stream, mk_handle** out);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): mk_create with the
 * workspace taken from a static device array of MK_STATIC_WORKSPACE_BYTES that
 * the library holds on every device it runs on until the process ends.  The
 * caller still provides the weights and the KV cache (kv_bytes as from
 * mk_query_sizes).  The call allocates no device or pinned host memory (it
 * builds the schedule in host memory, clears the array and uploads the schedule
 * and RoPE table on `stream`, then synchronises it).  Persistent mode only
 * (MK_MODE_MEGAKERNEL, or MK_MODE_ENV resolving to it), else MK_E_UNSUPPORTED;
 * a configuration whose workspace exceeds the array is MK_E_CAPACITY; one live
 * handle per device uses the array, a second is MK_E_STATE until the first is
 * destroyed (calls on handles that overlapped on one device would race on it).
 * Such a handle has no host-mapped error word (that would be an allocation): a
 * device error (watchdog, NaN logit) stays latched on the device and is
 * returned by the next mk_reset, which clears it. */
#define MK_STATIC_WORKSPACE_BYTES (32u << 20)
mk_status mk_create_static(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt, void* d_kv,
                           size_t kv_bytes, void* stream, mk_handle** out);

/* Layout of the caller's KV cache, which the step reads for attention and
 * appends to [MK: attention is one of the fused per-layer instructions; LOW: the
 * workload decodes against the cache its prompt left].  strides_out[0..4]
 * (host array of 5, written) are the element strides of the K cache
 * [L][B][Hkv][S][hd] (bf16 elements) for L, B, Hkv, S, hd; the V cache has the
 * same layout and starts kv_bytes / 2 bytes after K.  Host only, no device work.
 * MK_E_INVALID for a NULL argument. */
mk_status mk_kv_layout(const mk_handle* h, int64_t strides_out[5]);

/* Feed a prompt [LOW: the headline workload first consumes a 32-token prompt,
 * then decodes greedily; page "一个大内核不够：在哪里切分流式推理模型", section
 * "为什么切在哪里比融不融更关键": the prompt is processed once, before the decode
 * loop, and sets the first token's latency].  d_tokens: device int32 [B, P]
 * row-major, read only.  In the persistent mode, when the handle carries the
 * multi-position plan (see mk_verify_step), each sequence's prompt runs in
 * launches of up to 8 positions (causal attention within the launch, every
 * position's K/V appended); otherwise, and in the graph mode, it runs as P decode
 * steps.  Positions continue from the current context lengths and every context
 * grows by P.  Writes the last position's logits to d_logits (device
 * fp32 [B, V]) and its greedy tokens to d_next (device int32 [B]); the other
 * positions' logits land in the workspace.  Enqueued on `stream`; returns after
 * host-side checks.  B must equal max_batch (the schedule, the staging areas and
 * the kernel are built for max_batch sequences and every weight byte is read
 * once for all of them, so fewer sequences would cost the same launch: pad the
 * batch instead), else MK_E_INVALID; MK_E_CAPACITY if a context would pass
 * max_seq; MK_E_STATE / MK_E_DEVICE_* when a device error is latched. */
mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P, float* d_logits,
                     int32_t* d_next, void* stream);

/* Several positions of ONE sequence in one persistent launch [page
 * "16块谷歌TPU v7跑Kimi K3，每秒跑出了709个Token，比老黄的GB200快了57%", section
 * "不异16块芯片，TPU快57%": a draft model proposes several tokens and the target
 * model checks them in one pass, accepting about six per pass].  d_tokens: device
 * int32 [n], 1 <= n <= 8: tokens at positions ctx .. ctx + n - 1 of sequence
 * `seq` (0 <= seq < max_batch), ctx its current context length.  Every position
 * attends to the sequence's cache and to the earlier positions of the call
 * (causal), and appends its K/V.  Writes the logits of every position to d_logits
 * (device fp32 [n, V]) and their greedy tokens to d_next (device int32 [n]); the
 * context grows by n (to accept fewer draft tokens, set the length back with
 * mk_set_context_len; later steps overwrite the rejected positions).  The same
 * launch serves mk_prefill.  Available in the persistent mode for configurations
 * whose batch-8 layout fits (MK_E_UNSUPPORTED otherwise: hidden 4096 dense
 * models); MK_E_INVALID for bad arguments, MK_E_CAPACITY past max_seq,
 * MK_E_STATE / MK_E_DEVICE_* when a device error is latched.  Enqueued on
 * `stream`. */
mk_status mk_verify_step(mk_handle* h, int32_t seq, const int32_t* d_tokens, int32_t n, float* d_logits,
                         int32_t* d_next, void* stream);

/* Set the context length of each sequence after the caller filled the KV cache
 * directly (e.g. a synthetic context) [LOW: the low-concurrency measurements
 * include long contexts].  h_lens: host int32 [B], each 0..max_seq, copied.
 * The new lengths are uploaded on the handle's creation stream, which is then
 * synchronised.  B must equal max_batch (MK_E_INVALID), a length outside
 * 0..max_seq is MK_E_CAPACITY. */
mk_status mk_set_context_len(mk_handle* h, const int32_t* h_lens, int32_t B);

/* One decode step as ONE persistent kernel launch in MK_MODE_MEGAKERNEL [MK: the
 * whole forward pass fused into one kernel, per-CU instruction plans built
 * before launch, data-carried completion signals instead of a grid barrier], or
 * as the replay of a graph of one kernel per op in MK_MODE_GRAPH [ROOT].
 * d_tokens_in: device int32 [B], the token of each sequence at position
 * ctx_len[b]; d_tokens_out: device int32 [B], the greedy tokens (lowest id on
 * ties); d_logits: device fp32 [B, V].  d_tokens_in may alias d_tokens_out, so
 * steps chain on the device without the host.  Every context grows by one.
 * Enqueued on `stream`; returns after host-side checks.  MK_E_CAPACITY if a
 * sequence is full; B must equal max_batch (see mk_prefill), else MK_E_INVALID;
 * a device error of an earlier step (watchdog, NaN logit) is reported here as
 * MK_E_DEVICE_TIMEOUT / MK_E_DEVICE_NAN and latches the handle. */
mk_status mk_decode_step(mk_handle* h, const int32_t* d_tokens_in, int32_t B, int32_t* d_tokens_out,
                         float* d_logits, void* stream);

/* Host mirror of the context lengths (what the enqueued steps will have reached). */
mk_status mk_get_context_len(const mk_handle* h, int32_t* h_lens, int32_t B);

/* Recover after a device error [MK: nothing is decided at run time, so a step
 * that failed leaves only stale values and tickets behind].  Synchronises
 * `stream`, re-reads the context lengths from the device into the host mirror,
 * clears the merge tickets and the latched error, and synchronises again.  The
 * step counter behind the value tags keeps counting, so values an aborted step
 * left behind never satisfy a later step.  MK_E_HIP if a runtime call fails.
 * For a handle of mk_create_static (no host-mapped error word) it returns the
 * device error it cleared (MK_E_DEVICE_TIMEOUT / MK_E_DEVICE_NAN), MK_OK if none. */
mk_status mk_reset(mk_handle* h, void* stream);

/* Test hook: fault 1 = the next step runs with a 1 ms watchdog and its layer-0
 * attention waits for a value tag that no instruction writes, so every
 * workgroup times out or sees the error and exits (the step reports
 * MK_E_DEVICE_TIMEOUT); fault 0 clears a pending fault.  Both modes. */
mk_status mk_debug_inject(mk_handle* h, int32_t fault, int32_t arg);

/* Human-readable status / last host-side error of a handle. */
const char* mk_status_string(mk_status s);
const char* mk_last_error(const mk_handle* h);

/* Host-side description of the schedule (for tests and reports).  Fills up to
 * `cap` int64 values: [0] compute units, [1] instructions, [2] LDS ring chunks
 * (1 KB each), [3] max instructions on one CU, [4] weight bytes per step,
 * [5] verifier result (0 = ok), [6] attention splits, [7] phases, [8] LDS bytes of
 * staged activations, [9] LM-head instructions, [10] the GEMV kind in effect
 * (MK_GEMV_VALU or MK_GEMV_MFMA), [11] q-head groups per attention item (1, or
 * the q heads per KV head when one position split leaves compute units idle),
 * [12] the most ring chunks one compute wave holds while it waits for its data
 * (mk_create refuses a configuration where this exceeds [2]), [13] 1 when the dense
 * down projection is split by columns, then 1 when the batch-1 path applies: [14]
 * the (gate, up) rows computed by the loader waves from registers, [15] the down
 * projection reduced by column quarters, [16] the O rows computed by the loader
 * waves. */
mk_status mk_plan_inspect(const mk_model_config* cfg, const mk_runtime_config* rt, int32_t num_cus, int64_t* out,
                          int32_t cap);

/* Copy the device timeline of the last megakernel step (needs trace = 1).
 * Per compute unit `records_per_cu` records of 12 uint32: {op | layer << 16,
 * start, inputs staged, compute end, end, loader issue end, ticks waiting for
 * the loaders, ticks the loaders waited for ring space, staging start (after
 * the wave barrier), then for attention: inputs staged, KV groups consumed,
 * output written; for a (gate, up) instruction whose rows the loader waves stream
 * into registers (batch 1, hidden 2048): loader 0's rows requested, input seen,
 * rows done; for the other ops: compute end of waves 1, 2, 3}, times = low 32 bits of the 100 MHz
 * s_memrealtime clock, in queue order.  With h_buf == NULL only *written (the
 * byte size) is set.  Synchronises the handle's creation stream. */
mk_status mk_read_trace(mk_handle* h, void* h_buf, size_t bytes, size_t* written, int32_t* records_per_cu);

/* Expert slots the MoE layers have streamed since mk_create: per (step, MoE
 * layer) the shared experts plus the union of the experts the batch's sequences
 * selected [page "大模型吐一个字，显卡要启停两千四百次", section "两千四百次启停":
 * only the selected experts' weights are read].  Times the bytes of one
 * expert's three matrices, it is the expert weight traffic of those steps, so a
 * difference of two readings gives the exact algorithmic bytes of the steps in
 * between.  Dense models read 0.  Synchronises the streams the handle ran on;
 * *out is left unchanged on error. */
mk_status mk_moe_slots(mk_handle* h, uint64_t* out);

/* Cut each decode step into several persistent launches [page
 * "一个大内核不够：在哪里切分流式推理模型", sections "为什么切在哪里比融不融更关键" and
 * "规划器总览：只用常规画像排序切分": where the fused region ends is a design choice;
 * a step may run as k >= 1 resident launches].  h_layers: host int32 [n], strictly
 * increasing layer indices in 1..n_layers; a new launch starts before each of
 * those layers (n_layers: the LM head runs alone).  n = 0 restores one launch per
 * step.  Every launch runs its CUs' instructions of its layers in the usual order,
 * so the results are bit for bit those of one launch; each cut costs a launch and
 * the loss of the weights the loaders would have prefetched across it.  Persistent
 * mode without the device trace only (MK_E_UNSUPPORTED); MK_E_INVALID for bad
 * cuts or more than 63 of them.  Synchronises the handle's streams. */
mk_status mk_set_cuts(mk_handle* h, const int32_t* h_layers, int32_t n);

/* ---- Cut planner [page "一个大内核不够：在哪里切分流式推理模型", sections
 * "规划器总览：只用常规画像排序切分", "瓦片图如何估计单次服务时间" and
 * "事件图如何算出首次发布分数"]: candidate designs are scored by simulating their
 * launches as an event graph up to the first release, from per-region service
 * times; no candidate is run end to end.  Host only, no device work. */

#define MK_EVENT_MAX_DEPS 8
/* One event-graph task: it starts when its dependencies (earlier tasks) have
 * finished and the previous task of its stream has finished, plus its dispatch
 * cost, and runs for `duration`.  Tasks on different streams run side by side
 * (their durations are the ones for the resources each stream is given). */
typedef struct {
    double duration;  /* service time (any unit, the same for all tasks) */
    double dispatch;  /* launch / switch cost paid before it starts */
    int32_t stream;   /* 0..1023 */
    int32_t n_deps;   /* 0..MK_EVENT_MAX_DEPS */
    int32_t deps[MK_EVENT_MAX_DEPS]; /* indices of earlier tasks */
} mk_event_task;

/* Finish time of every task (host double [n]), tasks in dependency order.
 * MK_E_INVALID for a dependency on a later task, a negative time or a bad stream. */
mk_status mk_event_sim(const mk_event_task* tasks, int32_t n, double* h_finish);

/* Service table of a decode step: regions are the n_layers layers and the LM head. */
typedef struct {
    int32_t n_layers;
    double launch_us;         /* dispatch of one persistent launch */
    const double* layer_us;   /* [n_layers]: a layer inside a launch, its weights prefetched */
    const double* refill_us;  /* [n_layers + 1] or NULL: extra time when a launch starts at that
                                 region (nothing prefetched; index n_layers: the LM head) */
    double head_us;           /* final norm, LM head and argmax */
    double conventional_us;   /* the one-kernel-per-op step, 0 if not a candidate */
} mk_cut_costs;

/* Best design for the service table: one-kernel-per-op, or persistent launches
 * starting at region 0 and at the *n_cuts regions written to h_cut_layers (host
 * int32, room for n_layers; pass them to mk_set_cuts).  Every cut set is
 * simulated up to 16 layers, beyond that the optimum of the same additive score
 * is found by dynamic programming.  *predicted_us: the chosen design's step
 * time; *single_launch_us: one persistent launch's; *use_conventional: 1 if the
 * one-kernel-per-op path wins.  MK_E_INVALID for a bad table. */
mk_status mk_plan_cuts(const mk_cut_costs* costs, int32_t* h_cut_layers, int32_t* n_cuts, double* predicted_us,
                       double* single_launch_us, int32_t* use_conventional);

/* Number of kernel launches one decode step makes in the handle's mode. */
int32_t mk_kernels_per_step(const mk_handle* h);

mk_status mk_destroy(mk_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
