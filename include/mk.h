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
    MK_MODE_GRAPH = 1       /* one kernel per op, replayed as a hipGraph [ROOT] */
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

/* Element strides of the K (and V) cache [L][B][Hkv][S][hd]; the V cache starts
 * kv_bytes / 2 bytes after K.  strides_out[0..4] for L, B, Hkv, S, hd. */
mk_status mk_kv_layout(const mk_handle* h, int64_t strides_out[5]);

/* Feed a prompt: d_tokens [B, P] int32 row-major on the device.  Runs P decode
 * steps (positions continue from the current context lengths), then writes the
 * logits of the last position to d_logits [B, V] and the greedy tokens to
 * d_next [B].  B must equal max_batch. */
mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P, float* d_logits,
                     int32_t* d_next, void* stream);

/* Set the context length of each sequence (host array [B]) after the caller
 * filled the KV cache directly (e.g. a synthetic context).  Enqueued on the
 * handle's creation stream. */
mk_status mk_set_context_len(mk_handle* h, const int32_t* h_lens, int32_t B);

/* One decode step: d_tokens_in [B] at positions ctx_len[b]; writes the greedy
 * tokens d_tokens_out [B] and logits d_logits [B, V]; every context grows by one.
 * d_tokens_in may alias d_tokens_out, so steps chain without the host.
 * MK_E_CAPACITY if a sequence is full; B must equal max_batch. */
mk_status mk_decode_step(mk_handle* h, const int32_t* d_tokens_in, int32_t B, int32_t* d_tokens_out,
                         float* d_logits, void* stream);

/* Host mirror of the context lengths (what the enqueued steps will have reached). */
mk_status mk_get_context_len(const mk_handle* h, int32_t* h_lens, int32_t B);

/* Clear the merge tickets and a latched device error (enqueued on `stream`); the
 * host mirror of the context lengths is re-read from the device.  The step
 * counter behind the value tags keeps counting, so values an aborted step left
 * behind never satisfy a later step. */
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
 * the q heads per KV head when one position split leaves compute units idle). */
mk_status mk_plan_inspect(const mk_model_config* cfg, const mk_runtime_config* rt, int32_t num_cus, int64_t* out,
                          int32_t cap);

/* Copy the device timeline of the last megakernel step (needs trace = 1).
 * Per compute unit `records_per_cu` records of 12 uint32: {op | layer << 16,
 * start, inputs staged, compute end, end, loader issue end, ticks waiting for
 * the loaders, ticks the loaders waited for ring space, staging start (after
 * the wave barrier), then for attention: inputs staged, KV groups consumed,
 * output written; for the other ops: compute end of waves 1, 2, 3}, times = low 32 bits of the 100 MHz
 * s_memrealtime clock, in queue order.  With h_buf == NULL only *written (the
 * byte size) is set.  Synchronises the handle's creation stream. */
mk_status mk_read_trace(mk_handle* h, void* h_buf, size_t bytes, size_t* written, int32_t* records_per_cu);

/* Number of kernel launches one decode step makes in the handle's mode. */
int32_t mk_kernels_per_step(const mk_handle* h);

mk_status mk_destroy(mk_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
