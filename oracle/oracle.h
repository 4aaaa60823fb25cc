/*
 * CPU oracle for one decode step of a Llama-style decoder: TEST INFRASTRUCTURE.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code with the HIP path.
 *
 * Sources.  The ops come from the page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞"
 * (m.youleyou.com), section "Megakernel：从零设计的深度融合方案", which names the
 * per-layer units the megakernel fuses (RMSNorm + QKV projection + RoPE,
 * attention, MLP), and the workload from the page "大模型吐一个字，显卡要启停两千四百次"
 * (zhichai.net), reply section: Llama-3.2-1B, batch 1, greedy decoding.  The
 * pages print no formula, so each op is its textbook definition: RMSNorm (Zhang
 * and Sennrich 2019), rotary embedding with rotate-half pairs (Su et al.,
 * RoFormer), grouped-query attention (Ainslie et al. 2023), SwiGLU (Shazeer
 * 2020), top-k softmax routing for the MoE variant (Shazeer et al. 2017).
 *
 * Precision contract: weights and the KV cache are bf16 (round to nearest even
 * when K and V are stored); every activation is fp32; every dot product
 * accumulates in double in index order and is rounded once to fp32; norm
 * statistics, RoPE rotations, softmax and SiLU are evaluated in double and
 * rounded to fp32.  Logits are fp32.
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t n_experts, top_k, n_shared, expert_ffn; /* n_experts == 0: dense FFN */
    double rms_eps, rope_theta;
} orc_cfg;

typedef struct {
    const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm;
    const uint16_t *w_gate, *w_up, *w_down;                 /* dense FFN: [F,d], [F,d], [d,F] */
    const uint16_t *router;                                 /* MoE: [E,d] */
    const uint16_t *const *e_gate, *const *e_up, *const *e_down; /* [E] x ([Fe,d], [Fe,d], [d,Fe]) */
    const uint16_t *s_gate, *s_up, *s_down;                 /* shared expert */
} orc_layer;

typedef struct {
    const uint16_t *embed;      /* [V,d] */
    const uint16_t *lm_head;    /* [V,d]; equal to embed when tied */
    const uint16_t *final_norm; /* [d] */
    const orc_layer *layers;    /* [n_layers] */
} orc_weights;

/* KV cache [L][B][Hkv][S][hd] bf16 bit patterns. */
typedef struct {
    uint16_t *k, *v;
    int32_t batch, max_seq;
} orc_cache;

/* Error codes */
#define ORC_OK 0
#define ORC_E_ARG 1
#define ORC_E_NAN 2

/* One decode step for all B sequences: token tok[b] sits at position pos[b];
 * K/V for that position are written into the cache, attention covers positions
 * 0..pos[b].  Writes logits [B][V] and the greedy tokens next[B]. */
int orc_step(const orc_cfg* c, const orc_weights* w, orc_cache* kv, int32_t B, const int32_t* pos,
             const int32_t* tok, float* logits, int32_t* next);

/* P tokens per sequence [B][P] in one layer-major pass (token t of sequence b at
 * position pos[b] + t); K/V of the new positions are written into the cache.
 * Equal, bit for bit, to P calls of orc_step.  Writes the logits of the last
 * position [B][V] and the greedy tokens next[B]. */
int orc_prefill(const orc_cfg* c, const orc_weights* w, orc_cache* kv, int32_t B, int32_t P, const int32_t* pos,
                const int32_t* tokens, float* logits, int32_t* next);

/* Optional per-layer MoE trace of the step above: sel [L][B][top_k] expert ids
 * (ascending) and prob [L][B][E] router probabilities.  NULL disables. */
void orc_set_moe_trace(int32_t* sel, float* prob);

/* Layer-major forward of one whole sequence without a cache (positions 0..n-1);
 * logits [n][V]. */
int orc_sequence(const orc_cfg* c, const orc_weights* w, const int32_t* tokens, int32_t n, float* logits);

/* FFN block of one layer (dense SwiGLU, or shared + routed experts) applied to
 * B residual rows h [B][d] in place: h += FFN(RMSNorm(h)). */
int orc_ffn(const orc_cfg* c, const orc_layer* lw, int32_t B, float* h);

/* ---- primitives, exported for the pin tests ---- */
uint16_t orc_bf16_bits(float x);
float orc_dot(const uint16_t* w, const float* x, int32_t n);
void orc_rmsnorm(const float* h, const uint16_t* g, int32_t d, double eps, float* x);
void orc_rope(float* v, int32_t hd, int32_t pos, double theta);
void orc_attend(const float* q, const uint16_t* K, const uint16_t* V, int64_t stride, int32_t n, int32_t hd,
                float* o);
float orc_swiglu(float z, float u);
int32_t orc_argmax(const float* v, int32_t n);
void orc_route(const float* zeta, int32_t E, int32_t k, int32_t* sel, float* prob);
int32_t orc_threads(void);

#ifdef __cplusplus
}
#endif
#endif
