// Host runtime behind include/mk.h: validation, workspace layout, the static
// scheduler that fills per-CU instruction queues and its verifier, the RoPE
// table, and the launch of one decode step in either mode.
//
// Scheduling follows the page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞",
// section "Megakernel：从零设计的深度融合方案": before launch every compute unit gets
// an ordered plan of composite instructions and each dependency is fixed
// statically as (counter, number of producers); nothing is decided at run time.
// Every weight matrix is split by rows into one contiguous tile per compute unit
// (equal bytes per CU, so no CU forms a straggling tail - the wave-quantisation
// effect the page "大模型吐一个字，显卡要启停两千四百次", section "两千四百次启停",
// describes for 512 blocks on 148 SMs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {
hipError_t launch_megakernel(const Params& P, const StepArgs& A, hipStream_t stream);
bool megakernel_supports(int B, int hd);
hipError_t launch_conventional(const Params& P, const StepArgs& A, uint32_t* head_ticket, hipStream_t stream);
int conventional_kernels_per_step(const Params& P);
int conventional_head_blocks(const Params& P);
}  // namespace mk

using namespace mk;

namespace {

constexpr int kMaxCus = 1024;

struct Plan {
    std::vector<Instr> instrs;
    std::vector<uint32_t> qoff;  // [n_cu + 1]
    uint32_t n_ctr = 0, head_ctr = 0, conv_ticket_ctr = 0, n_head = 0;
    uint32_t n_phase = 0, flag_stride = 64;
    int n_cu = 0, nsplit = 1;
    int phases = 0;
    size_t max_per_cu = 0;
};

int auto_splits(const mk_model_config* c, const mk_runtime_config* rt, int n_cu) {
    if (rt->attn_splits > 0) return rt->attn_splits;
    const int pairs = std::max(1, rt->max_batch * c->n_kv_heads);
    int by_cu = std::max(1, n_cu / pairs);
    int by_len = std::max(1, (rt->max_seq + 63) / 64);
    return std::max(1, std::min(std::min(by_cu, by_len), 64));
}

mk_status validate(const mk_model_config* c, const mk_runtime_config* rt, std::string* why) {
    auto fail = [&](mk_status s, const char* m) {
        if (why) *why = m;
        return s;
    };
    if (!c || !rt) return fail(MK_E_INVALID, "null config");
    if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
        c->vocab <= 0)
        return fail(MK_E_INVALID, "non-positive model dimension");
    if (c->n_experts != 0) return fail(MK_E_UNSUPPORTED, "MoE decoders are not supported by this build");
    if (c->ffn <= 0) return fail(MK_E_INVALID, "ffn must be positive");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(MK_E_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->n_q_heads % c->n_kv_heads) return fail(MK_E_UNSUPPORTED, "n_q_heads must be a multiple of n_kv_heads");
    if (c->n_q_heads / c->n_kv_heads > kMaxGroup) return fail(MK_E_UNSUPPORTED, "more than 4 q heads per KV head");
    if (c->hidden % 256 || c->ffn % 64) return fail(MK_E_UNSUPPORTED, "hidden % 256 and ffn % 64 must be 0");
    if (c->n_q_heads * c->head_dim > 16384) return fail(MK_E_UNSUPPORTED, "attention width above 16384");
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.0)) return fail(MK_E_INVALID, "rms_eps and rope_theta must be > 0");
    if (rt->max_batch < 1 || rt->max_batch > kMaxBatch) return fail(MK_E_UNSUPPORTED, "max_batch must be 1..8");
    if (!megakernel_supports(rt->max_batch, c->head_dim))
        return fail(MK_E_UNSUPPORTED, "this build runs batch 1 and 2");
    if ((size_t)rt->max_batch * c->hidden * 4 > kXBytes) return fail(MK_E_UNSUPPORTED, "batch x hidden too large");
    if (rt->max_seq < 1 || rt->max_seq > (1 << 20)) return fail(MK_E_INVALID, "max_seq out of range");
    if (rt->mode != MK_MODE_MEGAKERNEL && rt->mode != MK_MODE_GRAPH) return fail(MK_E_INVALID, "unknown mode");
    if (rt->num_cus < 0 || rt->num_cus > kMaxCus) return fail(MK_E_INVALID, "num_cus out of range");
    if (rt->gemv_kind < 0 || rt->gemv_kind > 1) return fail(MK_E_UNSUPPORTED, "gemv_kind must be 0 or 1");
    if (rt->trace != 0 && rt->trace != 1) return fail(MK_E_INVALID, "trace must be 0 or 1");
    if (rt->attn_splits < 0 || rt->attn_splits > 256) return fail(MK_E_INVALID, "attn_splits out of range");
    return MK_OK;
}

// Rows [c*R/n, (c+1)*R/n) for compute unit c.
inline void tile(uint32_t R, int n, int c, uint32_t* b, uint32_t* cnt) {
    const uint64_t lo = (uint64_t)R * c / n, hi = (uint64_t)R * (c + 1) / n;
    *b = (uint32_t)lo;
    *cnt = (uint32_t)(hi - lo);
}

Plan build_plan(const mk_model_config* c, const mk_runtime_config* rt, int n_cu) {
    Plan pl;
    pl.n_cu = n_cu;
    pl.nsplit = auto_splits(c, rt, n_cu);
    const int L = c->n_layers, B = rt->max_batch;
    const uint32_t qkv_rows = (uint32_t)((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim);
    std::vector<std::vector<Instr>> q(n_cu);
    auto mk_instr = [](uint16_t op, int layer, uint32_t begin, uint32_t count, uint16_t wc, uint32_t wn, uint16_t sc) {
        Instr in;
        std::memset(&in, 0, sizeof(in));
        in.op = op;
        in.layer = (uint16_t)layer;
        in.begin = begin;
        in.count = count;
        in.wait_ctr = wc;
        in.wait_n = wn;
        in.sig_ctr = sc;
        return in;
    };
    uint16_t prev_ctr = kNoCounter;
    uint32_t prev_n = 0;
    auto gemv_phase = [&](uint16_t op, int layer, uint32_t R, uint16_t ctr) {
        uint32_t n = 0;
        for (int cu = 0; cu < n_cu; ++cu) {
            uint32_t b, cnt;
            tile(R, n_cu, cu, &b, &cnt);
            if (!cnt) continue;
            Instr in = mk_instr(op, layer, b, cnt, prev_ctr, prev_n, ctr);
            in.slot = n++;
            q[cu].push_back(in);
        }
        pl.flag_stride = std::max(pl.flag_stride, (n + 63u) & ~63u);
        prev_ctr = ctr;
        prev_n = n;
        ++pl.phases;
    };
    for (int l = 0; l < L; ++l) {
        const uint16_t base = (uint16_t)(l * kPhasesPerLayer);
        gemv_phase(OP_QKV, l, qkv_rows, base + 0);
        // attention items: (b, g, s) spread one per CU round-robin
        const uint32_t items = (uint32_t)(B * c->n_kv_heads * pl.nsplit);
        for (uint32_t it = 0; it < items; ++it) {
            Instr in = mk_instr(OP_ATTN, l, it, 1, prev_ctr, prev_n, (uint16_t)(base + 1));
            in.slot = it;
            q[it % n_cu].push_back(in);
        }
        pl.flag_stride = std::max(pl.flag_stride, (items + 63u) & ~63u);
        prev_ctr = (uint16_t)(base + 1);
        prev_n = items;
        ++pl.phases;
        gemv_phase(OP_O, l, (uint32_t)c->hidden, base + 2);
        gemv_phase(OP_GATEUP, l, (uint32_t)c->ffn, base + 3);
        gemv_phase(OP_DOWN, l, (uint32_t)c->hidden, base + 4);
    }
    pl.head_ctr = (uint32_t)(L * kPhasesPerLayer);
    gemv_phase(OP_HEAD, L, (uint32_t)c->vocab, (uint16_t)pl.head_ctr);
    pl.n_head = prev_n;
    pl.conv_ticket_ctr = pl.head_ctr + 1;
    pl.n_ctr = pl.head_ctr + 2;
    pl.n_phase = pl.head_ctr + 1;
    pl.qoff.resize(n_cu + 1);
    pl.qoff[0] = 0;
    for (int cu = 0; cu < n_cu; ++cu) {
        pl.qoff[cu + 1] = pl.qoff[cu] + (uint32_t)q[cu].size();
        pl.max_per_cu = std::max(pl.max_per_cu, q[cu].size());
        pl.instrs.insert(pl.instrs.end(), q[cu].begin(), q[cu].end());
    }
    return pl;
}

// Every row / item exactly once; each queue in strictly increasing phase order;
// every wait names the phase right before its own and the number of
// instructions that phase emitted.  Returns 0 or an error code.
int verify_plan(const mk_model_config* c, const mk_runtime_config* rt, const Plan& pl) {
    const int L = c->n_layers, B = rt->max_batch;
    const uint32_t qkv_rows = (uint32_t)((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim);
    const int nphase = L * kPhasesPerLayer + 1;
    std::vector<uint32_t> emitted(nphase, 0);
    std::vector<std::vector<uint8_t>> seen(nphase);
    auto phase_of = [&](const Instr& in) -> int {
        if (in.op == OP_HEAD) return L * kPhasesPerLayer;
        const int k = in.op == OP_QKV ? 0 : in.op == OP_ATTN ? 1 : in.op == OP_O ? 2 : in.op == OP_GATEUP ? 3 : 4;
        return in.layer * kPhasesPerLayer + k;
    };
    auto extent = [&](int ph) -> uint32_t {
        if (ph == L * kPhasesPerLayer) return (uint32_t)c->vocab;
        switch (ph % kPhasesPerLayer) {
            case 0: return qkv_rows;
            case 1: return (uint32_t)(B * c->n_kv_heads * pl.nsplit);
            case 2: return (uint32_t)c->hidden;
            case 3: return (uint32_t)c->ffn;
            default: return (uint32_t)c->hidden;
        }
    };
    for (int ph = 0; ph < nphase; ++ph) seen[ph].assign(extent(ph), 0);
    for (int cu = 0; cu < pl.n_cu; ++cu) {
        int last = -1;
        for (uint32_t i = pl.qoff[cu]; i < pl.qoff[cu + 1]; ++i) {
            const Instr& in = pl.instrs[i];
            if (in.op < OP_QKV || in.op > OP_HEAD) return 1;
            if (in.op != OP_HEAD && in.layer >= L) return 2;
            const int ph = phase_of(in);
            if (ph < last) return 3;  // queue not in phase order
            last = ph;
            if (in.sig_ctr != ph) return 4;
            const uint32_t ext = extent(ph);
            if (in.count == 0 || in.begin + in.count > ext) return 5;
            for (uint32_t r = in.begin; r < in.begin + in.count; ++r) {
                if (seen[ph][r]) return 6;  // covered twice
                seen[ph][r] = 1;
            }
            ++emitted[ph];
            if (ph == 0) {
                if (in.wait_ctr != kNoCounter) return 7;
            } else if (in.wait_ctr != ph - 1) {
                return 8;
            }
        }
    }
    for (int ph = 0; ph < nphase; ++ph)
        for (uint8_t s : seen[ph])
            if (!s) return 9;  // row never covered
    for (int cu = 0; cu < pl.n_cu; ++cu)
        for (uint32_t i = pl.qoff[cu]; i < pl.qoff[cu + 1]; ++i) {
            const Instr& in = pl.instrs[i];
            if (in.wait_ctr != kNoCounter && in.wait_n != emitted[in.wait_ctr]) return 10;
        }
    if (pl.n_head != emitted[L * kPhasesPerLayer]) return 11;
    std::vector<std::vector<uint8_t>> slot_seen(nphase);
    for (int ph = 0; ph < nphase; ++ph) slot_seen[ph].assign(emitted[ph], 0);
    for (const Instr& in : pl.instrs) {
        if (in.slot >= emitted[in.sig_ctr] || in.slot >= pl.flag_stride) return 12;
        if (slot_seen[in.sig_ctr][in.slot]++) return 13;  // two producers share a flag
    }
    return 0;
}

struct Layout {
    size_t state, counters, flags, flags_bytes, tickets, instrs, qoff, layers, rope, h, qkv, attn, act, attn_part, head_part, logits_scr,
        tok_scr, trace, trace_bytes, total;
    size_t head_slots;
};

inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(const mk_model_config* c, const mk_runtime_config* rt, int n_cu, int nsplit, size_t n_instr,
              uint32_t n_ctr, uint32_t flag_stride) {
    Layout lo{};
    const size_t B = (size_t)rt->max_batch, d = c->hidden, hd = c->head_dim;
    const size_t qkv_rows = (size_t)(c->n_q_heads + 2 * c->n_kv_heads) * hd;
    const size_t G = (size_t)(c->n_q_heads / c->n_kv_heads);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    lo.state = take(sizeof(DevState));
    lo.counters = take((size_t)n_ctr * kCtrStride * 4);
    lo.flags_bytes = (size_t)n_ctr * flag_stride * 4;
    lo.flags = take(lo.flags_bytes);
    lo.tickets = take((size_t)c->n_layers * B * c->n_kv_heads * kCtrStride * 4);
    lo.instrs = take(n_instr * sizeof(Instr));
    lo.qoff = take((size_t)(n_cu + 1) * 4);
    lo.layers = take((size_t)c->n_layers * sizeof(DevLayer));
    lo.rope = take((size_t)rt->max_seq * (hd / 2) * 8);
    lo.h = take(B * d * 4);
    lo.qkv = take(B * qkv_rows * 4);
    lo.attn = take(B * c->n_q_heads * hd * 4);
    lo.act = take(B * c->ffn * 4);
    lo.attn_part = take(B * c->n_kv_heads * nsplit * G * (hd + 2) * 4);
    const size_t conv_blocks = ((size_t)c->vocab + 15) / 16;
    lo.head_slots = std::max((size_t)n_cu, conv_blocks) * kComputeWaves;
    lo.head_part = take(lo.head_slots * B * sizeof(HeadPart));
    lo.logits_scr = take(B * c->vocab * 4);
    lo.tok_scr = take(B * 4);
    // trace: one record per instruction slot; a CU holds at most 5 per layer + the head,
    // plus the attention items beyond one per CU
    const size_t items = B * c->n_kv_heads * nsplit;
    const size_t per_cu = (size_t)c->n_layers * (4 + (items + n_cu - 1) / n_cu) + 1;
    lo.trace_bytes = rt->trace ? (size_t)n_cu * per_cu * kTraceWords * 4 : 0;
    lo.trace = take(lo.trace_bytes);
    lo.total = off;
    return lo;
}

// Upper bound on the instruction count for any n_cu <= cus.
size_t max_instrs(const mk_model_config* c, const mk_runtime_config* rt, int cus, int nsplit) {
    const size_t items = (size_t)rt->max_batch * c->n_kv_heads * nsplit;
    return (size_t)c->n_layers * (4 * (size_t)cus + items) + cus;
}

int device_cus() {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 256;
    return prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
}

int resolve_cus(const mk_runtime_config* rt) { return rt->num_cus > 0 ? rt->num_cus : device_cus(); }

}  // namespace

struct mk_handle {
    mk_model_config cfg;
    mk_runtime_config rt;
    Plan plan;
    Layout lo;
    Params P;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    void* kv = nullptr;
    size_t kv_bytes = 0;
    hipStream_t stream = nullptr;
    std::vector<int32_t> ctx;
    uint32_t epoch = 0;
    HostErr* host_err = nullptr;
    HostErr* host_err_dev = nullptr;
    bool latched = false;
    mk_status latched_status = MK_OK;
    std::string last_error;
    // graph mode
    hipGraphExec_t gexec = nullptr;
    hipGraph_t graph = nullptr;
    const void *g_in = nullptr, *g_out = nullptr, *g_logits = nullptr;
    int32_t inject = 0;
};

static mk_status hip_fail(mk_handle* h, hipError_t e, const char* what) {
    if (h) {
        h->last_error = std::string(what) + ": " + hipGetErrorString(e);
    }
    return MK_E_HIP;
}

#define HIPCHK(h, call)                                       \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return hip_fail((h), e_, #call); \
    } while (0)

extern "C" {

const char* mk_status_string(mk_status s) {
    switch (s) {
        case MK_OK: return "ok";
        case MK_E_INVALID: return "invalid argument";
        case MK_E_UNSUPPORTED: return "unsupported shape or option";
        case MK_E_CAPACITY: return "KV capacity exceeded";
        case MK_E_HIP: return "HIP runtime error";
        case MK_E_DEVICE_TIMEOUT: return "device spin-wait timed out";
        case MK_E_STATE: return "handle latched after a device error; call mk_reset";
        case MK_E_DEVICE_NAN: return "NaN in logits";
        default: return "unknown status";
    }
}

const char* mk_last_error(const mk_handle* h) { return h ? h->last_error.c_str() : "null handle"; }

mk_status mk_query_sizes(const mk_model_config* cfg, const mk_runtime_config* rt, size_t* workspace_bytes,
                         size_t* kv_bytes) {
    if (!workspace_bytes || !kv_bytes) return MK_E_INVALID;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    const int n_cu = rt->num_cus > 0 ? rt->num_cus : kMaxCus;
    int nsplit = 1;
    for (int cus = 1; cus <= n_cu; cus *= 2) nsplit = std::max(nsplit, auto_splits(cfg, rt, cus));
    nsplit = std::max(nsplit, auto_splits(cfg, rt, n_cu));
    const uint32_t n_ctr = (uint32_t)(cfg->n_layers * kPhasesPerLayer + 2);
    const uint32_t items = (uint32_t)(rt->max_batch * cfg->n_kv_heads * nsplit);
    const uint32_t fstride = (std::max((uint32_t)n_cu, items) + 63u) & ~63u;
    Layout lo = layout(cfg, rt, n_cu, nsplit, max_instrs(cfg, rt, n_cu, nsplit), n_ctr, fstride);
    *workspace_bytes = lo.total;
    *kv_bytes = 2ull * cfg->n_layers * rt->max_batch * cfg->n_kv_heads * (size_t)rt->max_seq * cfg->head_dim * 2;
    return MK_OK;
}

mk_status mk_plan_inspect(const mk_model_config* cfg, const mk_runtime_config* rt, int32_t num_cus, int64_t* out,
                          int32_t cap) {
    if (!out || cap < 0) return MK_E_INVALID;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    if (num_cus <= 0 || num_cus > kMaxCus) return MK_E_INVALID;
    if ((uint32_t)cfg->vocab < (uint32_t)num_cus) return MK_E_UNSUPPORTED;
    Plan pl = build_plan(cfg, rt, num_cus);
    const int64_t d = cfg->hidden, hd = cfg->head_dim;
    const int64_t per_layer = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * hd * d + d * cfg->n_q_heads * hd +
                              3 * (int64_t)cfg->ffn * d + 2 * d;
    int64_t vals[8] = {num_cus, (int64_t)pl.instrs.size(), pl.n_ctr, (int64_t)pl.max_per_cu,
                       2 * (cfg->n_layers * per_layer + (int64_t)cfg->vocab * d + d), verify_plan(cfg, rt, pl),
                       pl.nsplit, pl.phases};
    for (int i = 0; i < cap && i < 8; ++i) out[i] = vals[i];
    return MK_OK;
}

mk_status mk_create(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt, void* d_workspace,
                    size_t workspace_bytes, void* d_kv, size_t kv_bytes, void* stream, mk_handle** out) {
    if (!out) return MK_E_INVALID;
    *out = nullptr;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    if (!w || !w->tok_embedding || !w->final_norm || !w->layers || !d_workspace || !d_kv) return MK_E_INVALID;
    for (int l = 0; l < cfg->n_layers; ++l) {
        const mk_layer_weights& Lw = w->layers[l];
        if (!Lw.attn_norm || !Lw.wq || !Lw.wk || !Lw.wv || !Lw.wo || !Lw.mlp_norm || !Lw.w_gate || !Lw.w_up ||
            !Lw.w_down)
            return MK_E_INVALID;
    }
    if (!cfg->tied_embeddings && !w->lm_head) return MK_E_INVALID;
    size_t need_ws = 0, need_kv = 0;
    s = mk_query_sizes(cfg, rt, &need_ws, &need_kv);
    if (s != MK_OK) return s;
    mk_handle* h = new (std::nothrow) mk_handle();
    if (!h) return MK_E_INVALID;
    h->cfg = *cfg;
    h->rt = *rt;
    h->stream = (hipStream_t)stream;
    const int n_cu = resolve_cus(rt);
    if (n_cu <= 0 || n_cu > kMaxCus || (uint32_t)cfg->vocab < (uint32_t)n_cu) {
        delete h;
        return MK_E_UNSUPPORTED;
    }
    h->plan = build_plan(cfg, rt, n_cu);
    const int vr = verify_plan(cfg, rt, h->plan);
    if (vr != 0) {
        delete h;
        return MK_E_INVALID;
    }
    h->lo = layout(cfg, rt, n_cu, h->plan.nsplit, h->plan.instrs.size(), h->plan.n_ctr, h->plan.flag_stride);
    if (workspace_bytes < h->lo.total || workspace_bytes < need_ws || kv_bytes < need_kv) {
        delete h;
        return MK_E_INVALID;
    }
    h->ws = (char*)d_workspace;
    h->ws_bytes = workspace_bytes;
    h->kv = d_kv;
    h->kv_bytes = kv_bytes;
    h->ctx.assign(rt->max_batch, 0);

    // pinned, device-visible error word
    if (hipHostMalloc((void**)&h->host_err, sizeof(HostErr), hipHostMallocMapped | hipHostMallocCoherent) !=
        hipSuccess) {
        h->host_err = nullptr;
    } else {
        std::memset(h->host_err, 0, sizeof(HostErr));
        if (hipHostGetDevicePointer((void**)&h->host_err_dev, h->host_err, 0) != hipSuccess) h->host_err_dev = nullptr;
    }

    // ---- parameters
    Params& P = h->P;
    std::memset(&P, 0, sizeof(P));
    P.L = cfg->n_layers;
    P.d = cfg->hidden;
    P.Hq = cfg->n_q_heads;
    P.Hkv = cfg->n_kv_heads;
    P.hd = cfg->head_dim;
    P.F = cfg->ffn;
    P.V = cfg->vocab;
    P.B = rt->max_batch;
    P.S = rt->max_seq;
    P.G = cfg->n_q_heads / cfg->n_kv_heads;
    P.qkv_rows = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
    P.nsplit = h->plan.nsplit;
    P.n_cu = n_cu;
    P.kv_b = rt->max_batch;
    P.eps = cfg->rms_eps;
    P.attn_scale = (float)(1.0 / std::sqrt((double)cfg->head_dim));
    char* ws = h->ws;
    const Layout& lo = h->lo;
    P.layers = (const DevLayer*)(ws + lo.layers);
    P.embed = (const uint16_t*)w->tok_embedding;
    P.head = (const uint16_t*)(cfg->tied_embeddings || !w->lm_head ? w->tok_embedding : w->lm_head);
    P.final_norm = (const uint16_t*)w->final_norm;
    const size_t kv_half = (size_t)cfg->n_layers * rt->max_batch * cfg->n_kv_heads * (size_t)rt->max_seq *
                           cfg->head_dim;
    P.kcache = (uint16_t*)d_kv;
    P.vcache = (uint16_t*)d_kv + kv_half;
    P.rope = (const float2*)(ws + lo.rope);
    P.h = (float*)(ws + lo.h);
    P.qkv = (float*)(ws + lo.qkv);
    P.attn = (float*)(ws + lo.attn);
    P.act = (float*)(ws + lo.act);
    P.attn_part = (float*)(ws + lo.attn_part);
    P.attn_ticket = (uint32_t*)(ws + lo.tickets);
    P.head_part = (HeadPart*)(ws + lo.head_part);
    P.counters = (uint32_t*)(ws + lo.counters);
    P.flags = (uint32_t*)(ws + lo.flags);
    P.flag_stride = h->plan.flag_stride;
    P.state = (DevState*)(ws + lo.state);
    P.host_err = h->host_err_dev;
    P.instrs = (const Instr*)(ws + lo.instrs);
    P.queue_off = (const uint32_t*)(ws + lo.qoff);
    P.head_ctr = h->plan.head_ctr;
    P.n_head_instr = h->plan.n_head;
    if (rt->trace) {
        P.trace = (uint32_t*)(ws + lo.trace);
        P.trace_stride = (uint32_t)(lo.trace_bytes / ((size_t)n_cu * kTraceWords * 4));
        if (h->plan.max_per_cu > P.trace_stride) {
            delete h;
            return MK_E_INVALID;
        }
    }
    const uint32_t tmo = rt->spin_timeout_ms ? rt->spin_timeout_ms : 2000u;
    P.spin_ticks = (uint64_t)tmo * 100000ull;

    // ---- uploads (synchronous; create is not on the hot path)
    std::vector<DevLayer> dl(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; ++l) {
        const mk_layer_weights& Lw = w->layers[l];
        dl[l] = DevLayer{(const uint16_t*)Lw.attn_norm, (const uint16_t*)Lw.wq,     (const uint16_t*)Lw.wk,
                         (const uint16_t*)Lw.wv,        (const uint16_t*)Lw.wo,     (const uint16_t*)Lw.mlp_norm,
                         (const uint16_t*)Lw.w_gate,    (const uint16_t*)Lw.w_up,   (const uint16_t*)Lw.w_down};
    }
    // RoPE table: angle p * theta^(-2i/hd) in double, cos/sin rounded to fp32
    std::vector<float> rope((size_t)rt->max_seq * cfg->head_dim);
    const int half = cfg->head_dim / 2;
    for (int p = 0; p < rt->max_seq; ++p)
        for (int i = 0; i < half; ++i) {
            const double inv = std::pow(cfg->rope_theta, -2.0 * i / (double)cfg->head_dim);
            const double a = (double)p * inv;
            rope[((size_t)p * half + i) * 2 + 0] = (float)std::cos(a);
            rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
        }
    std::vector<HeadPart> hp(lo.head_slots * rt->max_batch, HeadPart{-INFINITY, 0x7FFFFFFF});
    hipError_t e = hipSuccess;
    auto cp = [&](size_t off, const void* src, size_t bytes) {
        if (e == hipSuccess && bytes) e = hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, h->stream);
    };
    if (e == hipSuccess) e = hipMemsetAsync(ws, 0, lo.total, h->stream);
    cp(lo.instrs, h->plan.instrs.data(), h->plan.instrs.size() * sizeof(Instr));
    cp(lo.qoff, h->plan.qoff.data(), h->plan.qoff.size() * 4);
    cp(lo.layers, dl.data(), dl.size() * sizeof(DevLayer));
    cp(lo.rope, rope.data(), rope.size() * 4);
    cp(lo.head_part, hp.data(), hp.size() * sizeof(HeadPart));
    if (e == hipSuccess) e = hipMemsetAsync(d_kv, 0, need_kv, h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) {
        mk_status st = hip_fail(h, e, "mk_create upload");
        if (h->host_err) (void)hipHostFree(h->host_err);
        delete h;
        return st;
    }
    *out = h;
    return MK_OK;
}

mk_status mk_kv_layout(const mk_handle* h, int64_t strides_out[5]) {
    if (!h || !strides_out) return MK_E_INVALID;
    const int64_t hd = h->cfg.head_dim, S = h->rt.max_seq, Hkv = h->cfg.n_kv_heads, B = h->rt.max_batch;
    strides_out[4] = 1;
    strides_out[3] = hd;
    strides_out[2] = S * hd;
    strides_out[1] = Hkv * S * hd;
    strides_out[0] = B * Hkv * S * hd;
    return MK_OK;
}

static mk_status check_latched(mk_handle* h) {
    if (h->latched) return MK_E_STATE;
    if (h->host_err) {
        const uint32_t code = __atomic_load_n(&h->host_err->code, __ATOMIC_ACQUIRE);
        if (code != 0) {
            h->latched = true;
            h->latched_status = code == DERR_NAN ? MK_E_DEVICE_NAN : MK_E_DEVICE_TIMEOUT;
            char buf[160];
            std::snprintf(buf, sizeof(buf), "device error %u (info %u %u, workgroup %u)", code, h->host_err->info[0],
                          h->host_err->info[1], h->host_err->info[2]);
            h->last_error = buf;
            return h->latched_status;
        }
    }
    return MK_OK;
}

static mk_status run_step(mk_handle* h, const int32_t* tok_in, int32_t stride, int32_t* tok_out, float* logits,
                          hipStream_t st) {
    for (int b = 0; b < h->rt.max_batch; ++b)
        if (h->ctx[b] + 1 > h->rt.max_seq) return MK_E_CAPACITY;
    StepArgs A;
    std::memset(&A, 0, sizeof(A));
    A.tok_in = tok_in;
    A.tok_stride = stride;
    A.tok_out = tok_out;
    A.logits = logits;
    A.epoch = ++h->epoch;
    Params P = h->P;
    if (h->inject == 1) {
        P.spin_ticks = 100000ull;  // 1 ms
        // the first QKV instruction of layer 0 waits for nothing; make the ATTN phase
        // of layer 0 wait for twice as many producers as exist
        std::vector<Instr> bad = h->plan.instrs;
        for (Instr& in : bad)
            if (in.op == OP_ATTN && in.layer == 0) in.wait_n *= 2;
        HIPCHK(h, hipMemcpyAsync(h->ws + h->lo.instrs, bad.data(), bad.size() * sizeof(Instr), hipMemcpyHostToDevice,
                                 st));
        HIPCHK(h, hipStreamSynchronize(st));
        h->inject = 2;  // restore after this step
    }
    if (h->rt.mode == MK_MODE_MEGAKERNEL) {
        HIPCHK(h, launch_megakernel(P, A, st));
    } else {
        // replay a graph captured for these pointers (re-captured when they change)
        if (!h->gexec || h->g_in != tok_in || h->g_out != tok_out || h->g_logits != logits || stride != 1) {
            if (stride != 1) {
                HIPCHK(h, launch_conventional(P, A, (uint32_t*)(h->ws + h->lo.counters) +
                                                        (size_t)h->plan.conv_ticket_ctr * kCtrStride,
                                              st));
                goto done;
            }
            if (h->gexec) {
                (void)hipGraphExecDestroy(h->gexec);
                h->gexec = nullptr;
            }
            if (h->graph) {
                (void)hipGraphDestroy(h->graph);
                h->graph = nullptr;
            }
            hipStream_t cap;
            HIPCHK(h, hipStreamCreateWithFlags(&cap, hipStreamNonBlocking));
            hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
            if (e == hipSuccess)
                e = launch_conventional(P, A, (uint32_t*)(h->ws + h->lo.counters) + (size_t)h->plan.conv_ticket_ctr *
                                                                                          kCtrStride,
                                        cap);
            hipGraph_t g = nullptr;
            hipError_t e2 = hipStreamEndCapture(cap, &g);
            (void)hipStreamDestroy(cap);
            if (e != hipSuccess) return hip_fail(h, e, "capture");
            if (e2 != hipSuccess) return hip_fail(h, e2, "end capture");
            h->graph = g;
            HIPCHK(h, hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0));
            h->g_in = tok_in;
            h->g_out = tok_out;
            h->g_logits = logits;
        }
        HIPCHK(h, hipGraphLaunch(h->gexec, st));
    }
done:
    for (int b = 0; b < h->rt.max_batch; ++b) h->ctx[b] += 1;
    if (h->inject == 2) {
        HIPCHK(h, hipStreamSynchronize(st));
        HIPCHK(h, hipMemcpyAsync(h->ws + h->lo.instrs, h->plan.instrs.data(), h->plan.instrs.size() * sizeof(Instr),
                                 hipMemcpyHostToDevice, st));
        HIPCHK(h, hipStreamSynchronize(st));
        h->inject = 0;
    }
    return MK_OK;
}

mk_status mk_decode_step(mk_handle* h, const int32_t* d_tokens_in, int32_t B, int32_t* d_tokens_out, float* d_logits,
                         void* stream) {
    if (!h || !d_tokens_in || !d_tokens_out || !d_logits) return MK_E_INVALID;
    if (B != h->rt.max_batch) return MK_E_INVALID;
    mk_status s = check_latched(h);
    if (s != MK_OK) return s;
    return run_step(h, d_tokens_in, 1, d_tokens_out, d_logits, (hipStream_t)stream);
}

mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P, float* d_logits, int32_t* d_next,
                     void* stream) {
    if (!h || !d_tokens || !d_logits || !d_next || P <= 0) return MK_E_INVALID;
    if (B != h->rt.max_batch) return MK_E_INVALID;
    mk_status s = check_latched(h);
    if (s != MK_OK) return s;
    for (int b = 0; b < B; ++b)
        if (h->ctx[b] + P > h->rt.max_seq) return MK_E_CAPACITY;
    float* scr_logits = (float*)(h->ws + h->lo.logits_scr);
    int32_t* scr_tok = (int32_t*)(h->ws + h->lo.tok_scr);
    for (int t = 0; t < P; ++t) {
        const bool last = t == P - 1;
        s = run_step(h, d_tokens + t, P, last ? d_next : scr_tok, last ? d_logits : scr_logits, (hipStream_t)stream);
        if (s != MK_OK) return s;
    }
    return MK_OK;
}

mk_status mk_set_context_len(mk_handle* h, const int32_t* h_lens, int32_t B) {
    if (!h || !h_lens || B != h->rt.max_batch) return MK_E_INVALID;
    for (int b = 0; b < B; ++b)
        if (h_lens[b] < 0 || h_lens[b] > h->rt.max_seq) return MK_E_CAPACITY;
    for (int b = 0; b < B; ++b) h->ctx[b] = h_lens[b];
    HIPCHK(h, hipMemcpyAsync(h->ws + h->lo.state + offsetof(DevState, ctx_len), h->ctx.data(), B * sizeof(int32_t),
                             hipMemcpyHostToDevice, h->stream));
    HIPCHK(h, hipStreamSynchronize(h->stream));
    return MK_OK;
}

mk_status mk_get_context_len(const mk_handle* h, int32_t* h_lens, int32_t B) {
    if (!h || !h_lens || B != h->rt.max_batch) return MK_E_INVALID;
    for (int b = 0; b < B; ++b) h_lens[b] = h->ctx[b];
    return MK_OK;
}

mk_status mk_reset(mk_handle* h, void* stream) {
    if (!h) return MK_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    HIPCHK(h, hipStreamSynchronize(st));
    DevState ds;
    HIPCHK(h, hipMemcpy(&ds, h->ws + h->lo.state, sizeof(ds), hipMemcpyDeviceToHost));
    for (int b = 0; b < h->rt.max_batch; ++b) h->ctx[b] = ds.ctx_len[b];
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.counters, 0, (size_t)h->plan.n_ctr * kCtrStride * 4, st));
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.flags, 0, h->lo.flags_bytes, st));
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.tickets, 0,
                             (size_t)h->cfg.n_layers * h->rt.max_batch * h->cfg.n_kv_heads * kCtrStride * 4, st));
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.state + offsetof(DevState, error), 0, 16, st));
    HIPCHK(h, hipStreamSynchronize(st));
    if (h->host_err) std::memset(h->host_err, 0, sizeof(HostErr));
    h->epoch = 0;
    h->latched = false;
    h->latched_status = MK_OK;
    h->last_error.clear();
    return MK_OK;
}

mk_status mk_debug_inject(mk_handle* h, int32_t fault, int32_t arg) {
    (void)arg;
    if (!h) return MK_E_INVALID;
    if (fault != 0 && fault != 1) return MK_E_INVALID;
    if (fault == 1 && h->rt.mode != MK_MODE_MEGAKERNEL) return MK_E_UNSUPPORTED;
    h->inject = fault;
    return MK_OK;
}

mk_status mk_read_trace(mk_handle* h, void* h_buf, size_t bytes, size_t* written, int32_t* records_per_cu) {
    if (!h || !written || !records_per_cu) return MK_E_INVALID;
    *written = 0;
    *records_per_cu = (int32_t)h->P.trace_stride;
    if (!h->rt.trace) return MK_E_UNSUPPORTED;
    if (!h_buf) {
        *written = h->lo.trace_bytes;
        return MK_OK;
    }
    const size_t n = std::min(bytes, h->lo.trace_bytes);
    HIPCHK(h, hipStreamSynchronize(h->stream));
    HIPCHK(h, hipMemcpy(h_buf, h->ws + h->lo.trace, n, hipMemcpyDeviceToHost));
    *written = n;
    return MK_OK;
}

int32_t mk_kernels_per_step(const mk_handle* h) {
    if (!h) return -1;
    return h->rt.mode == MK_MODE_MEGAKERNEL ? 1 : conventional_kernels_per_step(h->P);
}

mk_status mk_destroy(mk_handle* h) {
    if (!h) return MK_E_INVALID;
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    if (h->graph) (void)hipGraphDestroy(h->graph);
    if (h->host_err) (void)hipHostFree(h->host_err);
    delete h;
    return MK_OK;
}

}  // extern "C"
