// Host runtime behind include/mk.h: validation, workspace layout, the static
// scheduler that fills per-CU instruction queues and its verifier, the RoPE
// table, and the launch of one decode step in either mode.
//
// Scheduling follows the page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞",
// section "Megakernel：从零设计的深度融合方案": before launch every compute unit gets
// an ordered plan of composite instructions and each dependency is fixed
// statically as (producer phase, value tag): an instruction reads the values
// of an earlier phase only once each one carries its phase's tag for this step;
// nothing is decided at run time.
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
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {
hipError_t launch_megakernel(const Params& P, const StepArgs& A, hipStream_t stream);
hipError_t prepare_megakernel(const Params& P);
bool megakernel_supports(int B, int hd);
size_t megakernel_lds_bytes(const Params& P);
hipError_t launch_conventional(const Params& P, const StepArgs& A, hipStream_t stream);
hipError_t prepare_conventional(const Params& P);
hipError_t transpose_bf16(uint16_t* dst, const uint16_t* src, int rows, int cols, hipStream_t stream);
int conventional_kernels_per_step(const Params& P);
int conventional_head_blocks(const Params& P);
}  // namespace mk

using namespace mk;

namespace {

constexpr int kMaxCus = 1024;
constexpr int kMaxSplits = 64;

struct Plan {
    std::vector<Instr> instrs;
    std::vector<uint32_t> qoff;  // [n_cu + 1]
    uint32_t n_head = 0;         // LM-head instructions
    int n_cu = 0, nsplit = 1;
    int phases = 0;
    size_t max_per_cu = 0;
    int hsplit = 1;
};

uint32_t ring_chunks_for(size_t x_bytes) {
    const size_t avail = kLdsBytes - kStaticLds;
    return x_bytes >= avail ? 0u : (uint32_t)((avail - x_bytes) / kChunk);
}

size_t x_floats_kind(const mk_model_config* c, const mk_runtime_config* rt, int nsplit, bool mfma, int nnew = 1);

// Row lengths of the matrix-core instructions are whole tile units.
bool mfma_shapes_ok(const mk_model_config* c, int B) {
    return c->hidden % kMfmaUnitCols == 0 && (c->n_q_heads * c->head_dim) % kMfmaUnitCols == 0 &&
           down_slices_for(B, c->ffn, true) != 0;
}

// Smallest batch at which automatic selection takes the matrix cores (measured:
// VALU is faster at every supported batch, so automatic selection never does).
constexpr int kMfmaAutoMinBatch = kMaxBatch + 1;

// GEMV kind of a runtime configuration: the matrix cores run in the megakernel
// only; automatic selection takes them from kMfmaAutoMinBatch on where their
// activation area (bf16 parts: 6 bytes per element at 3 parts) leaves the weight
// ring room.
bool use_mfma(const mk_model_config* c, const mk_runtime_config* rt) {
    if (rt->mode != MK_MODE_MEGAKERNEL) return false;
    if (rt->gemv_kind == 1) return false;
    if (rt->gemv_kind == 2) return true;
    if (c->n_experts) return false;
    if (rt->max_batch < kMfmaAutoMinBatch || !mfma_shapes_ok(c, rt->max_batch)) return false;
    return ring_chunks_for((x_floats_kind(c, rt, 1, true) * 4 + 15) & ~(size_t)15) >= kMinRingChunks;
}

// The dense down projection split by columns (OP_DPART per part of kDownPart
// SwiGLU outputs, then OP_DRED per output row): each CU stages only its parts'
// inputs, not the whole B x F activation, at the cost of a transposed copy of
// Wdown in the workspace and a second, smaller all-to-all (the parts' partials).
// Automatic from batch 4, where staging B x F tagged words per CU dominates DOWN.
bool down_split_on(const mk_model_config* c, const mk_runtime_config* rt) {
    if (c->n_experts || rt->down_split < 0) return false;
    if (c->hidden > kDownSplitMaxHidden || c->ffn % (int)kDownPart || use_mfma(c, rt)) return false;
    return rt->down_split > 0 || rt->max_batch >= 4;
}

// DOWN by column quarters (batch 1, F = 8192, VALU, not split by columns).
bool down_q_on(const mk_model_config* c, const mk_runtime_config* rt) {
    return !c->n_experts && down_quarters_for(rt->max_batch, c->ffn) && !use_mfma(c, rt) && !down_split_on(c, rt);
}

// (gate, up) rows computed by the loader waves from registers (batch 1, dense, VALU,
// hidden 2048 with head_dim 64 or 4096 with head_dim 128).
bool gu_direct_on(const mk_model_config* c, const mk_runtime_config* rt) {
    return rt->max_batch == 1 && !c->n_experts && !use_mfma(c, rt) && (c->head_dim == 64 || c->head_dim == 128) &&
           c->hidden == 512 * gu_npl(c->head_dim);
}

// O rows computed by the loader waves (as gu_direct_on, hidden 4096 only).
bool o_direct_on(const mk_model_config* c, const mk_runtime_config* rt) {
    return gu_direct_on(c, rt) && c->head_dim == 128 && c->n_q_heads * c->head_dim == c->hidden;
}

uint32_t dred_rows_for(const mk_model_config* c) { return dred_rows((uint32_t)c->hidden, (uint32_t)c->ffn); }

// LDS floats of activations one instruction stages (x rows, residual rows of
// O / DOWN, or an attention item's area).
size_t x_floats_kind(const mk_model_config* c, const mk_runtime_config* rt, int nsplit, bool mfma, int nnew) {
    const size_t B = (size_t)rt->max_batch, hd = (size_t)c->head_dim, G = (size_t)(c->n_q_heads / c->n_kv_heads);
    if (mfma) {
        // bf16 parts of the input (one column slice for DOWN), the residual rows and
        // partial sums of O / DOWN, and the cross-wave partial tiles at the end
        const int b = (int)B;
        const int ns = std::max(1, down_slices_for(b, c->ffn, true));
        const size_t resid = 2 * B * kMaxResidRows * 4;
        size_t bytes = parts_bytes(b, c->hidden);
        bytes = std::max(bytes, parts_bytes(b, c->n_q_heads * c->head_dim) + resid);
        bytes = std::max(bytes, parts_bytes(b, c->ffn / ns) + resid);
        bytes += mfma_red_bytes(b);
        return std::max((bytes + 3) / 4, attn_lds_floats((int)G, (int)hd, nsplit, nnew));
    }
    const int xsl = std::max(1, x_slices_for((int)B, c->hidden, c->n_q_heads * c->head_dim, c->n_experts > 0));
    const size_t dw = (size_t)c->hidden / xsl, ow = (size_t)c->n_q_heads * hd / xsl;
    // QKV / router: one input slice (and, sliced, the partial sums of at most
    // kMaxResidRows rows); O: one input slice, the residual rows (and partial sums)
    size_t n = B * (dw + (xsl > 1 ? kMaxResidRows : 0));
    n = std::max(n, B * (ow + (xsl > 1 ? 2 : 1) * kMaxResidRows));
    if (c->n_experts > 0) {
        // EGU: x rows (one slice) and the router logits, and sliced the partial sums
        // of every selected slot's rows; EPART: the router logits and one slot's
        // SwiGLU rows; EDOWN: the router logits, the slots' weights, the residual rows
        // and every slot's outputs of its rows
        const size_t E = (size_t)c->n_experts;
        const size_t slots = (size_t)c->n_shared_experts + std::min(E, B * (size_t)c->top_k);
        n = std::max(n, B * (dw + E) + (xsl > 1 ? slots * 2 * kMaxEguSlicedRows * B : 0));
        n = std::max(n, B * ((size_t)c->expert_ffn + E));
        n = std::max(n, B * E + (slots + 1) * B + B * kMaxEredRows + slots * B * kMaxEredRows);
        return std::max(n, attn_lds_floats((int)G, (int)hd, nsplit, nnew));
    }
    if (down_split_on(c, rt)) {
        // DPART: the inputs of its parts and one part's outputs; DRED: the residual
        // rows and every part's partials of its rows
        const size_t np = (size_t)c->ffn / kDownPart, rows = dred_rows_for(c);
        n = std::max(n, B * (kMaxDpartParts * kDownPart + (size_t)c->hidden));
        n = std::max(n, B * rows * (np + 1));
        return std::max(n, attn_lds_floats((int)G, (int)hd, nsplit, nnew));
    }
    // DOWN: one column slice of the input, the residual rows and the partial sums
    // (by column quarters: the input, the residual rows and four values per row)
    const int ns = std::max(1, down_slices_for((int)B, c->ffn));
    n = std::max(n, B * ((size_t)(c->ffn / ns) + (down_q_on(c, rt) ? 5 : 2) * kMaxResidRows));
    return std::max(n, attn_lds_floats((int)G, (int)hd, nsplit, nnew));
}

// nnew: new positions one attention item holds (kChunkRows for a multi-position plan)
size_t x_bytes_for(const mk_model_config* c, const mk_runtime_config* rt, int nsplit, int nnew = 1) {
    return (x_floats_kind(c, rt, nsplit, use_mfma(c, rt), nnew) * 4 + 15) & ~(size_t)15;
}

// Most KV splits whose merge area still leaves the minimum weight ring (0: none).
int max_splits_lds(const mk_model_config* c, const mk_runtime_config* rt) {
    int best = 0;
    for (int n = 1; n <= kMaxSplits; ++n)
        if (ring_chunks_for(x_bytes_for(c, rt, n)) >= kMinRingChunks) best = n;
    return best;
}

// KV splits per (sequence, KV head): about 512 positions per split, at most one
// item per compute unit.  Short contexts get one split and no merge.
int auto_splits(const mk_model_config* c, const mk_runtime_config* rt, int n_cu) {
    if (rt->attn_splits > 0) return rt->attn_splits;
    const int pairs = std::max(1, rt->max_batch * c->n_kv_heads);
    const int by_cu = std::max(1, n_cu / pairs);
    const int by_len = std::max(1, (rt->max_seq + 511) / 512);
    return std::max(1, std::min(std::min(by_cu, by_len), std::min(kMaxSplits, max_splits_lds(c, rt))));
}

// q-head groups per attention item: with one position split and no more items
// than compute units, every q head of a KV head becomes an item of its own (the
// K/V of the group is streamed once per item; the append is done by head 0's).
int auto_hsplit(const mk_model_config* c, const mk_runtime_config* rt, int n_cu, int nsplit) {
    const int G = c->n_q_heads / c->n_kv_heads;
    if (rt->mode != MK_MODE_MEGAKERNEL || nsplit != 1 || G < 1) return 1;
    return (int64_t)rt->max_batch * c->n_kv_heads * G <= n_cu ? G : 1;
}

// The loader writes stream chunk c into ring slot c mod N only once every compute
// wave's mark (the first chunk it still needs) is above c - N.  A wave that waits
// for a row batch keeps its mark at the batch start, so one batch must fit the
// ring; and waves never hold a mark across a barrier inside an instruction (they
// move it to a region's end when they leave a GEMV region), so the slowest wave
// can always be served and no wait can close a cycle.  The stretch one wave
// holds, by instruction kind:
//  - a VALU row batch: ring_batch_rows rows (8 KB segments of long rows at batch
//    1 and 2), plus one chunk because packed rows may start inside a chunk;
//  - a matrix-core unit (16 rows x kMfmaUnitCols columns): 16 / kMfmaChunkRows chunks;
//  - an attention block: its RoPE chunk and kAttnBlockGroups groups of a K and a
//    V chunk (a long split goes in half blocks, a wave at most one half block ahead).
// Returns the largest of these for the configuration (chunks).
uint32_t max_wave_span(const mk_model_config* c, const mk_runtime_config* rt) {
    const int B = rt->max_batch;
    uint32_t span = 1u + 2u * (uint32_t)kAttnBlockGroups;
    if (use_mfma(c, rt)) return std::max(span, 16u / (uint32_t)kMfmaChunkRows);
    auto gemv = [&](uint32_t rb, bool pairs) { span = std::max(span, ring_batch_span(rb, B, pairs)); };
    const uint32_t xsl = (uint32_t)std::max(1, x_slices_for(B, c->hidden, c->n_q_heads * c->head_dim,
                                                            c->n_experts > 0));
    const uint32_t d2 = (uint32_t)c->hidden * 2u / xsl;             // one input slice
    gemv(d2, false);                                                // QKV, MoE router
    gemv((uint32_t)c->hidden * 2u, false);                          // LM head (streamed, never sliced)
    gemv((uint32_t)(c->n_q_heads * c->head_dim) * 2u / xsl, false); // O
    if (c->n_experts) {
        gemv(d2, true);                                             // expert (gate, up) pairs
        gemv((uint32_t)c->expert_ffn * 2u, false);                  // expert DOWN
    } else {
        gemv(d2, true);                                             // (gate, up) pairs
        if (down_split_on(c, rt)) {
            // a DPART wave waits for kDpartRowsPerGet transposed rows at a time
            span = std::max(span, ((uint32_t)kDpartRowsPerGet * (uint32_t)c->hidden * 2u + kChunk - 1u) / kChunk + 1u);
        } else {
            const int ns = std::max(1, down_slices_for(B, c->ffn));
            gemv((uint32_t)(c->ffn / ns) * 2u, false);              // DOWN column slice
        }
    }
    return span;
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
    const bool moe = c->n_experts != 0;
    if (moe) {
        if (c->n_experts < 0 || c->top_k <= 0 || c->top_k > c->n_experts || c->expert_ffn <= 0 ||
            c->n_shared_experts < 0)
            return fail(MK_E_INVALID, "MoE: need 0 < top_k <= n_experts, expert_ffn > 0, n_shared >= 0");
        if (c->n_experts > kMaxExperts || c->top_k > kMaxTopK || c->n_shared_experts > 1)
            return fail(MK_E_UNSUPPORTED, "MoE: at most 64 experts, top_k <= 8 and one shared expert");
        if (c->expert_ffn % 512 || c->hidden % 512 || ((c->hidden / 512) & (c->hidden / 512 - 1)))
            return fail(MK_E_UNSUPPORTED, "MoE: expert rows must be whole 1 KB chunks (power-of-two per hidden row)");
        if (rt->mode != MK_MODE_MEGAKERNEL) return fail(MK_E_UNSUPPORTED, "MoE runs in the persistent mode only");
        if (rt->gemv_kind == 2) return fail(MK_E_UNSUPPORTED, "MoE runs on the VALU GEMV");
    } else if (c->ffn <= 0) {
        return fail(MK_E_INVALID, "ffn must be positive");
    }
    if (c->head_dim != 64 && c->head_dim != 128) return fail(MK_E_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->n_q_heads % c->n_kv_heads) return fail(MK_E_UNSUPPORTED, "n_q_heads must be a multiple of n_kv_heads");
    if (c->n_q_heads / c->n_kv_heads > kMaxGroup) return fail(MK_E_UNSUPPORTED, "more than 4 q heads per KV head");
    if (c->hidden % 256 || (!moe && c->ffn % 64)) return fail(MK_E_UNSUPPORTED, "hidden % 256 and ffn % 64 must be 0");
    if (c->n_q_heads * c->head_dim > 16384) return fail(MK_E_UNSUPPORTED, "attention width above 16384");
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.0)) return fail(MK_E_INVALID, "rms_eps and rope_theta must be > 0");
    if (rt->max_batch < 1 || rt->max_batch > kMaxBatch) return fail(MK_E_UNSUPPORTED, "max_batch must be 1..8");
    if (!megakernel_supports(rt->max_batch, c->head_dim))
        return fail(MK_E_UNSUPPORTED, "this build runs batch 1, 2, 4 and 8");
    if (moe) {
        // hidden 4096 at batch 8: the hidden-wide inputs go in column slices, and the
        // LM-head input is staged over the (then idle) weight ring
        if (x_slices_for(rt->max_batch, c->hidden, c->n_q_heads * c->head_dim, true) == 0)
            return fail(MK_E_UNSUPPORTED, "MoE: the inputs of this batch need column slices of whole 1 KB chunks");
        if ((size_t)rt->max_batch * c->hidden * 4 > kLdsBytes - kStaticLds)
            return fail(MK_E_UNSUPPORTED, "the LM-head input of this batch exceeds the LDS");
    }
    if (rt->gemv_kind < 0 || rt->gemv_kind > 2) return fail(MK_E_UNSUPPORTED, "gemv_kind must be 0, 1 or 2");
    if (rt->gemv_kind == 2 && rt->mode != MK_MODE_MEGAKERNEL)
        return fail(MK_E_UNSUPPORTED, "the matrix-core GEMV runs in the megakernel only");
    if (rt->gemv_kind == 2 && !mfma_shapes_ok(c, rt->max_batch))
        return fail(MK_E_UNSUPPORTED, "matrix-core GEMV rows must be whole tile units of columns");
    if (!moe && down_slices_for(rt->max_batch, c->ffn, use_mfma(c, rt)) == 0)
        return fail(MK_E_UNSUPPORTED, "the DOWN input of this batch needs column slices of whole 1 KB chunks");
    if (rt->max_seq < 1 || rt->max_seq > (1 << 20)) return fail(MK_E_INVALID, "max_seq out of range");
    if (rt->mode != MK_MODE_MEGAKERNEL && rt->mode != MK_MODE_GRAPH) return fail(MK_E_INVALID, "unknown mode");
    if (rt->num_cus < 0 || rt->num_cus > kMaxCus) return fail(MK_E_INVALID, "num_cus out of range");
    if (rt->trace != 0 && rt->trace != 1) return fail(MK_E_INVALID, "trace must be 0 or 1");
    if (rt->attn_splits < 0 || rt->attn_splits > kMaxSplits) return fail(MK_E_INVALID, "attn_splits out of range");
    // the activations one instruction stages must leave room for the weight ring
    const int lds_splits = max_splits_lds(c, rt);
    if (lds_splits == 0) return fail(MK_E_UNSUPPORTED, "activations of one instruction exceed the LDS budget");
    if (rt->attn_splits > lds_splits) return fail(MK_E_UNSUPPORTED, "attention split merge exceeds the LDS budget");
    return MK_OK;
}

// Rows [c*R/n, (c+1)*R/n) for compute unit c.
inline void tile(uint32_t R, int n, int c, uint32_t* b, uint32_t* cnt) {
    const uint64_t lo = (uint64_t)R * c / n, hi = (uint64_t)R * (c + 1) / n;
    *b = (uint32_t)lo;
    *cnt = (uint32_t)(hi - lo);
}

// Every weight matrix is split by rows into one contiguous tile per compute unit;
// O and DOWN tiles are cut into instructions of at most kMaxResidRows rows (their
// residual rows are staged in LDS).  Attention items go round-robin, one per CU.
Plan build_plan(const mk_model_config* c, const mk_runtime_config* rt, int n_cu) {
    Plan pl;
    pl.n_cu = n_cu;
    pl.nsplit = auto_splits(c, rt, n_cu);
    pl.hsplit = auto_hsplit(c, rt, n_cu, pl.nsplit);
    const int L = c->n_layers, B = rt->max_batch;
    const uint32_t qkv_rows = (uint32_t)((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim);
    std::vector<std::vector<Instr>> q(n_cu);
    auto mk_instr = [](uint16_t op, int layer, uint32_t begin, uint32_t count) {
        Instr in;
        std::memset(&in, 0, sizeof(in));
        in.op = op;
        in.layer = (uint16_t)layer;
        in.begin = begin;
        in.count = count;
        return in;
    };
    auto gemv_phase = [&](uint16_t op, int layer, uint32_t R, uint32_t max_rows) {
        for (int cu = 0; cu < n_cu; ++cu) {
            uint32_t b, cnt;
            tile(R, n_cu, cu, &b, &cnt);
            for (uint32_t o = 0; o < cnt; o += max_rows) {
                Instr in = mk_instr(op, layer, b + o, std::min(max_rows, cnt - o));
                if (op == OP_HEAD) in.slot = pl.n_head++;
                q[cu].push_back(in);
            }
        }
        ++pl.phases;
    };
    const uint32_t all = 0xFFFFFFFFu;
    // sliced inputs: partial sums of every row of an instruction wait in LDS, so
    // instructions are cut to the rows that area holds
    const bool sliced = x_slices_for(B, c->hidden, c->n_q_heads * c->head_dim, c->n_experts > 0) > 1;
    for (int l = 0; l < L; ++l) {
        gemv_phase(OP_QKV, l, qkv_rows, sliced ? kMaxResidRows : all);
        const uint32_t items = (uint32_t)(B * c->n_kv_heads * pl.nsplit * pl.hsplit);
        for (uint32_t it = 0; it < items; ++it) q[it % n_cu].push_back(mk_instr(OP_ATTN, l, it, 1));
        ++pl.phases;
        gemv_phase(OP_O, l, (uint32_t)c->hidden, kMaxResidRows);
        if (c->n_experts) {
            // router rows; then on every CU its f-range of every selected expert; then
            // its share of the (selected expert, down row) pairs (begin: the CU); then
            // the weighted combine of its output rows
            gemv_phase(OP_ROUTE, l, (uint32_t)c->n_experts, sliced ? kMaxResidRows : all);
            gemv_phase(OP_EGU, l, (uint32_t)c->expert_ffn, sliced ? kMaxEguSlicedRows : all);
            for (int cu = 0; cu < n_cu; ++cu) q[cu].push_back(mk_instr(OP_EPART, l, (uint32_t)cu, 1));
            ++pl.phases;
            gemv_phase(OP_EDOWN, l, (uint32_t)c->hidden, kMaxEredRows);
        } else if (down_split_on(c, rt)) {
            // the F / kDownPart parts dealt like rows (a CU's parts are its GATEUP
            // f-range when F / n_cu is a multiple of kDownPart), then the row sums
            gemv_phase(OP_GATEUP, l, (uint32_t)c->ffn, all);
            gemv_phase(OP_DPART, l, (uint32_t)c->ffn / kDownPart, kMaxDpartParts);
            gemv_phase(OP_DRED, l, (uint32_t)c->hidden, dred_rows_for(c));
        } else {
            gemv_phase(OP_GATEUP, l, (uint32_t)c->ffn, all);
            gemv_phase(OP_DOWN, l, (uint32_t)c->hidden, kMaxResidRows);
        }
    }
    gemv_phase(OP_HEAD, L, (uint32_t)c->vocab, all);
    pl.qoff.resize(n_cu + 1);
    pl.qoff[0] = 0;
    for (int cu = 0; cu < n_cu; ++cu) {
        pl.qoff[cu + 1] = pl.qoff[cu] + (uint32_t)q[cu].size();
        pl.max_per_cu = std::max(pl.max_per_cu, q[cu].size());
        pl.instrs.insert(pl.instrs.end(), q[cu].begin(), q[cu].end());
    }
    return pl;
}

// Every row / item exactly once; each queue in non-decreasing phase order (an
// instruction only waits on values of earlier phases, so no queue can wait on
// itself or on a later queue position); O and DOWN instructions within the
// residual staging limit; LM-head slots 0..n_head-1 each once.  0 or an error code.
int verify_plan(const mk_model_config* c, const mk_runtime_config* rt, const Plan& pl) {
    const int L = c->n_layers, B = rt->max_batch;
    const uint32_t qkv_rows = (uint32_t)((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim);
    // sub-phases per layer: QKV, ATTN, O, ROUTE (MoE), GATEUP / EGU, EPART (MoE) / DPART (split DOWN),
    // DOWN / EDOWN / DRED
    constexpr int kSub = 7;
    const bool moe = c->n_experts != 0;
    const bool split = down_split_on(c, rt);
    const bool sliced = x_slices_for(B, c->hidden, c->n_q_heads * c->head_dim, moe) > 1;
    const int nphase = L * kSub + 1;
    std::vector<std::vector<uint8_t>> seen(nphase);
    auto phase_of = [&](const Instr& in) -> int {
        if (in.op == OP_HEAD) return L * kSub;
        const int k = in.op == OP_QKV ? 0 : in.op == OP_ATTN ? 1 : in.op == OP_O ? 2 : in.op == OP_ROUTE ? 3
                    : (in.op == OP_GATEUP || in.op == OP_EGU) ? 4 : (in.op == OP_EPART || in.op == OP_DPART) ? 5 : 6;
        return in.layer * kSub + k;
    };
    auto extent = [&](int ph) -> uint32_t {
        if (ph == L * kSub) return (uint32_t)c->vocab;
        switch (ph % kSub) {
            case 0: return qkv_rows;
            case 1: return (uint32_t)(B * c->n_kv_heads * pl.nsplit * pl.hsplit);
            case 2: return (uint32_t)c->hidden;
            case 3: return moe ? (uint32_t)c->n_experts : 0u;
            case 4: return moe ? (uint32_t)c->expert_ffn : (uint32_t)c->ffn;
            case 5: return moe ? (uint32_t)pl.n_cu : split ? (uint32_t)c->ffn / kDownPart : 0u;  // shares, parts
            default: return (uint32_t)c->hidden;
        }
    };
    for (int ph = 0; ph < nphase; ++ph) seen[ph].assign(extent(ph), 0);
    std::vector<uint8_t> slot_seen(pl.n_head, 0);
    if (pl.qoff.size() != (size_t)pl.n_cu + 1 || pl.qoff[pl.n_cu] != pl.instrs.size()) return 1;
    for (int cu = 0; cu < pl.n_cu; ++cu) {
        int last = -1;
        for (uint32_t i = pl.qoff[cu]; i < pl.qoff[cu + 1]; ++i) {
            const Instr& in = pl.instrs[i];
            if (in.op < OP_QKV || in.op > OP_DRED) return 1;
            const bool moe_op = in.op == OP_ROUTE || in.op == OP_EGU || in.op == OP_EDOWN || in.op == OP_EPART;
            if (moe_op != moe && in.op != OP_QKV && in.op != OP_ATTN && in.op != OP_O && in.op != OP_HEAD) return 1;
            if ((in.op == OP_DPART || in.op == OP_DRED) != split && (in.op == OP_DPART || in.op == OP_DRED ||
                                                                     in.op == OP_DOWN))
                return 1;
            if (in.op != OP_HEAD && in.layer >= L) return 2;
            const int ph = phase_of(in);
            if (ph < last) return 3;  // queue not in phase order
            last = ph;
            const uint32_t ext = extent(ph);
            if (in.count == 0 || in.begin + in.count > ext || in.begin + in.count < in.begin) return 5;
            if ((in.op == OP_O || in.op == OP_DOWN) && in.count > kMaxResidRows) return 4;
            if (in.op == OP_EDOWN && in.count > kMaxEredRows) return 4;
            if (in.op == OP_DPART && in.count > kMaxDpartParts) return 4;
            if (in.op == OP_DRED && in.count > dred_rows_for(c)) return 4;
            if (in.op == OP_EPART && (in.begin != (uint32_t)cu || in.count != 1)) return 4;
            if (sliced && (in.op == OP_QKV || in.op == OP_ROUTE) && in.count > kMaxResidRows) return 4;
            if (sliced && in.op == OP_EGU && in.count > kMaxEguSlicedRows) return 4;
            for (uint32_t r = in.begin; r < in.begin + in.count; ++r) {
                if (seen[ph][r]) return 6;  // covered twice
                seen[ph][r] = 1;
            }
            if (in.op == OP_HEAD) {
                if (in.slot >= pl.n_head) return 7;
                if (slot_seen[in.slot]++) return 8;
            }
        }
    }
    for (int ph = 0; ph < nphase; ++ph)
        for (uint8_t v : seen[ph])
            if (!v) return 9;  // row never covered
    return 0;
}

struct Layout {
    size_t state, tickets, instrs, qoff, layers, rope, h, qkv, attn, act, attn_part, head_part, logits_scr, tok_scr,
        trace, trace_bytes, route, eact, eptr, cuts, epart, dpart, wdt, total;
    size_t head_slots;  // argmax partial slots (per sequence)
};

inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Instruction counts of a plan on n compute units (total and the longest queue).
void plan_counts(const mk_model_config* c, const mk_runtime_config* rt, int n, int nsplit, size_t* total,
                 size_t* per_cu) {
    const size_t items = (size_t)rt->max_batch * c->n_kv_heads * nsplit * auto_hsplit(c, rt, n, nsplit);
    // instructions per CU of a phase of `rows` rows cut at `max_rows`
    auto cut = [&](size_t rows, size_t max_rows) { return ((rows + n - 1) / n + max_rows - 1) / max_rows; };
    const size_t od = cut((size_t)c->hidden, kMaxResidRows);  // O / DOWN instructions per CU
    const bool moe = c->n_experts > 0;
    const bool sliced = x_slices_for(rt->max_batch, c->hidden, c->n_q_heads * c->head_dim, moe) > 1;
    const size_t qkv_rows = (size_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
    const size_t qkv = sliced ? cut(qkv_rows, kMaxResidRows) : 1;  // sliced inputs: cut instructions
    const size_t route = !moe ? 0 : sliced ? cut((size_t)c->n_experts, kMaxResidRows) : 1;
    const size_t ffn = sliced ? cut((size_t)c->expert_ffn, kMaxEguSlicedRows) : 1;  // GATEUP / EGU
    // MoE: one expert-down share per CU, and combine instructions of kMaxEredRows rows;
    // split DOWN: part instructions, then row-sum instructions
    const bool split = down_split_on(c, rt);
    const size_t epart = moe ? 1 : split ? cut((size_t)c->ffn / kDownPart, kMaxDpartParts) : 0;
    const size_t down = moe ? cut((size_t)c->hidden, kMaxEredRows) : split ? cut((size_t)c->hidden, dred_rows_for(c)) : od;
    *per_cu = (size_t)c->n_layers * (qkv + route + ffn + epart + od + down + (items + n - 1) / n) + 1;
    *total = (size_t)c->n_layers * ((qkv + route + ffn + epart + od + down) * (size_t)n + items) + (size_t)n;
}

// with_wdt: also the transposed down matrices (the decode layout; a multi-position
// plan uses those of its decode handle).
Layout layout(const mk_model_config* c, const mk_runtime_config* rt, int n_cu, int nsplit, bool with_wdt = true) {
    Layout lo{};
    const size_t B = (size_t)rt->max_batch, d = c->hidden, hd = c->head_dim;
    const size_t qkv_rows = (size_t)(c->n_q_heads + 2 * c->n_kv_heads) * hd;
    const size_t G = (size_t)(c->n_q_heads / c->n_kv_heads);
    size_t n_instr = 0, per_cu = 0;
    plan_counts(c, rt, n_cu, nsplit, &n_instr, &per_cu);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    lo.state = take(sizeof(DevState));
    lo.tickets = take(((size_t)c->n_layers * B * c->n_kv_heads + 1) * kCtrStride * 4);
    lo.instrs = take(n_instr * sizeof(Instr));
    lo.qoff = take((size_t)(n_cu + 1) * 4);
    lo.layers = take((size_t)c->n_layers * sizeof(DevLayer));
    lo.rope = take((size_t)rt->max_seq * (hd / 2) * 8);
    lo.h = take(B * d * 8);
    lo.qkv = take(B * qkv_rows * 8);
    lo.attn = take(B * c->n_q_heads * hd * 8);
    lo.act = take(B * (size_t)std::max(c->ffn, 0) * 8);
    const size_t nx = c->n_experts ? (size_t)(c->n_shared_experts + c->n_experts) : 0;
    lo.route = take(B * (size_t)c->n_experts * 8);
    lo.eact = take(nx * B * (size_t)c->expert_ffn * 8);
    // selected slots of a layer at most: the shared experts and B x top_k routed ones
    const size_t slots = c->n_experts ? (size_t)c->n_shared_experts + std::min((size_t)c->n_experts, B * c->top_k) : 0;
    lo.epart = take(slots * B * d * 8);
    const bool split = down_split_on(c, rt);
    lo.dpart = take(split ? (size_t)c->ffn / kDownPart * B * d * 8 : 0);
    lo.wdt = take(split && with_wdt ? (size_t)c->n_layers * c->ffn * d * 2 : 0);
    lo.eptr = take((size_t)c->n_layers * 3 * nx * 8);
    lo.attn_part = take(B * c->n_kv_heads * nsplit * G * (hd + 2) * 8);
    // argmax partial slots: one LM-head instruction per CU (persistent), or the
    // one-kernel-per-op path's head workgroups (bounded by one per 16 rows)
    const size_t conv_blocks = ((size_t)c->vocab + 15) / 16;
    lo.head_slots = (rt->mode == MK_MODE_GRAPH ? std::max((size_t)n_cu, conv_blocks) : (size_t)n_cu) *
                    (kComputeWaves + kLoaderWaves);
    lo.head_part = take(lo.head_slots * B * 2 * 8);
    lo.logits_scr = take(B * c->vocab * 4);
    lo.tok_scr = take(B * 4);
    lo.trace_bytes = rt->trace ? (size_t)n_cu * per_cu * kTraceWords * 4 : 0;
    lo.trace = take(lo.trace_bytes);
    lo.cuts = rt->mode == MK_MODE_MEGAKERNEL ? take((size_t)kMaxCuts * n_cu * 2 * 4) : 0;  // per-launch queue ranges
    lo.total = off;
    return lo;
}

// MK_MODE_ENV resolved: the persistent kernel only when the environment opts in.
mk_runtime_config resolve_mode(const mk_runtime_config* rt) {
    mk_runtime_config r = *rt;
    if (r.mode == MK_MODE_ENV) {
        const char* v = std::getenv("MK_MEGAKERNEL");
        r.mode = (v && std::strcmp(v, "1") == 0) ? MK_MODE_MEGAKERNEL : MK_MODE_GRAPH;
    }
    return r;
}

int device_cus() {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 256;
    return prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
}

int resolve_cus(const mk_runtime_config* rt) { return rt->num_cus > 0 ? rt->num_cus : device_cus(); }

// The multi-position plan of a persistent decode handle: kChunkRows rows of one
// sequence per launch (prompt chunks, draft verification), VALU GEMVs, one
// attention split per item.
mk_runtime_config chunk_rt(const mk_model_config* c, const mk_runtime_config* rt) {
    mk_runtime_config r = *rt;
    r.down_split = down_split_on(c, rt) ? 1 : -1;  // the decode handle's transposed Wdown, if any
    r.max_batch = kChunkRows;
    r.mode = MK_MODE_MEGAKERNEL;
    r.gemv_kind = 1;
    r.attn_splits = 1;
    r.trace = 0;
    return r;
}

// Whether a handle of this configuration carries the multi-position plan.
bool chunk_supported(const mk_model_config* c, const mk_runtime_config* rt) {
    if (rt->mode != MK_MODE_MEGAKERNEL) return false;
    const mk_runtime_config r = chunk_rt(c, rt);
    if (validate(c, &r, nullptr) != MK_OK) return false;
    const uint32_t ring = ring_chunks_for(x_bytes_for(c, &r, 1, kChunkRows));
    return ring >= kMinRingChunks && max_wave_span(c, &r) <= ring;
}

// Workspace bytes of a handle on n CUs: the decode plan's layout, then (when
// supported) the multi-position plan's.
size_t handle_bytes(const mk_model_config* c, const mk_runtime_config* rt, int n, Layout* main_lo, Layout* chunk_lo) {
    const Layout m = layout(c, rt, n, auto_splits(c, rt, n));
    size_t total = (m.total + 255) & ~(size_t)255;
    Layout k{};
    if (chunk_supported(c, rt)) {
        const mk_runtime_config r = chunk_rt(c, rt);
        k = layout(c, &r, n, 1, false);
        total += k.total;
    }
    if (main_lo) *main_lo = m;
    if (chunk_lo) *chunk_lo = k;
    return total;
}

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
    hipStream_t last_stream = nullptr;  // stream of the last enqueued step (mk_destroy waits for it)
    bool used = false;
    int static_dev = -1;  // >= 0: the workspace is that device's static array (mk_create_static)
    std::vector<int32_t> ctx;
    uint32_t epoch = 0;
    HostErr* host_err = nullptr;
    HostErr* host_err_dev = nullptr;
    bool latched = false;
    mk_status latched_status = MK_OK;
    std::string last_error;
    // multi-position plan (persistent mode, when supported): its own workspace
    // region after the decode plan's, the decode plan's KV cache and context lengths
    int ncut = 1;  // persistent launches per decode step (mk_set_cuts)
    bool chunk_ok = false;
    Plan cplan;
    Layout clo;
    Params cP;
    size_t coff = 0;
    // graph mode
    hipGraphExec_t gexec = nullptr;
    hipGraph_t graph = nullptr;
    const void *g_in = nullptr, *g_out = nullptr, *g_logits = nullptr;
    int32_t inject = 0;
};

// Workspace of the handles made by mk_create_static, for callers that cannot
// allocate device memory.  Each device the library runs on holds its own copy
// for the life of the process.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[MK_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];   // device address of `scratch` on each device, once known
bool g_static_busy[kMaxDevices];   // a live handle of mk_create_static uses that device's array
}  // namespace

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

mk_status mk_query_sizes(const mk_model_config* cfg, const mk_runtime_config* rt_in, size_t* workspace_bytes,
                         size_t* kv_bytes) {
    if (!workspace_bytes || !kv_bytes || !rt_in) return MK_E_INVALID;
    const mk_runtime_config rt_r = resolve_mode(rt_in);
    const mk_runtime_config* rt = &rt_r;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    // the compute-unit count may be resolved only at mk_create: size for every count up to the bound
    const int n_max = rt->num_cus > 0 ? rt->num_cus : kMaxCus;
    size_t ws = 0;
    for (int n = rt->num_cus > 0 ? n_max : 1; n <= n_max; ++n) ws = std::max(ws, handle_bytes(cfg, rt, n, nullptr, nullptr));
    *workspace_bytes = ws;
    *kv_bytes = 2ull * cfg->n_layers * rt->max_batch * cfg->n_kv_heads * (size_t)rt->max_seq * cfg->head_dim * 2;
    return MK_OK;
}

mk_status mk_plan_inspect(const mk_model_config* cfg, const mk_runtime_config* rt_in, int32_t num_cus, int64_t* out,
                          int32_t cap) {
    if (!out || cap < 0 || !rt_in) return MK_E_INVALID;
    const mk_runtime_config rt_r = resolve_mode(rt_in);
    const mk_runtime_config* rt = &rt_r;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    if (num_cus <= 0 || num_cus > kMaxCus) return MK_E_INVALID;
    if ((uint32_t)cfg->vocab < (uint32_t)num_cus) return MK_E_UNSUPPORTED;
    Plan pl = build_plan(cfg, rt, num_cus);
    const int64_t d = cfg->hidden, hd = cfg->head_dim;
    const int64_t ffn_w = cfg->n_experts
                              ? (int64_t)cfg->n_experts * d +
                                    (int64_t)(cfg->n_shared_experts + cfg->n_experts) * 3 * cfg->expert_ffn * d
                              : 3 * (int64_t)cfg->ffn * d;
    const int64_t per_layer = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * hd * d + d * cfg->n_q_heads * hd + ffn_w + 2 * d;
    const size_t xb = x_bytes_for(cfg, rt, pl.nsplit);
    const bool pm = rt->mode == MK_MODE_MEGAKERNEL;  // (the three batch-1 paths are persistent-kernel paths)
    int64_t vals[17] = {num_cus, (int64_t)pl.instrs.size(), (int64_t)ring_chunks_for(xb), (int64_t)pl.max_per_cu,
                        2 * (cfg->n_layers * per_layer + (int64_t)cfg->vocab * d + d), verify_plan(cfg, rt, pl),
                        pl.nsplit, pl.phases, (int64_t)xb, (int64_t)pl.n_head, use_mfma(cfg, rt) ? 2 : 1, pl.hsplit,
                        (int64_t)max_wave_span(cfg, rt), down_split_on(cfg, rt) ? 1 : 0,
                        (pm && gu_direct_on(cfg, rt)) ? 1 : 0, down_q_on(cfg, rt) ? 1 : 0,
                        (pm && o_direct_on(cfg, rt)) ? 1 : 0};
    for (int i = 0; i < cap && i < 17; ++i) out[i] = vals[i];
    return MK_OK;
}

}  // extern "C"

// mk_create, and mk_create_static with static_dev >= 0 (the workspace is that
// device's static array: no size query of every CU count, no pinned error word).
static mk_status create_impl(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt_in,
                             void* d_workspace, size_t workspace_bytes, void* d_kv, size_t kv_bytes, void* stream,
                             mk_handle** out, int static_dev) {
    if (!out || !rt_in) return MK_E_INVALID;
    *out = nullptr;
    const mk_runtime_config rt_r = resolve_mode(rt_in);
    const mk_runtime_config* rt = &rt_r;
    mk_status s = validate(cfg, rt, nullptr);
    if (s != MK_OK) return s;
    if (!w || !w->tok_embedding || !w->final_norm || !w->layers || !d_workspace || !d_kv) return MK_E_INVALID;
    for (int l = 0; l < cfg->n_layers; ++l) {
        const mk_layer_weights& Lw = w->layers[l];
        if (!Lw.attn_norm || !Lw.wq || !Lw.wk || !Lw.wv || !Lw.wo || !Lw.mlp_norm) return MK_E_INVALID;
        if (cfg->n_experts == 0 && (!Lw.w_gate || !Lw.w_up || !Lw.w_down)) return MK_E_INVALID;
        if (cfg->n_experts) {
            if (!Lw.router || !Lw.e_gate || !Lw.e_up || !Lw.e_down) return MK_E_INVALID;
            if (cfg->n_shared_experts && (!Lw.s_gate || !Lw.s_up || !Lw.s_down)) return MK_E_INVALID;
            for (int e = 0; e < cfg->n_experts; ++e)
                if (!Lw.e_gate[e] || !Lw.e_up[e] || !Lw.e_down[e]) return MK_E_INVALID;
        }
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
    if (n_cu <= 0 || n_cu > kMaxCus || (uint32_t)cfg->vocab < (uint32_t)n_cu ||
        (rt->mode == MK_MODE_MEGAKERNEL && n_cu > device_cus())) {
        // the persistent kernel needs every workgroup resident: one per compute unit
        delete h;
        return MK_E_UNSUPPORTED;
    }
    h->plan = build_plan(cfg, rt, n_cu);
    const int vr = verify_plan(cfg, rt, h->plan);
    if (vr != 0) {
        delete h;
        return MK_E_INVALID;
    }
    const size_t hb = handle_bytes(cfg, rt, n_cu, &h->lo, &h->clo);
    h->coff = (h->lo.total + 255) & ~(size_t)255;
    h->chunk_ok = chunk_supported(cfg, rt);
    if (h->chunk_ok && workspace_bytes < hb) h->chunk_ok = false;  // (a static array too small for it)
    if (workspace_bytes < h->lo.total || (static_dev < 0 && workspace_bytes < need_ws) || kv_bytes < need_kv) {
        delete h;
        return static_dev < 0 ? MK_E_INVALID : MK_E_CAPACITY;
    }
    h->ws = (char*)d_workspace;
    h->ws_bytes = workspace_bytes;
    h->kv = d_kv;
    h->kv_bytes = kv_bytes;
    h->ctx.assign(rt->max_batch, 0);
    h->static_dev = static_dev;

    // pinned, device-visible error word (not for mk_create_static: an allocation)
    if (static_dev >= 0 ||
        hipHostMalloc((void**)&h->host_err, sizeof(HostErr), hipHostMallocMapped | hipHostMallocCoherent) !=
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
    P.gemv_mfma = use_mfma(cfg, rt) ? 1 : 0;
    P.down_slices = cfg->n_experts ? 1 : down_slices_for(rt->max_batch, cfg->ffn, P.gemv_mfma != 0);
    P.x_slices = x_slices_for(rt->max_batch, cfg->hidden, cfg->n_q_heads * cfg->head_dim, cfg->n_experts > 0);
    P.E = cfg->n_experts;
    P.top_k = cfg->top_k;
    P.n_shared = cfg->n_experts ? cfg->n_shared_experts : 0;
    P.Fe = cfg->expert_ffn;
    P.down_split = down_split_on(cfg, rt) ? 1 : 0;
    P.down_q = down_q_on(cfg, rt) ? 1 : 0;
    P.gu_direct = gu_direct_on(cfg, rt) ? 1 : 0;
    P.o_direct = o_direct_on(cfg, rt) ? 1 : 0;
    P.V = cfg->vocab;
    P.B = rt->max_batch;
    P.S = rt->max_seq;
    P.G = cfg->n_q_heads / cfg->n_kv_heads;
    P.qkv_rows = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
    P.nsplit = h->plan.nsplit;
    P.hsplit = h->plan.hsplit;
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
    P.h = (uint64_t*)(ws + lo.h);
    P.qkv = (uint64_t*)(ws + lo.qkv);
    P.attn = (uint64_t*)(ws + lo.attn);
    P.act = (uint64_t*)(ws + lo.act);
    P.attn_part = (uint64_t*)(ws + lo.attn_part);
    P.head_part = (uint64_t*)(ws + lo.head_part);
    P.route = (uint64_t*)(ws + lo.route);
    P.eact = (uint64_t*)(ws + lo.eact);
    P.eptr = (const uint16_t* const*)(ws + lo.eptr);
    P.epart = (uint64_t*)(ws + lo.epart);
    P.dpart = (uint64_t*)(ws + lo.dpart);
    P.attn_ticket = (uint32_t*)(ws + lo.tickets);
    P.head_ticket = P.attn_ticket + (size_t)cfg->n_layers * rt->max_batch * cfg->n_kv_heads * kCtrStride;
    P.state = (DevState*)(ws + lo.state);
    P.ctx_len = (int32_t*)(ws + lo.state + offsetof(DevState, ctx_len));
    P.chunk = 0;
    P.host_err = h->host_err_dev;
    P.instrs = (const Instr*)(ws + lo.instrs);
    P.queue_off = (const uint32_t*)(ws + lo.qoff);
    P.x_bytes = (uint32_t)x_bytes_for(cfg, rt, h->plan.nsplit);
    P.ring_chunks = ring_chunks_for(P.x_bytes);
    // argmax partials: one per wave that computes LM-head rows (all eight waves of a
    // CU in the VALU and MoE kernels, the four compute waves on the matrix cores)
    P.n_head_slots = rt->mode == MK_MODE_MEGAKERNEL
                         ? h->plan.n_head * (uint32_t)(P.gemv_mfma ? kComputeWaves : kComputeWaves + kLoaderWaves)
                         : (uint32_t)conventional_head_blocks(P) * (uint32_t)kComputeWaves;
    auto give_up = [&](mk_status st) {
        if (h->host_err) (void)hipHostFree(h->host_err);
        delete h;
        return st;
    };
    if (P.ring_chunks < kMinRingChunks || P.n_head_slots > lo.head_slots ||
        h->plan.instrs.size() * sizeof(Instr) > lo.qoff - lo.instrs)
        return give_up(MK_E_UNSUPPORTED);
    if (P.x_slices > 1 && (size_t)P.B * P.d * 4 > (size_t)P.ring_chunks * kChunk + P.x_bytes) {
        h->last_error = "the LM-head input does not fit the ring and staging area";
        return give_up(MK_E_UNSUPPORTED);
    }
    if (rt->mode == MK_MODE_MEGAKERNEL && max_wave_span(cfg, rt) > P.ring_chunks) {
        h->last_error = "a compute wave's row batch does not fit the LDS ring";
        return give_up(MK_E_UNSUPPORTED);
    }
    if (rt->trace) {
        P.trace = (uint32_t*)(ws + lo.trace);
        P.trace_stride = (uint32_t)(lo.trace_bytes / ((size_t)n_cu * kTraceWords * 4));
        if (h->plan.max_per_cu > P.trace_stride) return give_up(MK_E_INVALID);
    }
    if (rt->mode == MK_MODE_GRAPH) {
        // kernel attributes are set before any capture
        const hipError_t pe = prepare_conventional(P);
        if (pe != hipSuccess) {
            hip_fail(h, pe, "prepare_conventional");
            return give_up(MK_E_HIP);
        }
    } else {
        const hipError_t pe = prepare_megakernel(P);
        if (pe == hipErrorInvalidConfiguration) {
            h->last_error = "one workgroup of the persistent kernel does not fit a compute unit";
            return give_up(MK_E_UNSUPPORTED);
        }
        if (pe != hipSuccess) {
            hip_fail(h, pe, "prepare_megakernel");
            return give_up(MK_E_HIP);
        }
    }
    const uint32_t tmo = rt->spin_timeout_ms ? rt->spin_timeout_ms : 2000u;
    P.spin_ticks = (uint64_t)tmo * 100000ull;

    // ---- the multi-position plan: same weights, KV cache, context lengths and error
    // state as the decode plan; its own schedule, activations and tickets
    if (h->chunk_ok) {
        const mk_runtime_config r8 = chunk_rt(cfg, rt);
        h->cplan = build_plan(cfg, &r8, n_cu);
        Params& C = h->cP;
        C = P;
        char* cb = ws + h->coff;
        const Layout& cl = h->clo;
        C.B = kChunkRows;
        C.gemv_mfma = 0;
        C.down_slices = cfg->n_experts ? 1 : down_slices_for(kChunkRows, cfg->ffn, false);
        C.x_slices = x_slices_for(kChunkRows, cfg->hidden, cfg->n_q_heads * cfg->head_dim, cfg->n_experts > 0);
        C.nsplit = h->cplan.nsplit;
        C.hsplit = h->cplan.hsplit;
        C.layers = (const DevLayer*)(cb + cl.layers);
        C.rope = (const float2*)(cb + cl.rope);
        C.h = (uint64_t*)(cb + cl.h);
        C.qkv = (uint64_t*)(cb + cl.qkv);
        C.attn = (uint64_t*)(cb + cl.attn);
        C.act = (uint64_t*)(cb + cl.act);
        C.attn_part = (uint64_t*)(cb + cl.attn_part);
        C.head_part = (uint64_t*)(cb + cl.head_part);
        C.route = (uint64_t*)(cb + cl.route);
        C.eact = (uint64_t*)(cb + cl.eact);
        C.epart = (uint64_t*)(cb + cl.epart);
        C.dpart = (uint64_t*)(cb + cl.dpart);
        C.down_split = down_split_on(cfg, &r8) ? 1 : 0;
        C.gu_direct = 0;  // (the multi-position kernels stream every GEMV through the ring)
        C.down_q = 0;
        C.o_direct = 0;
        C.eptr = (const uint16_t* const*)(cb + cl.eptr);
        C.attn_ticket = (uint32_t*)(cb + cl.tickets);
        C.head_ticket = C.attn_ticket + (size_t)cfg->n_layers * kChunkRows * cfg->n_kv_heads * kCtrStride;
        C.instrs = (const Instr*)(cb + cl.instrs);
        C.queue_off = (const uint32_t*)(cb + cl.qoff);
        C.x_bytes = (uint32_t)x_bytes_for(cfg, &r8, C.nsplit, kChunkRows);
        C.ring_chunks = ring_chunks_for(C.x_bytes);
        C.n_head_slots = h->cplan.n_head * (uint32_t)(kComputeWaves + kLoaderWaves);
        C.trace = nullptr;
        C.trace_stride = 0;
        C.inject = 0;
        C.chunk = 1;
        C.chunk_seq = 0;
        h->chunk_ok = verify_plan(cfg, &r8, h->cplan) == 0 && C.nsplit == 1 && C.ring_chunks >= kMinRingChunks &&
                      C.n_head_slots <= cl.head_slots &&
                      h->cplan.instrs.size() * sizeof(Instr) <= cl.qoff - cl.instrs &&
                      max_wave_span(cfg, &r8) <= C.ring_chunks &&
                      (C.x_slices == 1 || (size_t)C.B * C.d * 4 <= (size_t)C.ring_chunks * kChunk + C.x_bytes) &&
                      prepare_megakernel(C) == hipSuccess;
    }

    // ---- uploads (synchronous; create is not on the hot path)
    std::vector<DevLayer> dl(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; ++l) {
        const mk_layer_weights& Lw = w->layers[l];
        dl[l] = DevLayer{(const uint16_t*)Lw.attn_norm, (const uint16_t*)Lw.wq,     (const uint16_t*)Lw.wk,
                         (const uint16_t*)Lw.wv,        (const uint16_t*)Lw.wo,     (const uint16_t*)Lw.mlp_norm,
                         (const uint16_t*)Lw.w_gate,    (const uint16_t*)Lw.w_up,   (const uint16_t*)Lw.w_down,
                         (const uint16_t*)Lw.router,    nullptr};
        if (P.down_split)
            dl[l].w_down_t = (const uint16_t*)(ws + lo.wdt + (size_t)l * cfg->ffn * cfg->hidden * 2);
    }
    // MoE expert table [L][gate, up, down][shared (if any), experts 0..E-1]
    const int nx = cfg->n_experts ? cfg->n_shared_experts + cfg->n_experts : 0;
    std::vector<const void*> ep((size_t)cfg->n_layers * 3 * nx);
    for (int l = 0; l < cfg->n_layers && nx; ++l) {
        const mk_layer_weights& Lw = w->layers[l];
        for (int m = 0; m < 3; ++m) {
            const void* const* routed = m == 0 ? Lw.e_gate : m == 1 ? Lw.e_up : Lw.e_down;
            const void* shared = m == 0 ? Lw.s_gate : m == 1 ? Lw.s_up : Lw.s_down;
            const void** row = ep.data() + ((size_t)l * 3 + m) * nx;
            for (int x = 0; x < cfg->n_shared_experts; ++x) row[x] = shared;
            for (int e = 0; e < cfg->n_experts; ++e) row[cfg->n_shared_experts + e] = routed[e];
        }
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
    hipError_t e = hipSuccess;
    auto cp = [&](size_t off, const void* src, size_t bytes) {
        if (e == hipSuccess && bytes) e = hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, h->stream);
    };
    if (e == hipSuccess) e = hipMemsetAsync(ws, 0, h->chunk_ok ? h->coff + h->clo.total : lo.total, h->stream);
    cp(lo.instrs, h->plan.instrs.data(), h->plan.instrs.size() * sizeof(Instr));
    cp(lo.qoff, h->plan.qoff.data(), h->plan.qoff.size() * 4);
    cp(lo.layers, dl.data(), dl.size() * sizeof(DevLayer));
    cp(lo.rope, rope.data(), rope.size() * 4);
    cp(lo.eptr, ep.data(), ep.size() * sizeof(void*));
    if (h->chunk_ok) {
        const Layout& cl = h->clo;
        cp(h->coff + cl.instrs, h->cplan.instrs.data(), h->cplan.instrs.size() * sizeof(Instr));
        cp(h->coff + cl.qoff, h->cplan.qoff.data(), h->cplan.qoff.size() * 4);
        cp(h->coff + cl.layers, dl.data(), dl.size() * sizeof(DevLayer));
        cp(h->coff + cl.rope, rope.data(), rope.size() * 4);
        cp(h->coff + cl.eptr, ep.data(), ep.size() * sizeof(void*));
    }
    // the split down projection's transposed Wdown, [F][d] per layer
    for (int l = 0; l < cfg->n_layers && P.down_split && e == hipSuccess; ++l)
        e = transpose_bf16((uint16_t*)dl[l].w_down_t, (const uint16_t*)dl[l].w_down, cfg->hidden, cfg->ffn, h->stream);
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

extern "C" {

mk_status mk_create(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt, void* d_workspace,
                    size_t workspace_bytes, void* d_kv, size_t kv_bytes, void* stream, mk_handle** out) {
    return create_impl(cfg, w, rt, d_workspace, workspace_bytes, d_kv, kv_bytes, stream, out, -1);
}

mk_status mk_create_static(const mk_model_config* cfg, const mk_weights* w, const mk_runtime_config* rt_in, void* d_kv,
                           size_t kv_bytes, void* stream, mk_handle** out) {
    if (!out || !rt_in || !cfg) return MK_E_INVALID;
    *out = nullptr;
    mk_runtime_config rt = resolve_mode(rt_in);
    if (rt.mode != MK_MODE_MEGAKERNEL) return MK_E_UNSUPPORTED;
    rt.down_split = -1;  // the transposed Wdown would not fit the array
    mk_status s = validate(cfg, &rt, nullptr);
    if (s != MK_OK) return s;
    // the workspace this handle lays out, against the array (host-only arithmetic)
    const int n_cu = resolve_cus(&rt);
    if (n_cu <= 0 || n_cu > kMaxCus) return MK_E_UNSUPPORTED;
    if (layout(cfg, &rt, n_cu, auto_splits(cfg, &rt, n_cu)).total > (size_t)MK_STATIC_WORKSPACE_BYTES)
        return MK_E_CAPACITY;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MK_E_HIP;
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        if (g_static_busy[dev]) return MK_E_STATE;  // one live handle per device shares the array
        if (!g_static_ptr[dev]) {
            // once per device, with that device current: the array's device address
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MK_E_HIP;
            g_static_ptr[dev] = ptr;
        }
        ptr = g_static_ptr[dev];
        g_static_busy[dev] = true;
    }
    // create_impl zeroes the workspace before the first step, so nothing an earlier
    // handle left in the array survives
    s = create_impl(cfg, w, &rt, ptr, (size_t)MK_STATIC_WORKSPACE_BYTES, d_kv, kv_bytes, stream, out, dev);
    if (s != MK_OK) {
        std::lock_guard<std::mutex> lock(g_static_mu);
        g_static_busy[dev] = false;
    }
    return s;
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
    A.tok_rows = h->rt.max_batch;
    A.tok_out = tok_out;
    A.logits = logits;
    A.tag0 = (++h->epoch) * tags_per_step(h->cfg.n_layers);
    Params P = h->P;
    if (h->inject == 1) {
        // one step whose layer-0 attention waits for a tag no producer writes, with a
        // 1 ms watchdog: every workgroup times out or sees the error and leaves
        P.spin_ticks = 100000ull;
        P.inject = 1;
        h->inject = 0;
    }
    if (h->rt.mode == MK_MODE_MEGAKERNEL) {
        for (int j = 0; j < h->ncut; ++j) {  // one launch, or the parts of a cut step in order
            if (h->ncut > 1) P.cut_q = (const uint32_t*)(h->ws + h->lo.cuts) + (size_t)j * h->P.n_cu * 2;
            HIPCHK(h, launch_megakernel(P, A, st));
        }
    } else if (stride != 1 || P.inject) {
        // prompt positions (strided tokens) and the fault test run uncaptured
        HIPCHK(h, launch_conventional(P, A, st));
    } else {
        // replay a graph captured for these pointers (re-captured when they change); the
        // captured tag base stays fixed, which is enough because kernel order alone
        // orders the one-kernel-per-op path
        if (!h->gexec || h->g_in != tok_in || h->g_out != tok_out || h->g_logits != logits) {
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
            if (e == hipSuccess) e = launch_conventional(P, A, cap);
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
    for (int b = 0; b < h->rt.max_batch; ++b) h->ctx[b] += 1;
    h->last_stream = st;
    h->used = true;
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

// One multi-position launch: rows 0..n-1 are tokens tok[0..n-1] of sequence seq at
// positions ctx[seq] .. ctx[seq] + n - 1 (later rows repeat the last token, and
// their results are ignored); logits and greedy tokens of all rows land in the
// plan's scratch rows; the sequence advances by n on the device.
static mk_status run_chunk(mk_handle* h, int seq, const int32_t* tok, int n, hipStream_t st) {
    if (h->ctx[seq] + n > h->rt.max_seq) return MK_E_CAPACITY;
    StepArgs A;
    std::memset(&A, 0, sizeof(A));
    A.tok_in = tok;
    A.tok_stride = 1;
    A.tok_rows = n;
    A.tok_out = (int32_t*)(h->ws + h->coff + h->clo.tok_scr);
    A.logits = (float*)(h->ws + h->coff + h->clo.logits_scr);
    A.tag0 = (++h->epoch) * tags_per_step(h->cfg.n_layers);
    Params C = h->cP;
    C.chunk_seq = seq;
    HIPCHK(h, launch_megakernel(C, A, st));
    h->ctx[seq] += n;
    h->last_stream = st;
    h->used = true;
    return MK_OK;
}

mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P, float* d_logits, int32_t* d_next,
                     void* stream) {
    if (!h || !d_tokens || !d_logits || !d_next || P <= 0) return MK_E_INVALID;
    if (B != h->rt.max_batch) return MK_E_INVALID;
    mk_status s = check_latched(h);
    if (s != MK_OK) return s;
    for (int b = 0; b < B; ++b)
        if (h->ctx[b] + P > h->rt.max_seq) return MK_E_CAPACITY;
    if (h->chunk_ok) {
        // kChunkRows prompt positions per launch; the last one's logits and token
        // are the sequence's
        const hipStream_t st = (hipStream_t)stream;
        const size_t V = (size_t)h->cfg.vocab;
        const char* crow = h->ws + h->coff;
        for (int b = 0; b < B; ++b) {
            int n = 0;
            for (int t0 = 0; t0 < P; t0 += n) {
                n = std::min(kChunkRows, P - t0);
                s = run_chunk(h, b, d_tokens + (size_t)b * P + t0, n, st);
                if (s != MK_OK) return s;
            }
            HIPCHK(h, hipMemcpyAsync(d_logits + (size_t)b * V, crow + h->clo.logits_scr + (size_t)(n - 1) * V * 4, V * 4,
                                     hipMemcpyDeviceToDevice, st));
            HIPCHK(h, hipMemcpyAsync(d_next + b, crow + h->clo.tok_scr + (size_t)(n - 1) * 4, 4, hipMemcpyDeviceToDevice,
                                     st));
        }
        return MK_OK;
    }
    float* scr_logits = (float*)(h->ws + h->lo.logits_scr);
    int32_t* scr_tok = (int32_t*)(h->ws + h->lo.tok_scr);
    for (int t = 0; t < P; ++t) {
        const bool last = t == P - 1;
        s = run_step(h, d_tokens + t, P, last ? d_next : scr_tok, last ? d_logits : scr_logits, (hipStream_t)stream);
        if (s != MK_OK) return s;
    }
    return MK_OK;
}

mk_status mk_verify_step(mk_handle* h, int32_t seq, const int32_t* d_tokens, int32_t n, float* d_logits,
                         int32_t* d_next, void* stream) {
    if (!h || !d_tokens || !d_logits || !d_next || n < 1 || n > kChunkRows) return MK_E_INVALID;
    if (seq < 0 || seq >= h->rt.max_batch) return MK_E_INVALID;
    if (!h->chunk_ok) return MK_E_UNSUPPORTED;
    mk_status s = check_latched(h);
    if (s != MK_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    s = run_chunk(h, seq, d_tokens, n, st);
    if (s != MK_OK) return s;
    const char* crow = h->ws + h->coff;
    HIPCHK(h, hipMemcpyAsync(d_logits, crow + h->clo.logits_scr, (size_t)n * h->cfg.vocab * 4, hipMemcpyDeviceToDevice,
                             st));
    HIPCHK(h, hipMemcpyAsync(d_next, crow + h->clo.tok_scr, (size_t)n * 4, hipMemcpyDeviceToDevice, st));
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
    // a handle without the host-mapped error word learns of a device error here
    const mk_status cleared = (!h->host_err && ds.error) ? (ds.error == DERR_NAN ? MK_E_DEVICE_NAN : MK_E_DEVICE_TIMEOUT)
                                                         : MK_OK;
    // tickets back to zero; the step counter (tag base) keeps counting, so values
    // left by an aborted step never match a later step's tags
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.tickets, 0,
                             ((size_t)h->cfg.n_layers * h->rt.max_batch * h->cfg.n_kv_heads + 1) * kCtrStride * 4, st));
    if (h->chunk_ok)
        HIPCHK(h, hipMemsetAsync(h->ws + h->coff + h->clo.tickets, 0,
                                 ((size_t)h->cfg.n_layers * kChunkRows * h->cfg.n_kv_heads + 1) * kCtrStride * 4, st));
    HIPCHK(h, hipMemsetAsync(h->ws + h->lo.state + offsetof(DevState, error), 0, 16, st));
    HIPCHK(h, hipStreamSynchronize(st));
    if (h->host_err) std::memset(h->host_err, 0, sizeof(HostErr));
    h->latched = false;
    h->latched_status = MK_OK;
    h->last_error.clear();
    return cleared;
}

mk_status mk_moe_slots(mk_handle* h, uint64_t* out) {
    if (!h || !out) return MK_E_INVALID;
    if (h->used) HIPCHK(h, hipStreamSynchronize(h->last_stream));
    HIPCHK(h, hipStreamSynchronize(h->stream));
    unsigned long long v = 0;
    HIPCHK(h, hipMemcpy(&v, h->ws + h->lo.state + offsetof(DevState, moe_slots), sizeof(v), hipMemcpyDeviceToHost));
    *out = (uint64_t)v;
    return MK_OK;
}

mk_status mk_debug_inject(mk_handle* h, int32_t fault, int32_t arg) {
    (void)arg;
    if (!h) return MK_E_INVALID;
    if (fault != 0 && fault != 1) return MK_E_INVALID;
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

mk_status mk_set_cuts(mk_handle* h, const int32_t* h_layers, int32_t n) {
    if (!h || n < 0 || (n > 0 && !h_layers) || n >= kMaxCuts) return MK_E_INVALID;
    if (h->rt.mode != MK_MODE_MEGAKERNEL || h->rt.trace) return MK_E_UNSUPPORTED;
    const int L = h->cfg.n_layers;
    for (int i = 0; i < n; ++i)
        if (h_layers[i] < 1 || h_layers[i] > L || (i > 0 && h_layers[i] <= h_layers[i - 1])) return MK_E_INVALID;
    if (n == 0) {
        h->ncut = 1;
        return MK_OK;
    }
    // launch j runs the instructions of phases [b_j, b_{j+1}): phase = layer * 7 +
    // sub-phase (QKV, ATTN, O, ROUTE, GATEUP / EGU, EPART / DPART, DOWN / EDOWN / DRED), the LM head L * 7
    constexpr int kSub = 7;
    auto phase_of = [&](const Instr& in) -> int {
        if (in.op == OP_HEAD) return L * kSub;
        const int k = in.op == OP_QKV ? 0 : in.op == OP_ATTN ? 1 : in.op == OP_O ? 2 : in.op == OP_ROUTE ? 3
                    : (in.op == OP_GATEUP || in.op == OP_EGU) ? 4 : (in.op == OP_EPART || in.op == OP_DPART) ? 5 : 6;
        return in.layer * kSub + k;
    };
    std::vector<int> bnd(1, 0);
    for (int i = 0; i < n; ++i) bnd.push_back(h_layers[i] * kSub);
    bnd.push_back(L * kSub + 1);
    const int k = n + 1, ncu = h->P.n_cu;
    std::vector<uint32_t> q((size_t)k * ncu * 2);
    for (int cu = 0; cu < ncu; ++cu) {
        const uint32_t a = h->plan.qoff[cu], e = h->plan.qoff[cu + 1];
        uint32_t i = a;
        for (int j = 0; j < k; ++j) {
            q[((size_t)j * ncu + cu) * 2] = i;
            while (i < e && phase_of(h->plan.instrs[i]) < bnd[j + 1]) ++i;
            q[((size_t)j * ncu + cu) * 2 + 1] = i;
        }
    }
    HIPCHK(h, hipStreamSynchronize(h->stream));
    if (h->used) HIPCHK(h, hipStreamSynchronize(h->last_stream));
    HIPCHK(h, hipMemcpy(h->ws + h->lo.cuts, q.data(), q.size() * 4, hipMemcpyHostToDevice));
    h->ncut = k;
    return MK_OK;
}

int32_t mk_kernels_per_step(const mk_handle* h) {
    if (!h) return -1;
    return h->rt.mode == MK_MODE_MEGAKERNEL ? h->ncut : conventional_kernels_per_step(h->P);
}

mk_status mk_destroy(mk_handle* h) {
    if (!h) return MK_E_INVALID;
    // work enqueued on the handle's stream may still write the pinned error word
    // or replay the graph: let it finish before either is freed
    (void)hipStreamSynchronize(h->stream);
    if (h->used && h->last_stream != h->stream) (void)hipStreamSynchronize(h->last_stream);
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    if (h->graph) (void)hipGraphDestroy(h->graph);
    if (h->host_err) (void)hipHostFree(h->host_err);
    if (h->static_dev >= 0) {
        std::lock_guard<std::mutex> lock(g_static_mu);
        g_static_busy[h->static_dev] = false;
    }
    delete h;
    return MK_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Cut planner [page "一个大内核不够：在哪里切分流式推理模型", sections "规划器总览：只用常规画像排序切分",
// "瓦片图如何估计单次服务时间" and "事件图如何算出首次发布分数"]: candidates are scored by
// simulating their launches as an event graph up to the first release; nothing is
// run end to end.  For a decode step the regions are the layers and the LM head, the
// candidates one-kernel-per-op or one persistent launch per run of regions, and the
// release is the step's token.
// ------------------------------------------------------------------------------------------------
extern "C" {

mk_status mk_event_sim(const mk_event_task* tasks, int32_t n, double* h_finish) {
    if (!tasks || !h_finish || n < 0) return MK_E_INVALID;
    std::vector<double> stream_free;
    for (int32_t i = 0; i < n; ++i) {
        const mk_event_task& t = tasks[i];
        if (t.stream < 0 || t.stream >= 1024 || t.duration < 0 || t.dispatch < 0) return MK_E_INVALID;
        if (t.n_deps < 0 || t.n_deps > MK_EVENT_MAX_DEPS) return MK_E_INVALID;
        double ready = 0.0;
        for (int32_t d = 0; d < t.n_deps; ++d) {
            const int32_t j = t.deps[d];
            if (j < 0 || j >= i) return MK_E_INVALID;  // dependencies come earlier (a DAG in order)
            ready = std::max(ready, h_finish[j]);
        }
        if ((size_t)t.stream >= stream_free.size()) stream_free.resize(t.stream + 1, 0.0);
        // the task waits for its inputs and for its stream, then pays its dispatch
        const double start = std::max(ready, stream_free[t.stream]) + t.dispatch;
        h_finish[i] = start + t.duration;
        stream_free[t.stream] = h_finish[i];
    }
    return MK_OK;
}

// Score of one candidate: its launches on one stream as an event graph.
static double score_cuts(const mk_cut_costs* c, const std::vector<int>& starts) {
    const int L = c->n_layers;
    std::vector<mk_event_task> ev;
    for (size_t j = 0; j < starts.size(); ++j) {
        const int a = starts[j], b = j + 1 < starts.size() ? starts[j + 1] : L + 1;  // regions [a, b), L = head
        mk_event_task t;
        std::memset(&t, 0, sizeof(t));
        t.stream = 0;
        t.dispatch = c->launch_us;
        double d = c->refill_us ? c->refill_us[a] : 0.0;  // nothing prefetched at a launch's start
        for (int r = a; r < b; ++r) d += r < L ? c->layer_us[r] : c->head_us;
        t.duration = d;
        if (j > 0) {
            t.n_deps = 1;
            t.deps[0] = (int32_t)j - 1;
        }
        ev.push_back(t);
    }
    std::vector<double> fin(ev.size());
    if (mk_event_sim(ev.data(), (int32_t)ev.size(), fin.data()) != MK_OK) return NAN;  // a negative duration
    return fin.back();
}

mk_status mk_plan_cuts(const mk_cut_costs* c, int32_t* h_cut_layers, int32_t* n_cuts, double* predicted_us,
                       double* single_launch_us, int32_t* use_conventional) {
    if (!c || !h_cut_layers || !n_cuts || !predicted_us || !single_launch_us || !use_conventional) return MK_E_INVALID;
    const int L = c->n_layers;
    if (L < 1 || L > 4096 || !c->layer_us || c->launch_us < 0) return MK_E_INVALID;
    // regions 0..L (L: the LM head); a candidate is the set of regions that start a launch
    // (region 0 always does).  Up to 16 regions every candidate is simulated; beyond,
    // the best cut set is found by dynamic programming over the same additive score
    // (one stream: the event graph of a candidate is a chain of its launches).
    const int R = L + 1;
    std::vector<int> best_starts{0};
    double best = score_cuts(c, best_starts);
    if (std::isnan(best)) return MK_E_INVALID;
    *single_launch_us = best;
    if (R - 1 <= 16) {
        for (uint32_t m = 1; m < (1u << (R - 1)); ++m) {
            std::vector<int> st{0};
            for (int r = 1; r < R; ++r)
                if (m & (1u << (r - 1))) st.push_back(r);
            const double s = score_cuts(c, st);
            if (std::isnan(s)) return MK_E_INVALID;
            if (s < best) {
                best = s;
                best_starts = st;
            }
        }
    } else {
        auto region = [&](int r) { return r < L ? c->layer_us[r] : c->head_us; };
        std::vector<double> f(R + 1, 1e300);
        std::vector<int> from(R + 1, 0);
        f[0] = 0.0;
        for (int b = 1; b <= R; ++b) {
            double run = 0.0;
            for (int a = b - 1; a >= 0; --a) {
                run += region(a);
                const double s = f[a] + c->launch_us + (c->refill_us ? c->refill_us[a] : 0.0) + run;
                if (s < f[b]) {
                    f[b] = s;
                    from[b] = a;
                }
            }
        }
        std::vector<int> st;
        for (int b = R; b > 0; b = from[b]) st.push_back(from[b]);
        std::reverse(st.begin(), st.end());
        best_starts = st;
        best = score_cuts(c, st);
        if (std::isnan(best)) return MK_E_INVALID;
    }
    *use_conventional = c->conventional_us > 0 && c->conventional_us < best ? 1 : 0;
    *predicted_us = *use_conventional ? c->conventional_us : best;
    *n_cuts = (int32_t)best_starts.size() - 1;
    for (size_t j = 1; j < best_starts.size(); ++j) h_cut_layers[j - 1] = best_starts[j];
    return MK_OK;
}

}  // extern "C"
