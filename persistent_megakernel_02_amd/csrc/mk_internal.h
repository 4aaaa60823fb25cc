// Definitions shared by the host runtime and the HIP kernels: the instruction
// record of the per-CU queues, the kernel parameter block, the device state and
// the tagged activation word that carries the dependencies between compute units.
//
// The schedule follows the page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞",
// section "Megakernel：从零设计的深度融合方案": every compute unit receives an
// ordered list of composite instructions before launch and its dependencies are
// fixed statically.  The page's completion counters are realised here in the
// activations themselves: every cross-CU value is written as one 8-byte word
// {fp32 value, tag} whose tag names (step, layer, phase), and a consumer polls the
// words it needs until every tag matches.  One agent-scope 8-byte store publishes
// a value and its readiness together, so no fence, flag or cache writeback sits
// between producer and consumer.
#pragma once
#include <stdint.h>

namespace mk {

constexpr int kComputeWaves = 4;                    // waves that run instructions
constexpr int kLoaderWaves = 4;                     // waves that stream weights HBM -> LDS
constexpr int kThreads = 64 * (kComputeWaves + kLoaderWaves);
constexpr uint32_t kChunk = 1024;                   // one loader issue: 64 lanes x 16 B
constexpr uint32_t kLdsBytes = 160 * 1024;          // LDS of one gfx950 compute unit
constexpr uint32_t kStaticLds = 1024;               // reserved for the control block
constexpr uint32_t kMinRingChunks = 72;             // >= one attention block (2 x 32 KV chunks) + its RoPE chunk
constexpr int kLoaderLag = 4;                       // chunks in flight per loader wave (deeper queues slow the polls)
// The same by batch: at batch 1 and 2 (long rows streamed in segments) six measured best.
template <int B> constexpr int loader_lag() { return B <= 2 ? 6 : kLoaderLag; }
constexpr int kMaxBatch = 8;
constexpr int kMaxGroup = 4;                        // q heads per KV head
constexpr uint32_t kMaxResidRows = 64;              // O / DOWN rows per instruction
constexpr uint32_t kCtrStride = 32;                 // uint32 per counter (128 B apart)
constexpr int kStageWords = 16;                     // tagged words per lane in flight (argmax reduce)
constexpr int kStagePassWords = 4;                  // tagged words per lane per staging pass (two in flight)
constexpr int kStagePassWordsWide = 8;              // the same for the wide inputs of O and DOWN
// The persistent kernel's dense VALU path up to batch 4 has the registers for
// twice the words per pass of the RMSNorm inputs (a 2048-wide input at batch 1 then
// takes one pass per lane); batch 8, and wider passes of the O / DOWN inputs, would
// spill.  The per-lane
// element order does not depend on the pass width, so the sums of squares are the
// same bits either way.
template <int B> constexpr int stage_words() { return B <= 4 ? 2 * kStagePassWords : kStagePassWords; }
template <int B> constexpr int stage_words_wide() { return kStagePassWordsWide; }
constexpr int kAttnBlockGroups = 32;                // KV position groups (2 KB each) one attention pass holds
static_assert(kMinRingChunks >= 2 * kAttnBlockGroups + 1, "an attention block and its RoPE chunk fit the ring");
constexpr int kAttnWavePositions = 64;              // positions one wave scores per block (its score area)
constexpr uint32_t kDownSliceBytes = 64 * 1024;     // largest fp32 DOWN input slice (all batch rows) staged at once

// Matrix-core GEMV: bf16 parts of each activation (3 while 3 B columns fit the
// 16 of a tile, else 2) and the LDS bytes of the parts of K activations of B rows.
// Rows of a 16-row matrix-core tile per 1 KB weight chunk, and the columns of a
// tile's unit (16 rows x kMfmaUnitCols, 16 / kMfmaChunkRows chunks): every row
// length of a matrix-core instruction is a multiple of kMfmaUnitCols.
constexpr int kMfmaChunkRows = 2;
constexpr int kMfmaUnitCols = 512 / kMfmaChunkRows;
__host__ __device__ constexpr int mfma_parts(int B) { return 3 * B <= 16 ? 3 : 2; }
// 16-byte slots per (k-block, k-group) row of the parts area: the PRT * B used
// columns rounded up to an odd count, so the eight k-groups that 64 consecutive
// elements fall in start in eight different LDS bank groups.
__host__ __device__ constexpr int parts_pitch(int B) { return (mfma_parts(B) * B) | 1; }
__host__ __device__ constexpr size_t parts_bytes(int B, int K) { return (size_t)2 * parts_pitch(B) * K; }
constexpr uint32_t kMfmaPartsBytes = 72 * 1024;     // largest parts area of a DOWN column slice
// Partial tiles of a matrix-core GEMV instruction summed across the waves:
// [wave][tile < 4][k-group][batch row] x 16 bytes.
__host__ __device__ constexpr size_t mfma_red_bytes(int B) { return (size_t)4 * 4 * 4 * B * 16; }

// Column slices of the DOWN projection: the fewest (a power of two) whose input
// slice fits the LDS budget (fp32: B rows of F / slices values in kDownSliceBytes;
// matrix cores: their parts in kMfmaPartsBytes); 0 if the slices would not be
// whole 1 KB chunks (VALU) or whole units of kMfmaUnitCols columns (matrix cores) of a row.
__host__ __device__ constexpr int down_slices_for(int B, int F, bool mfma = false) {
    int n = 1;
    if (mfma) {
        while (parts_bytes(B, F / n) > kMfmaPartsBytes && n < 64) n *= 2;
        return (F % n == 0 && (F / n) % kMfmaUnitCols == 0) ? n : 0;
    }
    while ((size_t)B * (size_t)(F / n) * 4u > kDownSliceBytes && n < 64) n *= 2;
    if (n > 1) {
        const int chunks = F % n ? 0 : (F / n) * 2 / 1024;  // 1 KB chunks per row slice: a power of two
        if (chunks == 0 || ((F / n) * 2) % 1024 != 0 || (chunks & (chunks - 1)) != 0) return 0;
    }
    return n;
}

// Column slices of the hidden-wide and attention-wide GEMV inputs (QKV, router,
// expert gate/up, O): 1, except for MoE models whose B x hidden fp32 input does
// not fit the LDS next to the weight ring (hidden 4096 at batch 8): then the fewest
// power-of-two slices of at most kDownSliceBytes (0: no such slicing).
__host__ __device__ constexpr int x_slices_for(int B, int hidden, int attn_width, bool moe) {
    if (!moe || (size_t)B * (size_t)hidden * 4u <= kDownSliceBytes) return 1;
    const int a = down_slices_for(B, hidden), b = down_slices_for(B, attn_width);
    return (a == 0 || b == 0) ? 0 : (a > b ? a : b);
}
// f values of one expert (gate, up) instruction when its input is sliced: the
// partial sums of every selected slot's rows wait in LDS between slices.
constexpr uint32_t kMaxEguSlicedRows = 6;

// Rows of one compute wave's batch for a row of `rb` bytes: about 8 KB per wave.
// From batch 4 on two rows share each x piece read from LDS (one row per batch
// left the wave waiting on LDS reads of x).
__host__ __device__ constexpr int rows_per_batch(uint32_t rb, int B = 1) {
    return B >= 4 ? 2 : rb <= 2048u ? 4 : rb <= 4096u ? 2 : 1;
}

// Long rows at batch 1 and 2 stream through the ring in segments of kSegBytes
// (measured: 2 KB and 16 KB segments were slower, 4 KB too; 4 KB rows segmented:
// slower).
constexpr uint32_t kSegBytes = 8192;
constexpr uint32_t kSegRowBytes = 8192;
__host__ __device__ constexpr bool segmented_rows(uint32_t rb, int B) { return B <= 2 && rb >= kSegRowBytes; }

// Rows of a wave's batch in the persistent kernel's ring GEMV (1, 2 or 4); a
// (gate, up) pair always shares one batch.
__host__ __device__ constexpr int ring_batch_rows(uint32_t rb, int B, bool pairs) {
    return rows_per_batch(rb, B) >= 4 ? 4 : (rows_per_batch(rb, B) == 2 || pairs) ? 2 : 1;
}

// Chunks of the ring one compute wave holds at most while it waits for a row
// batch of `rb`-byte rows: from the chunk its mark names (the batch start) to the
// chunk holding the batch end.  Rows are packed back to back, so a batch may
// start inside a chunk.
__host__ __device__ constexpr uint32_t ring_batch_span(uint32_t rb, int B, bool pairs) {
    return segmented_rows(rb, B) ? kSegBytes / kChunk + 1u
                                 : ((uint32_t)ring_batch_rows(rb, B, pairs) * rb + kChunk - 1u) / kChunk + 1u;
}

// LDS floats one attention item uses: raw q (G heads), k and v; rotated q; the new
// K and V as bf16; the scores of every wave ([wave][position][kMaxGroup]); the wave
// partials ([wave][G]: maximum, sum, four 16-lane rows of HD); when the item
// merges splits, the split partials ([split][G]: maximum, sum, HD); one flag word.
__host__ __device__ constexpr size_t attn_lds_floats(int G, int HD, int nsplit, int nnew = 1) {
    return (size_t)(2 * G * HD + 3 * nnew * HD + kComputeWaves * kAttnWavePositions * kMaxGroup +
                    kComputeWaves * G * (4 * HD + 2) + nsplit * G * (HD + 2) + 4);
}

enum Op : uint16_t {
    OP_QKV = 1,     // RMSNorm + rows of [Wq; Wk; Wv] -> raw q/k/v (fp32)
    OP_ATTN = 2,    // RoPE + KV append + attention of one (sequence, KV head, split)
    OP_O = 3,       // rows of Wo, residual add
    OP_GATEUP = 4,  // RMSNorm + (gate, up) row pairs -> silu(g) * u (fp32)
    OP_DOWN = 5,    // rows of Wdown, residual add
    OP_HEAD = 6,    // final RMSNorm + LM-head rows + argmax partials
    OP_ROUTE = 7,   // MoE: RMSNorm + router rows -> router logits (fp32)
    OP_EGU = 8,     // MoE: RMSNorm + top-k routing + (gate, up) row pairs of the selected experts
    OP_EDOWN = 9,   // MoE: per output row, the selected experts' outputs weighted in ascending order, residual add
    OP_EPART = 10,  // MoE: down rows of the CU's share of (selected expert, row) pairs -> unweighted outputs
    OP_DPART = 11,  // dense DOWN by columns: parts [begin, begin + count) of F -> partial outputs of every row
    OP_DRED = 12,   // dense DOWN by columns: per output row the parts' partials in order, residual add
};

// Batch 1 with F = 8192: the down projection is reduced by column quarters.  Compute
// wave q keeps x[2048 q, 2048 q + 2048) in registers (4 pieces per lane) and reduces
// quarter q of every row of the instruction; a row is its quarters' sums added in
// quarter order (Params::down_q).  Each wave reads only its quarter of the weights
// from LDS, not the whole 32 KB input once per row.
constexpr uint32_t kDownQPieces = 256;  // 16-byte pieces of one quarter row
__host__ __device__ constexpr bool down_quarters_for(int B, int F) { return B == 1 && F == 4 * (int)kDownQPieces * 8; }

// Batch 1: the loader waves load the (gate, up) rows from HBM into registers
// instead of reading them from the LDS ring (Params::gu_direct), for the Llama
// shapes each head_dim instantiation serves: head_dim 64 kernels rows of hidden
// 2048 (4 KB: 4 pieces per lane), head_dim 128 kernels hidden 4096 (8 KB: 8).
// 128 registers of rows in flight per loader wave, unrolled blocks of 16 KB x 4.
__host__ __device__ constexpr int gu_npl(int head_dim) { return head_dim == 64 ? 4 : 8; }
__host__ __device__ constexpr int gu_ahead(int npl) { return 32 / npl; }  // rows in flight per loader wave
__host__ __device__ constexpr int gu_block(int npl) { return 64 / npl; }  // rows per unrolled block

// The dense down projection split by columns (batch 4 and 8; opt-in below): F is
// cut into parts of kDownPart SwiGLU outputs.  Part j's partial output of every
// row i is the sum over its f of act[f] * Wdown[i][f], accumulated in ascending f
// from a transposed copy of Wdown (rows of d, so a part streams contiguously); the
// owner of a row adds the parts' partials in part order.  The transposed rows are
// read whole by all four compute waves: lane l of wave w takes outputs
// 8 (64 w + l) .. + 7, so d <= kDownSplitMaxHidden.
constexpr uint32_t kDownPart = 32;
constexpr int kDownSplitMaxHidden = 8 * 64 * 4;
constexpr uint32_t kMaxDpartParts = 8;  // parts per OP_DPART instruction (their inputs staged at once)
constexpr int kDpartRowsPerGet = 4;     // transposed rows a wave waits for at a time
// Output rows per OP_DRED instruction (and per row-sum workgroup of the
// one-kernel-per-op path): the staged partials, parts x B x rows words, stay
// within the B x hidden floats a QKV instruction stages.
__host__ __device__ inline uint32_t dred_rows(uint32_t d, uint32_t F) {
    const uint32_t np = F / kDownPart, r = np ? d / np : 1u;
    return r < 1u ? 1u : r > kMaxResidRows ? kMaxResidRows : r;
}

// MoE expert down projection: the (selected slot, output row) pairs of a layer,
// n_slots x d of them in slot-major order, are dealt to the CUs in contiguous
// ranges, so a CU stages the SwiGLU outputs of at most a few slots; the row
// owners then combine the slots' outputs (OP_EDOWN instructions of at most
// kMaxEredRows rows, whose staged outputs of every slot fit the LDS).
constexpr uint32_t kMaxEredRows = 16;
__host__ __device__ inline void moe_part_range(uint32_t n_slots, uint32_t d, int n_cu, int c, uint32_t* t0,
                                               uint32_t* t1) {
    const uint64_t T = (uint64_t)n_slots * d;
    *t0 = (uint32_t)(T * (uint64_t)c / (uint64_t)n_cu);
    *t1 = (uint32_t)(T * (uint64_t)(c + 1) / (uint64_t)n_cu);
}

// MoE limits: the selected-expert set of a layer is one 64-bit mask.
constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 8;

constexpr int kPhasesPerLayer = 5;  // QKV, ATTN, O, GATEUP (MoE: ROUTE, EGU), DOWN (MoE: EDOWN)

// Tag of the values a phase writes in one step: tag0 + layer * 5 + k + 1 with
// k = 0 QKV output, 1 attention output (and split partials), 2 residual after O
// (and the MoE router logits, a buffer of their own), 3 SwiGLU output, 4 residual
// after DOWN; the LM-head partials use L * 5 + 1.
// tag0 = epoch * (5 L + 2) (mod 2^32) with the epoch counting steps and never
// reset, so a value left from an earlier step never carries a current tag.
__host__ __device__ constexpr uint32_t phase_tag(uint32_t tag0, int layer, int k) {
    return tag0 + (uint32_t)(layer * kPhasesPerLayer + k + 1);
}
__host__ __device__ constexpr uint32_t tags_per_step(int L) { return (uint32_t)(L * kPhasesPerLayer + 2); }

// One queue entry (16 bytes).  For GEMV ops `begin/count` are rows (GATEUP:
// f-index pairs); for ATTN `begin` is the item id b*Hkv*nsplit + g*nsplit + s;
// for HEAD `slot` numbers the instruction among the LM-head instructions.
struct Instr {
    uint16_t op, layer;
    uint32_t begin, count;
    uint32_t slot;
};
static_assert(sizeof(Instr) == 16, "instruction record is 16 bytes");

struct DevLayer {
    const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
    const uint16_t* router;  // MoE [E, d], else nullptr
    const uint16_t* w_down_t;  // Wdown transposed [F][d] (the split down projection), else nullptr
};

// Device-resident state (in the workspace).
struct DevState {
    int32_t ctx_len[kMaxBatch];
    uint32_t error;  // first device error code (0 = none)
    uint32_t err_info[3];
    unsigned long long moe_slots;  // expert slots streamed by MoE layers, summed over layers and steps
    uint32_t pad[18];
};

// Host-mapped error report (pinned host memory written by the device).
struct HostErr {
    uint32_t code;
    uint32_t info[3];
};

enum DevErr : uint32_t { DERR_NONE = 0, DERR_TIMEOUT = 1, DERR_NAN = 2 };

struct Params {
    // shape
    int32_t L, d, Hq, Hkv, hd, F, V, B, S, G;  // G = Hq / Hkv
    int32_t qkv_rows, nsplit, n_cu, kv_b;      // kv_b = max_batch of the cache layout
    int32_t hsplit;                            // attention items per (sequence, KV head, split): q-head groups
    int32_t down_slices;                       // DOWN runs over F in this many column slices (power of 2)
    int32_t x_slices;                          // QKV, router, expert gate/up and O inputs: column slices (power of 2)
    int32_t gemv_mfma;                         // 1: GEMVs on the matrix cores (tile-major weight chunks)
    int32_t E, top_k, n_shared, Fe;            // MoE: experts, selected per token, shared experts, expert width
    int32_t down_split;                        // 1: DOWN as OP_DPART + OP_DRED (F / kDownPart parts)
    float eps, attn_scale;
    // weights
    const DevLayer* layers;
    const uint16_t *embed, *head, *final_norm;
    // KV cache [L][kv_b][Hkv][S][hd]
    uint16_t *kcache, *vcache;
    const float2* rope;  // [S][hd/2] (cos, sin)
    // tagged activations: {fp32 value, tag} words
    uint64_t* h;          // [B][d] residual stream
    uint64_t* qkv;        // [B][qkv_rows] raw projections
    uint64_t* attn;       // [B][Hq*hd] attention output
    uint64_t* act;        // [B][F] SwiGLU output
    uint64_t* attn_part;  // [B][Hkv][nsplit][G][hd + 2] split partials (m, l, o)
    uint64_t* head_part;  // [n_head_slots][B][2] argmax partials (value, index)
    uint64_t* route;      // MoE [B][E] router logits
    uint64_t* eact;       // MoE [n_shared + E][B][Fe] SwiGLU outputs of the experts
    uint64_t* epart;      // MoE [selected slot][B][d] unweighted down outputs of the selected experts
    uint64_t* dpart;      // split DOWN [F / kDownPart][B][d] partial outputs of the parts
    const uint16_t* const* eptr;  // MoE [L][3 (gate, up, down)][n_shared + E] expert matrices (shared first)
    uint32_t* attn_ticket;  // [L][B][Hkv] * kCtrStride, reset by the merger
    uint32_t* head_ticket;  // kCtrStride, reset by the reducer
    DevState* state;
    HostErr* host_err;  // pinned, host-mapped
    // schedule
    const Instr* instrs;
    const uint32_t* queue_off;  // [n_cu + 1]
    uint32_t n_head_slots;      // argmax partials per step (4 per LM-head instruction)
    uint32_t ring_chunks;       // LDS ring size in chunks
    uint32_t x_bytes;           // LDS staging area in bytes
    uint32_t inject;            // 1: layer-0 attention expects a tag nobody writes (watchdog test)
    uint64_t spin_ticks;        // watchdog in s_memrealtime ticks (100 MHz)
    uint32_t* trace;            // nullptr, or [n_cu][trace_stride][kTraceWords] records
    uint32_t trace_stride;      // records per CU
    // Context lengths the step reads at launch and advances at its end (the decode
    // handle's state).  chunk = 1: the B rows are consecutive positions of ONE
    // sequence, chunk_seq, of the decode handle (its KV cache rows): row r sits at
    // position ctx_len[chunk_seq] + r, attends to the cached positions and to rows
    // 0..r, and the step advances that sequence by the rows it was given.
    int32_t* ctx_len;
    int32_t chunk, chunk_seq;
    // A step cut into several persistent launches: this launch runs instructions
    // [cut_q[2 cu], cut_q[2 cu + 1]) of each CU's queue (nullptr: the whole queue).
    const uint32_t* cut_q;
    int32_t gu_direct;  // 1: (gate, up) rows HBM -> loader-wave registers, not the ring (batch 1, hidden 2048)
    int32_t down_q;     // 1: DOWN reduced by column quarters (down_quarters_for)
    int32_t o_direct;   // 1: O rows HBM -> loader-wave registers, computed there (batch 1, hidden 4096)
};
// Most persistent launches one decode step may be cut into.
constexpr int kMaxCuts = 64;
// Rows of a multi-position step (one sequence's prompt chunk or draft tokens).
constexpr int kChunkRows = kMaxBatch;

// Trace record of one instruction on one CU (s_memrealtime ticks, low 32 bits):
// {op | layer << 16, start, inputs staged, compute end, end, loader issue end,
//  ticks waiting for landed chunks, ticks the loaders waited for ring space,
//  staging start (after the wave barrier), then three op-specific words: for
//  attention the marks inputs staged, KV groups consumed, merged output
//  written; for (gate, up) rows streamed by the loader waves loader 0's rows
//  requested, input seen, rows done; for the other ops the compute ends of
//  waves 1, 2, 3; 0 = unused}
constexpr int kTraceWords = 12;

// Per-launch arguments.
struct StepArgs {
    const int32_t* tok_in;
    int32_t tok_stride;
    int32_t tok_rows;  // rows with tokens; later rows repeat the last one (a multi-position step's short chunk)
    uint32_t tag0;
    int32_t* tok_out;
    float* logits;
};

}  // namespace mk
