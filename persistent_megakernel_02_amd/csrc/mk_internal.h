// Definitions shared by the host runtime and the HIP kernels: the instruction
// record of the per-CU queues, the kernel parameter block, and the device state.
//
// The schedule follows the page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞",
// section "Megakernel：从零设计的深度融合方案": every compute unit receives an
// ordered list of composite instructions before launch, dependencies are fixed
// statically, and an instruction that needs an earlier result watches a global
// counter that every producer increments when it finishes.
#pragma once
#include <stdint.h>

namespace mk {

constexpr int kComputeWaves = 4;                        // waves that run instructions
constexpr int kThreads = 64 * (kComputeWaves + 1);      // + one loader wave
constexpr uint32_t kChunk = 1024;                       // one loader issue: 64 lanes x 16 B
constexpr uint32_t kRingBytes = 128 * 1024;             // LDS pages of the weight stream
constexpr uint32_t kRingChunks = kRingBytes / kChunk;
constexpr int kLoaderLag = 48;                          // loader chunks in flight (vmcnt <= 63)
constexpr uint32_t kXBytes = 16 * 1024;                 // LDS for the normed activations (fp32)
constexpr int kMaxBatch = 8;
constexpr int kMaxGroup = 4;                            // q heads per KV head
constexpr uint32_t kCtrStride = 32;                     // uint32 per counter (128 B apart)

enum Op : uint16_t {
    OP_QKV = 1,     // RMSNorm + rows of [Wq; Wk; Wv] -> raw q/k/v (fp32)
    OP_ATTN = 2,    // RoPE + KV append + attention of one (sequence, KV head, split)
    OP_O = 3,       // rows of Wo, residual add
    OP_GATEUP = 4,  // RMSNorm + (gate, up) row pairs -> bf16(silu(g) * u)
    OP_DOWN = 5,    // rows of Wdown, residual add
    OP_HEAD = 6,    // final RMSNorm + LM-head rows + argmax partials
};

constexpr int kPhasesPerLayer = 5;  // QKV, ATTN, O, GATEUP, DOWN
constexpr uint16_t kNoCounter = 0xFFFF;

// One queue entry (32 bytes).  For GEMV ops `begin/count` are rows (GATEUP:
// f-index pairs); for ATTN `begin` is the item id b*Hkv*nsplit + g*nsplit + s.
// Dependencies: every instruction of phase c owns one completion flag
// flags[c][slot]; a dependant waits until the wait_n flags of phase wait_ctr
// all hold the current epoch.
struct Instr {
    uint16_t op, layer;
    uint32_t begin, count;
    uint16_t wait_ctr, sig_ctr;
    uint32_t wait_n;   // producers of phase wait_ctr
    uint32_t slot;     // this instruction's flag in phase sig_ctr
    uint32_t aux[2];
};
static_assert(sizeof(Instr) == 32, "instruction record is 32 bytes");

struct DevLayer {
    const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
};

// Device-resident state (in the workspace).
struct DevState {
    int32_t ctx_len[kMaxBatch];
    uint32_t error;       // first device error code (0 = none)
    uint32_t err_info[3];
    uint32_t pad[20];
};

struct HeadPart {
    float v;
    int32_t i;
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
    float eps, attn_scale;
    // weights
    const DevLayer* layers;
    const uint16_t *embed, *head, *final_norm;
    // KV cache [L][kv_b][Hkv][S][hd]
    uint16_t *kcache, *vcache;
    const float2* rope;  // [S][hd/2] (cos, sin)
    // activations
    float* h;            // [B][d] residual stream
    float* qkv;          // [B][qkv_rows] raw projections
    float* attn;         // [B][Hq*hd] attention output
    float* act;          // [B][F] SwiGLU output
    float* attn_part;    // [B][Hkv][nsplit][G][hd + 2] split partials (m, l, o)
    uint32_t* attn_ticket;  // [L][B][Hkv] * kCtrStride, reset by the merger
    HeadPart* head_part; // [n_cu * kComputeWaves][B]
    uint32_t* counters;  // [n_ctr] * kCtrStride (LM-head ticket, one-kernel-per-op ticket)
    uint32_t* flags;     // [n_phase][flag_stride] completion epochs
    uint32_t flag_stride;
    uint32_t pad_fl;
    DevState* state;
    HostErr* host_err;   // pinned, host-mapped
    // schedule
    const Instr* instrs;
    const uint32_t* queue_off;  // [n_cu + 1]
    uint32_t head_ctr, n_head_instr;
    uint64_t spin_ticks;        // watchdog in s_memrealtime ticks (100 MHz)
    uint32_t* trace;            // nullptr, or [n_cu][trace_stride][kTraceWords] records
    uint32_t trace_stride;      // records per CU
    uint32_t pad_tr;
};

// Trace record of one instruction on one CU (s_memrealtime ticks, low 32 bits):
// {op | layer << 16, wait start, wait end, compute end, signal end, loader issue end}
constexpr int kTraceWords = 8;

// Per-launch arguments.
struct StepArgs {
    const int32_t* tok_in;
    int32_t tok_stride;
    int32_t pad0;
    int32_t* tok_out;
    float* logits;
    uint32_t epoch;
    uint32_t pad1;
};

}  // namespace mk
