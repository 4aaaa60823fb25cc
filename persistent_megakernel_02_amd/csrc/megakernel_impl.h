// The persistent decode megakernel: one launch runs a whole decode step.
//
// Design (page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "Megakernel：从零设计的深度融合方案", re-made for CDNA4):
//  - one workgroup per compute unit walks that CU's instruction queue, built on
//    the host before launch (the per-SM plan);
//  - shared memory cut into pages lets the next instructions' weights load while
//    the current one computes: LOADER waves stream the CU's weight and KV bytes
//    HBM -> LDS with 16-byte-per-lane direct-to-LDS loads
//    (global_load_lds_dwordx4) into a ring of 1 KB chunks that fills every byte
//    of LDS the activations do not need, ahead of the four COMPUTE waves, and
//    keep streaming while those wait on other compute units.  One wave's
//    direct-to-LDS issue rate tops out near 16 GB/s, below a compute unit's
//    share of HBM bandwidth, so the stream is dealt to kLoaderWaves waves:
//    chunk c of the CU stream belongs to loader c mod kLoaderWaves;
//  - dependencies travel with the data: every cross-CU activation is a tagged
//    word (see mk_internal.h) and an instruction first stages its inputs into
//    LDS, polling until every tag names the current step and phase;
//  - every spin is bounded by a watchdog (s_memrealtime, 100 MHz): on expiry the
//    CU records an error and all waves leave, so a launch always terminates.
//
// A loader's vector-memory instructions are only these LDS loads, so its vmcnt
// counter counts exactly its chunks in flight; after `s_waitcnt vmcnt(N)` it
// publishes, in LDS, the first of its own chunks not yet resident (its j-th chunk
// is stream chunk j * kLoaderWaves + k), and the stream prefix resident in the
// ring is the minimum over the loaders.  Compute waves publish, per wave, the
// first stream chunk they still need; loaders reuse ring space below the minimum.
//
// This header holds the kernel templates; each kind (dense VALU, dense matrix
// cores, MoE) is instantiated in a translation unit of its own.
#pragma once
#include <hip/hip_runtime.h>

#include "mk_device.h"

namespace mk {

struct Ctl {
    uint32_t landed[kLoaderWaves];       // loader k: first stream chunk of its own not yet resident
    uint32_t consumed[kComputeWaves];    // first chunk each compute wave still needs
    uint32_t bar;                        // compute-wave barrier arrivals (monotonic)
    uint32_t abort;                      // set when a wave gives up (error)
    int32_t ctx[kMaxBatch];              // context lengths at launch
    float ss[kMaxBatch][kComputeWaves];  // RMSNorm partials of the current instruction
    // MoE: the selected experts of the current EGU / EDOWN instruction, published
    // by compute wave 0 for the loaders (moe_seq = queue index + 1 once valid)
    uint32_t moe_seq, moe_n;
    uint8_t moe_list[kMaxExperts + 1];  // expert-table slots, shared first, then ascending experts
    // LM head: queue index + 1 once the final-norm input is staged and its statistics
    // are in ss (published by compute wave 0 for the loader waves, which join the head)
    uint32_t head_seq;
    // (gate, up) rows streamed by the loader waves (batch 1, 4 KB rows): queue index +
    // 1 once the input is staged and its statistics are in ss (compute wave 0), and
    // the loaders that have finished such an instruction (monotonic, one per loader
    // and instruction)
    uint32_t gu_seq, gu_done;
    // compute wave 0's progress: 2 qi + 1 once instruction qi has started, 2 qi + 2
    // once an O instruction's input is staged (monotonic)
    uint32_t prog;
    // O rows computed by the loader waves: loaders done (monotonic), and the layer + 1
    // whose QKV input compute wave 0 has staged
    uint32_t o_done, qkv_layer;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t align_chunk(uint32_t b) { return (b + kChunk - 1u) & ~(kChunk - 1u); }

// Context length of sequence b (LDS copy made at launch), wave-uniform so the
// stream arithmetic that depends on it stays on the scalar unit.
__device__ __forceinline__ int ctx_of(const int32_t* ctx, int b) { return __builtin_amdgcn_readfirstlane(ctx[b]); }

// GEMV instructions of the dense decoder (the ones the matrix-core kernel runs)
__device__ __forceinline__ bool is_gemv(uint32_t op) {
    return op == OP_QKV || op == OP_O || op == OP_GATEUP || op == OP_DOWN || op == OP_HEAD;
}
__device__ __forceinline__ bool is_moe_expert(uint32_t op) { return op == OP_EGU || op == OP_EPART; }

// Stream bytes of an MoE expert instruction with n selected expert slots: per slot
// the CU's (gate, up) row pairs (EGU), or the down rows of the CU's share of the
// (slot, row) pairs (EPART); whole rows.
__device__ __forceinline__ uint32_t moe_bytes(const Params& P, const Instr& in, uint32_t n) {
    if (in.op == OP_EGU) return n * 2u * in.count * (uint32_t)P.d * 2u;
    uint32_t t0, t1;
    moe_part_range(n, (uint32_t)P.d, P.n_cu, (int)in.begin, &t0, &t1);
    return (t1 - t0) * (uint32_t)P.Fe * 2u;
}

// Bytes of the CU stream that instruction `in` consumes (whole chunks).  With the
// matrix cores (MF) a GEMV streams whole 16-row tiles of 1 KB chunks.
template <int HD, bool MF = false, bool ODIR = false>
__device__ __forceinline__ uint32_t instr_bytes(const Params& P, const Instr& in, const int32_t* ctx) {
    if (MF && is_gemv(in.op)) return mfma_geo<HD>(P, in).chunks() * kChunk;
    switch (in.op) {
        case OP_HEAD: return 0;  // all eight waves stream the LM head into registers (head_direct)
        case OP_QKV:
        case OP_ROUTE: return align_chunk(in.count * (uint32_t)P.d * 2u);
        case OP_O: return (ODIR && P.o_direct) ? 0u : align_chunk(in.count * (uint32_t)(P.Hq * HD) * 2u);
        case OP_GATEUP: return P.gu_direct ? 0u : align_chunk(2u * in.count * (uint32_t)P.d * 2u);
        case OP_DOWN: return align_chunk(in.count * (uint32_t)P.F * 2u);
        case OP_DPART: return in.count * kDownPart * (uint32_t)P.d * 2u;  // whole 16 KB multiples
        case OP_ATTN: {
            const AttnItem it = attn_item_of(P, in.begin);
            const SplitRange R = split_range<HD>(ctx_of(ctx, it.b), it.s, P.nsplit);
            return (1u + (uint32_t)R.ngroups * 2u) * kChunk;  // RoPE row of position p, then the K/V groups
        }
        default: return 0;
    }
}

// Global source address of this lane's 16 bytes of chunk c of instruction `in`
// (rows packed back to back; lanes past the end re-read the first row).  Used
// for rows that are not a whole number of chunks.  (No kind streams the LM head
// through the ring: the VALU and MoE kernels read it into registers, the
// matrix-core kernel lays it out tile-major.)
template <int HD>
__device__ __forceinline__ const char* chunk_src(const Params& P, const Instr& in, const DevLayer& Lw, uint32_t c,
                                                 const int32_t* ctx) {
    const uint32_t off = c * kChunk + (uint32_t)lane_id() * 16u;
    switch (in.op) {
        case OP_QKV: {
            const uint32_t rb = (uint32_t)P.d * 2u;
            uint32_t r = off / rb, col = off - r * rb;
            if (r >= in.count) { r = 0; col = 0; }
            const uint32_t row = in.begin + r, nq = (uint32_t)(P.Hq * HD), nk = (uint32_t)(P.Hkv * HD);
            const uint16_t* base = row < nq ? Lw.wq + (size_t)row * P.d
                                 : row < nq + nk ? Lw.wk + (size_t)(row - nq) * P.d
                                                 : Lw.wv + (size_t)(row - nq - nk) * P.d;
            return (const char*)base + col;
        }
        case OP_O: {
            const uint32_t K = (uint32_t)(P.Hq * HD), rb = K * 2u;
            uint32_t r = off / rb, col = off - r * rb;
            if (r >= in.count) { r = 0; col = 0; }
            return (const char*)(Lw.wo + (size_t)(in.begin + r) * K) + col;
        }
        case OP_GATEUP: {
            const uint32_t rb = (uint32_t)P.d * 2u;
            uint32_t j = off / rb, col = off - j * rb;
            if (j >= 2u * in.count) { j = 0; col = 0; }
            const uint16_t* W = (j & 1u) ? Lw.w_up : Lw.w_gate;
            return (const char*)(W + (size_t)(in.begin + (j >> 1)) * P.d) + col;
        }
        case OP_DOWN: {
            const uint32_t rb = (uint32_t)P.F * 2u;
            uint32_t r = off / rb, col = off - r * rb;
            if (r >= in.count) { r = 0; col = 0; }
            return (const char*)(Lw.w_down + (size_t)(in.begin + r) * P.F) + col;
        }
        case OP_ROUTE: {
            const uint32_t rb = (uint32_t)P.d * 2u;
            uint32_t r = off / rb, col = off - r * rb;
            if (r >= in.count) { r = 0; col = 0; }
            return (const char*)(Lw.router + (size_t)(in.begin + r) * P.d) + col;
        }
        case OP_ATTN: {
            constexpr uint32_t rbkv = HD * 2u;
            const AttnItem it = attn_item_of(P, in.begin);
            const int b = kv_seq(P, it.b), g = it.g, s = it.s;
            const int pc = ctx_of(ctx, it.b), p = attn_pos(P, pc, it.b);
            if (c == 0) {  // (cos, sin) row of position p: HD / 2 float2, lanes past it re-read its start
                const uint32_t lo = (uint32_t)lane_id() * 16u;
                return (const char*)(P.rope + (size_t)p * (HD / 2)) + (lo < HD * 4u ? lo : 0u);
            }
            const SplitRange R = split_range<HD>(pc, s, P.nsplit);
            const uint32_t o = off - kChunk;
            const uint32_t t = o >> 11, w = o & 2047u, inner = w & 1023u;
            int pos = R.s0 + (int)(t * AttnGeom<HD>::PPW + inner / rbkv);
            uint32_t col = inner % rbkv;
            if (pos >= R.s0 + R.ncached) { pos = R.s0; col = 0; }
            const uint16_t* cache = (w >= 1024u) ? P.vcache : P.kcache;
            return (const char*)(cache + ((((size_t)in.layer * P.kv_b + b) * P.Hkv + g) * P.S + pos) * HD) + col;
        }
        default: return (const char*)P.embed;
    }
}

__device__ __forceinline__ uint32_t min_consumed(const Ctl* ctl) {
    uint32_t m = lds_ld(&ctl->consumed[0]);
#pragma unroll
    for (int w = 1; w < kComputeWaves; ++w) m = min(m, lds_ld(&ctl->consumed[w]));
    return m;
}

// One 1 KB chunk HBM -> LDS: each lane moves 16 bytes from `src` to
// lds_addr + 16 * lane.  Written as one asm block (M0 is set and consumed inside
// it, the instruction has no destination register) so the compiler neither
// counts it nor guards later LDS accesses with vmcnt waits: this wave's vmcnt is
// managed explicitly by the loader.
// Weight and KV bytes are read once per step, so the loads carry the
// non-temporal hint: in a measured dependency edge under full streaming this
// kept the exchanged words faster to reach (about 0.7 us less per edge).
__device__ __forceinline__ void dma_chunk(const char* src, uint32_t lds_addr) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt"
        :
        : "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
        : "memory");
}

// Same transfer with a wave-uniform base in SGPRs and a per-lane 32-bit offset.
// The base usually comes out of v_readfirstlane, a VALU write of an SGPR, and a
// VMEM instruction that reads such an SGPR as its address needs five wait
// states after the write (CDNA3/CDNA4 ISA, manually inserted wait states).  The
// compiler does not look inside asm for hazards, so the block supplies them
// itself; the same s_nop also covers the one wait state after the M0 write.
__device__ __forceinline__ void dma_chunk_s(const char* base, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:0 nt"
        :
        : "v"(voff), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory");
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char*)(((uint64_t)hi << 32) | lo);
}

// Byte model of an instruction's stream on the fast path.  Consecutive rows of a
// row-major matrix are consecutive bytes, so every stream is one of:
//  - up to three contiguous byte ranges read in order (QKV: the q, k and v rows
//    of the tile; O, DOWN, HEAD: one range);
//  - two matrices interleaved row by row (GATEUP: gate row r then up row r),
//    2^per_shift chunks of each in turn;
//  - the K and V blocks of consecutive position groups interleaved (ATTN), one
//    chunk each, lanes past the cached positions re-reading the block start.
// Only pointers and chunk counts, all wave-uniform: the address of any chunk is
// a few scalar operations, so a loader can take every kLoaderWaves-th chunk.
struct Stream {
    const char *p0, *p1, *p2;
    const char* head;     // ATTN: the (cos, sin) row streamed as chunk 0 ahead of the groups
    uint32_t end0, end1;  // ranges: chunk ends of the first two ranges; sliced: row ends of the first two
    uint32_t per_shift;   // interleaved: log2(chunks of each matrix per turn); sliced: log2(chunks per row slice)
    int ncached;          // ATTN: valid positions of the split
    uint32_t nrow, row_bytes, slice_bytes;  // sliced (DOWN over column slices): rows, row stride, slice width
    bool inter, attn, sliced;
};

// Slice-major order of an instruction's rows (row_bytes each) over ns column
// slices: the rows' first slices, then their second, ...; row ranges keep their
// bases (end0 / end1 in rows).  Slices are whole power-of-two chunk counts.
__device__ __forceinline__ bool slice_stream(Stream& S, uint32_t nrow, uint32_t row_bytes, uint32_t ns) {
    S.sliced = true;
    S.nrow = nrow;
    S.row_bytes = row_bytes;
    S.slice_bytes = row_bytes / ns;
    const uint32_t cps = S.slice_bytes / kChunk;
    S.per_shift = (uint32_t)__builtin_ctz(cps);
    return (S.slice_bytes & (kChunk - 1u)) == 0 && cps != 0 && (cps & (cps - 1u)) == 0;
}

template <int HD>
__device__ __forceinline__ bool setup_stream(const Params& P, const Instr& in, const DevLayer& Lw, const int32_t* ctx,
                                             Stream& S) {
    S.inter = false;
    S.attn = false;
    S.sliced = false;
    S.nrow = S.row_bytes = S.slice_bytes = 0;
    S.ncached = 0;
    S.per_shift = 0;
    S.p1 = S.p2 = S.head = nullptr;
    S.end0 = S.end1 = 0xFFFFFFFFu;
    uint32_t rb = 0;
    switch (in.op) {
        case OP_QKV: {
            rb = (uint32_t)P.d * 2u;
            if (rb & (kChunk - 1u)) return false;
            const uint32_t cpr = rb / kChunk;
            const uint32_t nq = (uint32_t)(P.Hq * HD), nk = (uint32_t)(P.Hkv * HD);
            const uint32_t r0 = in.begin, r1 = in.begin + in.count;
            const uint32_t q0 = min(r0, nq), q1 = min(r1, nq);
            const uint32_t k0 = min(max(r0, nq), nq + nk) - nq, k1 = min(max(r1, nq), nq + nk) - nq;
            const uint32_t v0 = max(r0, nq + nk) - nq - nk;
            S.p0 = (const char*)Lw.wq + (size_t)q0 * rb;
            S.p1 = (const char*)Lw.wk + (size_t)k0 * rb;
            S.p2 = (const char*)Lw.wv + (size_t)v0 * rb;
            if (P.x_slices > 1) {  // rows of the three matrices, slice-major
                S.end0 = q1 - q0;
                S.end1 = S.end0 + (k1 - k0);
                return slice_stream(S, in.count, rb, (uint32_t)P.x_slices);
            }
            S.end0 = (q1 - q0) * cpr;
            S.end1 = S.end0 + (k1 - k0) * cpr;
            return true;
        }
        case OP_O:
            rb = (uint32_t)(P.Hq * HD) * 2u;
            S.p0 = (const char*)uniform_p(Lw.wo) + (size_t)in.begin * rb;
            if (P.x_slices > 1) return slice_stream(S, in.count, rb, (uint32_t)P.x_slices);
            break;
        case OP_DOWN:
            rb = (uint32_t)P.F * 2u;
            S.p0 = (const char*)Lw.w_down + (size_t)in.begin * rb;
            if (P.down_slices > 1) return slice_stream(S, in.count, rb, (uint32_t)P.down_slices);
            break;
        case OP_ROUTE:
            rb = (uint32_t)P.d * 2u;
            S.p0 = (const char*)uniform_p(Lw.router) + (size_t)in.begin * rb;
            if (P.x_slices > 1) return slice_stream(S, in.count, rb, (uint32_t)P.x_slices);
            break;
        case OP_DPART:  // the parts' transposed Wdown rows: one contiguous run of whole chunks
            S.p0 = (const char*)uniform_p(Lw.w_down_t) + (size_t)in.begin * kDownPart * P.d * 2u;
            return true;
        case OP_GATEUP: {
            rb = (uint32_t)P.d * 2u;
            const uint32_t cpr = rb / kChunk;
            if ((rb & (kChunk - 1u)) || (cpr & (cpr - 1u))) return false;  // whole, power-of-two chunks per row
            S.p0 = (const char*)Lw.w_gate + (size_t)in.begin * rb;
            S.p1 = (const char*)Lw.w_up + (size_t)in.begin * rb;
            S.per_shift = (uint32_t)__builtin_ctz(cpr);
            S.inter = true;
            return true;
        }
        case OP_ATTN: {
            const AttnItem it = attn_item_of(P, in.begin);
            const int b = kv_seq(P, it.b), g = it.g, s = it.s;
            const int pc = ctx_of(ctx, it.b), p = attn_pos(P, pc, it.b);
            const SplitRange Rg = split_range<HD>(pc, s, P.nsplit);
            const size_t base = ((((size_t)in.layer * P.kv_b + b) * P.Hkv + g) * P.S + Rg.s0) * HD;
            S.p0 = (const char*)(P.kcache + base);
            S.p1 = (const char*)(P.vcache + base);
            S.head = (const char*)(P.rope + (size_t)p * (HD / 2));
            S.ncached = Rg.ncached;
            S.inter = true;
            S.attn = true;
            return true;
        }
        default: return false;
    }
    return (rb & (kChunk - 1u)) == 0;  // fast path needs whole chunks per row
}

// Wave-uniform base and per-lane offset of chunk c (instruction-relative) of a
// fast-path stream.
template <int HD>
__device__ __forceinline__ const char* stream_chunk(const Stream& S, uint32_t c, uint32_t& voff) {
    const uint32_t lane16 = (uint32_t)lane_id() * 16u;
    if (S.sliced) {
        const uint32_t seg = c >> S.per_shift, within = c & ((1u << S.per_shift) - 1u);
        const uint32_t slice = seg / S.nrow;
        uint32_t row = seg - slice * S.nrow;
        const char* base = S.p0;
        if (row >= S.end1) {
            base = S.p2;
            row -= S.end1;
        } else if (row >= S.end0) {
            base = S.p1;
            row -= S.end0;
        }
        voff = row * S.row_bytes + slice * S.slice_bytes + within * kChunk + lane16;
        return base;
    }
    if (!S.inter) {
        if (c < S.end0) {
            voff = c * kChunk + lane16;
            return S.p0;
        }
        if (c < S.end1) {
            voff = (c - S.end0) * kChunk + lane16;
            return S.p1;
        }
        voff = (c - S.end1) * kChunk + lane16;
        return S.p2;
    }
    if (S.attn) {
        if (c == 0) {  // the (cos, sin) row: HD * 4 bytes, lanes past it re-read its start
            voff = lane16 < (uint32_t)HD * 4u ? lane16 : 0u;
            return S.head;
        }
        c -= 1u;
    }
    const uint32_t pair = c >> (S.per_shift + 1u);
    const uint32_t within = c & ((2u << S.per_shift) - 1u);
    const uint32_t off = ((pair << S.per_shift) + (within & ((1u << S.per_shift) - 1u))) * kChunk;
    bool valid = true;
    if (S.attn) valid = (int)(pair * AttnGeom<HD>::PPW) + lane_id() / AttnGeom<HD>::LPP < S.ncached;
    voff = off + (valid ? lane16 : 0u);
    return (within >> S.per_shift) ? S.p1 : S.p0;
}

// ------------------------------------------------------------------------------------------------
// loader waves
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t landed_prefix(const Ctl* ctl) {
    uint32_t m = lds_ld(&ctl->landed[0]);
#pragma unroll
    for (int k = 1; k < kLoaderWaves; ++k) m = min(m, lds_ld(&ctl->landed[k]));
    return m;
}

// Returns the queue index of the LM-head instruction when this kernel kind has
// the loader waves join it (head_direct), else q1.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// (gate, up) rows at batch 1 (rows of 4 KB at hidden 2048, 8 KB at 4096), from HBM
// straight into the loader waves' registers.  Through the ring each pair cost a compute wave
// about 0.7 us of LDS traffic (8 KB of weights and 8 KB of fp32 x read per pair,
// next to the loaders' writes of the same bytes); the compute waves have no
// registers to spare for rows in flight, the loader waves do.  A loader reaching
// the instruction in its stream retires its chunks in flight, requests its first
// first rows (during attention and O, while the ring is full and it would only
// wait), waits for the compute waves to publish the staged input, copies its
// pieces of x to registers, and computes pairs k, k + 4, ... (the gate row, then
// the up row), refilling a row's registers as soon as its products have read them.
// It stores its SwiGLU outputs after the last row (a store between the row loads
// would make every later wait on a load also wait for the write-through store),
// then streams the down projection into the ring.  Each lane accumulates its
// pieces lane, lane + 64, ... in ascending order and wave_total reduces in its
// fixed tree: the values are bit for bit those of the ring GEMV.
typedef __attribute__((address_space(1))) const u32x4_t* gu32x4_ptr;  // global memory (no flat loads)

template <int NPL>
struct GuRows {
    gu32x4_ptr gate;  // uniform: the instruction's first gate row
    gu32x4_ptr up;
    uint32_t off;     // this lane's first piece of the wave's first row (16-byte units)
    uint32_t nu;      // rows of this wave: two per pair
    // row u of the wave (the callers' unrolled loops make is_up a constant) into dst
    __device__ __forceinline__ void issue(uint32_t u, bool is_up, uint4 (&dst)[NPL]) const {
        const gu32x4_ptr base = is_up ? up : gate;
        const uint32_t o = off + (u >> 1) * (uint32_t)(kLoaderWaves * 64 * NPL);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const u32x4_t v = __builtin_nontemporal_load(base + o + 64u * (uint32_t)g);
            dst[g] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
};

// Waits (with the watchdog) until the LDS word *p reaches `want`; false on abort.
__device__ __forceinline__ bool wait_lds_at_least(const Params& P, Ctl* ctl, const uint32_t* p, uint32_t want,
                                                  uint32_t code) {
    const uint64_t t0 = now_ticks();
    uint32_t polls = 0;
    while ((int32_t)(lds_ld(p) - want) < 0) {
        if (lds_ld(&ctl->abort)) return false;
        if ((++polls & 255u) == 0 && now_ticks() - t0 > P.spin_ticks) {
            raise_error_impl(P.state, P.host_err, &ctl->abort, DERR_TIMEOUT, code, want);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return true;
}

// Loader wave k's part of (gate, up) instruction qi (its stream has no ring bytes);
// rows of 64 NPL pieces.
template <int NPL>
__device__ __forceinline__ bool gu_loader(const Params& P, Ctl* ctl, const float* xs, const Instr& in, int k,
                                          uint32_t qi, uint32_t tag0, uint32_t* tr) {
    constexpr int D = gu_ahead(NPL), BLK = gu_block(NPL);
    constexpr uint32_t RP = 64u * NPL;  // pieces of a row
    static_assert(D % 2 == 0 && BLK % D == 0, "a row's parity must be its slot's parity");
    const uint32_t lane = (uint32_t)lane_id(), nw = (uint32_t)kLoaderWaves;
    const DevLayer Lw = ld_const(P.layers + (in.layer < P.L ? in.layer : 0));
    const uint32_t npair = in.count > (uint32_t)k ? (in.count - (uint32_t)k + nw - 1u) / nw : 0u;
    const size_t first = (size_t)in.begin * RP;
    const GuRows<NPL> gr{(gu32x4_ptr)uniform_p(Lw.w_gate) + first, (gu32x4_ptr)uniform_p(Lw.w_up) + first,
                         (uint32_t)k * RP + lane, 2u * npair};
    // Rows go in blocks of BLK (one block per instruction at 1B on 256 CUs): inside a
    // block the loop is unrolled, so every row buffer is a fixed register and every
    // wait on a row's loads counts exactly the loads issued after it (a buffer
    // carried around a loop back edge gets a full vmcnt wait).  Rows after the last
    // whole block go D at a time.
    const bool blocked = gr.nu >= (uint32_t)BLK;
    uint4 w[D][NPL];
    // The first rows are requested once the compute waves have staged the O input
    // before this instruction (or started this one): early enough to land before
    // the (gate, up) input is staged, late enough to stay out of the QKV and
    // attention edges, whose polls the burst would slow.
    if (!wait_lds_at_least(P, ctl, &ctl->prog, 2u * qi, 0xFFFFFFF8u)) return false;
    if (blocked) {
#pragma unroll
        for (int i = 0; i < D; ++i) gr.issue((uint32_t)i, (i & 1) != 0, w[i]);
    }
    if (tr && lane == 0) tr[9] = (uint32_t)now_ticks();
    // the staged input (h * g in xs) and its RMSNorm statistics
    if (!wait_lds_at_least(P, ctl, &ctl->gu_seq, qi + 1u, 0xFFFFFFF9u)) return false;
    if (tr && lane == 0) tr[10] = (uint32_t)now_ticks();
    const float r = rms_scale(ctl->ss[0], kComputeWaves, P.d, P.eps);
    const XLds x{xs, (uint32_t)P.d};
    float4 xa[NPL], xb[NPL];
#pragma unroll
    for (int g = 0; g < NPL; ++g) x.piece(0, lane + 64u * (uint32_t)g, xa[g], xb[g]);
    const uint32_t tag_out = phase_tag(tag0, in.layer, 3);
    float g_val = 0.f, keep = 0.f;
    // row u's products; after an up row, pair u / 2's output goes to lane (u / 2) mod
    // 64, and 64 pairs (or the last) are stored
    auto row = [&](uint32_t u, bool is_up, const uint4 (&v)[NPL]) {
        float acc[1] = {0.f};
#pragma unroll
        for (int g = 0; g < NPL; ++g) acc[0] = dot8(v[g], xa[g], xb[g], acc[0]);
        wave_total_n<1>(acc);
        if (!is_up) {
            g_val = acc[0];
            return;
        }
        const uint32_t t = u >> 1, tl = t & 63u;
        const float o = silu_mul(g_val * r, acc[0] * r);
        keep = lane == tl ? o : keep;
        if (tl == 63u || t + 1u == npair) {
            if (lane <= tl) st_tagged(P.act + in.begin + (uint32_t)k + nw * (t - tl + lane), keep, tag_out);
        }
    };
    uint32_t u0 = 0;
    if (blocked) {
        for (;; u0 += (uint32_t)BLK) {
            const bool next = u0 + 2u * (uint32_t)BLK <= gr.nu;  // another whole block follows
#pragma unroll
            for (int i = 0; i < BLK; ++i) {
                const uint32_t u = u0 + (uint32_t)i;
                row(u, (i & 1) != 0, w[i % D]);
                if (i + D < BLK) gr.issue(u + D, (i & 1) != 0, w[i % D]);
                else if (next) gr.issue(u + D, (i & 1) != 0, w[i % D]);
            }
            if (!next) break;
        }
        u0 += (uint32_t)BLK;
    }
    for (; u0 < gr.nu; u0 += (uint32_t)D) {  // the rest (u0 even): D rows requested at once
#pragma unroll
        for (int i = 0; i < D; ++i)
            if (u0 + (uint32_t)i < gr.nu) gr.issue(u0 + (uint32_t)i, (i & 1) != 0, w[i]);
#pragma unroll
        for (int i = 0; i < D; ++i)
            if (u0 + (uint32_t)i < gr.nu) row(u0 + (uint32_t)i, (i & 1) != 0, w[i]);
    }
    if (tr && lane == 0) tr[11] = (uint32_t)now_ticks();
    // done: the compute waves, waiting for every loader, go on to stage the down
    // projection's input (polling it while this CU still streams its rows would only
    // slow the stream), and may overwrite xs
    if (lane == 0) __hip_atomic_fetch_add(&ctl->gu_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // (the stores may still be in flight when the chunk stream resumes: they are
    // older than every chunk, so a vmcnt bound that guarantees a chunk has landed
    // still does, since loads land in order)
    return true;
}

// Loader wave k's part of O instruction qi at batch 1 with hidden 4096 (the 8B
// shape; Params::o_direct; rows of 64 NPL pieces): rows k, k + 4, ... of the
// instruction.  (At hidden 2048 the O rows are light and the loaders, busy with
// them when the O input is staged, requested the (gate, up) rows later: 786 -> 816
// us per 1B step; at 4096: 3778 -> 3691 us per 8B step.)
// The rows are requested once this layer's QKV input is staged (not during the QKV
// staging polls); the loader then waits for the O input (the attention output and
// the residual rows, staged by the compute waves), keeps its pieces of x in
// registers and stores h = residual + row.  Each lane accumulates its pieces in
// ascending order and wave_total reduces in its fixed tree: the ring GEMV's bits.
template <int NPL>
__device__ __forceinline__ bool o_loader(const Params& P, Ctl* ctl, const float* xs, const Instr& in, int k,
                                         uint32_t qi, uint32_t tag0) {
    constexpr int D = 16 / NPL;  // rows in flight: 64 registers (more spilled with x at hidden 4096)
    constexpr uint32_t RP = 64u * NPL;
    const uint32_t lane = (uint32_t)lane_id(), nw = (uint32_t)kLoaderWaves;
    const DevLayer Lw = ld_const(P.layers + (in.layer < P.L ? in.layer : 0));
    const uint32_t nrw = in.count > (uint32_t)k ? (in.count - (uint32_t)k + nw - 1u) / nw : 0u;
    const gu32x4_ptr base = (gu32x4_ptr)uniform_p(Lw.wo) + (size_t)in.begin * RP;
    const uint32_t off = (uint32_t)k * RP + lane;
    auto issue = [&](uint32_t j, uint4 (&dst)[NPL]) {
        const uint32_t o = off + j * nw * RP;
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const u32x4_t v = __builtin_nontemporal_load(base + o + 64u * (uint32_t)g);
            dst[g] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    if (!wait_lds_at_least(P, ctl, &ctl->qkv_layer, (uint32_t)in.layer + 1u, 0xFFFFFFF7u)) return false;
    uint4 w[D][NPL];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if ((uint32_t)i < nrw) issue((uint32_t)i, w[i]);
    if (!wait_lds_at_least(P, ctl, &ctl->prog, 2u * qi + 2u, 0xFFFFFFF6u)) return false;
    const uint32_t K = (uint32_t)(P.Hq * P.hd);
    const XLds x{xs, K};
    const float* hres = xs + K;
    float4 xa[NPL], xb[NPL];
#pragma unroll
    for (int g = 0; g < NPL; ++g) x.piece(0, lane + 64u * (uint32_t)g, xa[g], xb[g]);
    const uint32_t tag_out = phase_tag(tag0, in.layer, 2);
    float keep = 0.f;
    for (uint32_t j0 = 0; j0 < nrw; j0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {  // (no break: w must stay register-indexed)
            const uint32_t j = j0 + (uint32_t)i;
            if (j < nrw) {
                float acc[1] = {0.f};
#pragma unroll
                for (int g = 0; g < NPL; ++g) acc[0] = dot8(w[i][g], xa[g], xb[g], acc[0]);
                if (j + D < nrw) issue(j + D, w[i]);
                wave_total_n<1>(acc);
                // row j of this loader is row k + 4 j of the instruction; 64 rows (or the
                // last) are stored at once
                const uint32_t jl = j & 63u;
                const float v = hres[(uint32_t)k + nw * j] + acc[0];
                keep = lane == jl ? v : keep;
                if (jl == 63u || j + 1u == nrw) {
                    if (lane <= jl) st_tagged(P.h + in.begin + (uint32_t)k + nw * (j - jl + lane), keep, tag_out);
                }
            }
        }
    }
    if (lane == 0) __hip_atomic_fetch_add(&ctl->o_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
}

template <int B, int HD, bool MF, bool MOE>
__device__ __forceinline__ uint32_t loader_wave(const Params& P, Ctl* ctl, char* ring, int k, uint32_t q0, uint32_t q1,
                                                const int32_t* ctx, const float* xs, uint32_t tag0) {
    constexpr int LAG = loader_lag<B>();
    const uint32_t N = P.ring_chunks;
    const uint32_t NL = (uint32_t)kLoaderWaves;
    const uint32_t ring_base = (uint32_t)(size_t)(lds_ptr_t)ring;
    const uint32_t ring_end = ring_base + N * kChunk;
    uint32_t issued = 0, landed = 0;  // this loader's own chunks
    uint32_t limit = N;               // stream chunks below it may be written
    uint32_t cb = 0;                  // stream index of the current instruction's first chunk
    uint32_t c = (uint32_t)k;         // stream index of this loader's next chunk (c = k mod NL)
    uint32_t slot = ring_base + ((uint32_t)k % N) * kChunk;  // LDS address of ring slot c mod N
    bool stop = false;
    uint32_t stall = 0;
    auto publish = [&](uint32_t n) {
        landed = n;
        lds_st(&ctl->landed[k], n * NL + (uint32_t)k);
    };
    // Ring full: retire this loader's chunks in flight in steps (so compute waves
    // can free space without the pipe draining), then sleep until space appears.
    auto make_room = [&]() -> bool {
        const uint32_t ts = P.trace ? (uint32_t)now_ticks() : 0u;
        uint64_t t0 = 0;
        uint32_t polls = 0;
        bool ok = true;
        for (;;) {
            limit = __builtin_amdgcn_readfirstlane(min_consumed(ctl)) + N;
            if (c < limit) break;
            const uint32_t fly = issued - landed;
            if (fly > 12u) {
                wait_vmcnt<12>();
                publish(issued - 12u);
            } else if (fly > 4u) {
                wait_vmcnt<4>();
                publish(issued - 4u);
            } else if (fly > 0u) {
                wait_vmcnt<0>();
                publish(issued);
            } else {
                if (lds_ld(&ctl->abort)) {
                    ok = false;
                    break;
                }
                if (polls++ == 0) t0 = now_ticks();
                if ((polls & 255u) == 0 && now_ticks() - t0 > P.spin_ticks) {
                    raise_error_impl(P.state, P.host_err, &ctl->abort, DERR_TIMEOUT, 0xFFFFFFFDu, issued);
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (P.trace) stall += (uint32_t)now_ticks() - ts;
        return ok;
    };
    // after each issue: next own chunk and slot, and keep at most LAG in
    // flight.  (Throttling the loaders while the compute waves poll for their
    // inputs measured slower: the polls barely sped up and the stream lost more.)
    auto advance = [&]() {
        c += NL;
        slot += NL * kChunk;
        if (slot >= ring_end) slot -= N * kChunk;
        ++issued;
        if (issued - landed > (uint32_t)LAG) {
            wait_vmcnt<LAG>();
            publish(issued - (uint32_t)LAG);
        }
    };
    // MoE expert instructions: the streamed experts are known only once the compute
    // waves have routed.  Retire every chunk in flight first (the compute waves may
    // still need them to reach this instruction), then wait for the published list.
    auto wait_moe = [&](uint32_t want) -> bool {
        if (issued != landed) {
            wait_vmcnt<0>();
            publish(issued);
        }
        const uint64_t t0 = now_ticks();
        uint32_t polls = 0;
        while (lds_ld(&ctl->moe_seq) != want) {
            if (lds_ld(&ctl->abort)) return false;
            if ((++polls & 255u) == 0 && now_ticks() - t0 > P.spin_ticks) {
                raise_error_impl(P.state, P.host_err, &ctl->abort, DERR_TIMEOUT, 0xFFFFFFFCu, want);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        return true;
    };
    uint32_t head_at = q1;
    for (uint32_t i = q0; i < q1 && !stop; ++i) {
        const Instr in = ld_const(P.instrs + i);
        if (!MF && in.op == OP_HEAD) {  // the last instruction of every queue
            head_at = i;
            break;
        }
        if constexpr (B == 1 && !MF && !MOE) {
            if (HD == 128 && in.op == OP_O && P.o_direct) {  // rows into registers, no ring bytes
                if (k == 0 && P.trace && lane_id() == 0 && i > q0) {
                    uint32_t* rec = P.trace + ((size_t)blockIdx.x * P.trace_stride + (i - 1 - q0)) * kTraceWords;
                    rec[5] = (uint32_t)now_ticks();
                    rec[7] = stall;
                }
                stall = 0;
                if (issued != landed) {  // retire the chunks in flight: vmcnt counts the row loads next
                    wait_vmcnt<0>();
                    publish(issued);
                }
                if (!o_loader<gu_npl(128)>(P, ctl, xs, in, k, i, tag0)) {
                    stop = true;
                    break;
                }
                continue;
            }
            if (in.op == OP_GATEUP && P.gu_direct) {  // rows into registers, no ring bytes
                if (k == 0 && P.trace && lane_id() == 0 && i > q0) {
                    uint32_t* rec = P.trace + ((size_t)blockIdx.x * P.trace_stride + (i - 1 - q0)) * kTraceWords;
                    rec[5] = (uint32_t)now_ticks();
                    rec[7] = stall;
                }
                stall = 0;
                if (issued != landed) {  // retire the chunks in flight: vmcnt counts the row loads next
                    wait_vmcnt<0>();
                    publish(issued);
                }
                uint32_t* tr = (k == 0 && P.trace) ? P.trace + ((size_t)blockIdx.x * P.trace_stride + (i - q0)) * kTraceWords
                                                   : nullptr;
                if (!gu_loader<gu_npl(HD)>(P, ctl, xs, in, k, i, tag0, tr)) {
                    stop = true;
                    break;
                }
                continue;
            }
        }
        uint32_t nch;
        if (MOE && is_moe_expert(in.op)) {
            if (!wait_moe(i + 1u)) {
                stop = true;
                break;
            }
            nch = moe_bytes(P, in, lds_ld(&ctl->moe_n)) / kChunk;
        } else {
            nch = instr_bytes<HD, MF, B == 1 && !MF && !MOE && HD == 128>(P, in, ctx) / kChunk;
        }
        if (k == 0 && P.trace && lane_id() == 0 && i > q0) {
            uint32_t* rec = P.trace + ((size_t)blockIdx.x * P.trace_stride + (i - 1 - q0)) * kTraceWords;
            rec[5] = (uint32_t)now_ticks();
            rec[7] = stall;
        }
        stall = 0;
        const uint32_t ce = cb + nch;
        if (c < ce) {
            const DevLayer Lw = ld_const(P.layers + (in.layer < P.L ? in.layer : 0));
            Stream S;
            if (MF && is_gemv(in.op)) {
                // tile-major chunks: slot l holds row rr = l / PPR of the chunk (tile
                // row r), piece (l % PPR) ^ (r % PPR) of its run.  Rows past the end
                // (only in a last-group chunk) re-read the last row: every chunk must
                // be one load in flight, since the landed count is derived from
                // vmcnt and a chunk without a load would let an older one be
                // published early.  Per slice, the full groups and the last group
                // are walked as two regions.  In the full groups this loader takes
                // chunks h0 and h0 + 4 of every unit (h0 = its phase at the region
                // start; the region is a multiple of four chunks long), so its lanes'
                // rows are fixed and a chunk's address is a lane base plus a uniform
                // tile and column offset.
                const MfmaGeo g = mfma_geo<HD>(P, in);
                const uint32_t ks = g.K / g.slices, lane = (uint32_t)lane_id();
                const uint32_t rr = lane / kMfmaPiecesPerRow, pp = lane % kMfmaPiecesPerRow;
                const bool qkv = in.op == OP_QKV, gu = in.op == OP_GATEUP;
                const char* ra = (const char*)gemv_row(P, Lw, in, 0u);
                const char* rb = (const char*)gemv_row(P, Lw, in, gu ? 1u : 0u);
                const uint32_t shift = gu ? 1u : 0u;
                const uint64_t stride = (uint64_t)(gu ? (uint32_t)P.d : g.K) * 2u;
                auto row_ptr = [&](uint32_t j) -> const char* {  // row j of the instruction
                    return qkv ? (const char*)gemv_row(P, Lw, in, j)
                               : ((j & shift) ? rb : ra) + (uint64_t)(j >> shift) * stride;
                };
                const uint64_t tile_stride = (uint64_t)stride * (16u >> shift);  // rows of one tile
                const uint32_t FC = g.full_chunks(), LC = g.KU * g.CR;
                for (uint32_t sl = 0, rs = cb; sl < g.slices && !stop && c < ce; ++sl) {
                    const uint32_t col0 = sl * ks * 2u;
                    if (FC && c < rs + FC) {
                        const uint32_t h0 = c - rs;  // < 4
                        const uint32_t r0 = h0 * kMfmaChunkRows + rr, r1 = (h0 + 4u) * kMfmaChunkRows + rr;
                        const uint32_t p0 = col0 + (pp ^ (r0 % kMfmaPiecesPerRow)) * 16u;
                        const uint32_t p1 = col0 + (pp ^ (r1 % kMfmaPiecesPerRow)) * 16u;
                        const char* b0 = row_ptr(r0) + p0;
                        const char* b1 = row_ptr(r1) + p1;
                        uint32_t hs = 0, tl = 0, ku = 0, grp = 0;
                        for (; c < rs + FC; ) {
                            if (c >= limit && !make_room()) {
                                stop = true;
                                break;
                            }
                            const uint32_t t = grp * 4u + tl, kc = ku * (64u * kMfmaUnitKb);
                            // QKV rows span three matrices: their address is taken per chunk
                            const char* src = qkv ? row_ptr(t * 16u + (hs ? r1 : r0)) + (hs ? p1 : p0) + kc
                                                  : (hs ? b1 : b0) + (uint64_t)t * tile_stride + kc;
                            dma_chunk(src, slot);
                            advance();
                            if (kMfmaUnitChunks == 8u && hs == 0u) {
                                hs = 1u;
                                continue;
                            }
                            hs = 0u;
                            if (++tl == 4u) {
                                tl = 0;
                                if (++ku == g.KU) ku = 0, ++grp;
                            }
                        }
                    }
                    rs += FC;
                    if (stop) break;
                    // the last group: CR chunks per k-unit holding its rows in order
                    if (c < rs + LC) {
                        uint32_t x = c - rs, ku = x / g.CR, ch = x - ku * g.CR;
                        for (; c < rs + LC; ) {
                            if (c >= limit && !make_room()) {
                                stop = true;
                                break;
                            }
                            const uint32_t gr = ch * kMfmaChunkRows + rr, r = gr & 15u;
                            const uint32_t j = min(g.G4 * 64u + gr, g.nrows - 1u);
                            dma_chunk(row_ptr(j) + col0 + ku * (64u * kMfmaUnitKb) + (pp ^ (r % kMfmaPiecesPerRow)) * 16u,
                                      slot);
                            advance();
                            for (ch += kLoaderWaves; ch >= g.CR; ch -= g.CR) ++ku;
                        }
                    }
                    rs += LC;
                }
            } else if (MOE && in.op == OP_EPART) {
                // the CU's (selected slot, down row) pairs [t0, t1) in slot-major order:
                // per slot a run of consecutive rows of its down matrix, cpr chunks a row
                const uint32_t n = lds_ld(&ctl->moe_n), nx = (uint32_t)(P.n_shared + P.E);
                const uint16_t* const* tab = P.eptr + ((size_t)in.layer * 3u + 2u) * nx;
                const uint32_t d = (uint32_t)P.d, cpr = (uint32_t)P.Fe * 2u / kChunk;
                uint32_t t0, t1;
                moe_part_range(n, d, P.n_cu, (int)in.begin, &t0, &t1);
                const uint32_t w = c - cb, r = w / cpr;
                uint32_t wc = w - r * cpr, a = (t0 + r) / d, i = t0 + r - a * d;
                const char* base =
                    (const char*)ld_const(tab + __builtin_amdgcn_readfirstlane((uint32_t)ctl->moe_list[a]));
                for (; c < ce; ) {
                    if (c >= limit && !make_room()) {
                        stop = true;
                        break;
                    }
                    dma_chunk_s(uniform_ptr(base), (i * cpr + wc) * kChunk + (uint32_t)lane_id() * 16u, slot);
                    advance();
                    for (wc += NL; wc >= cpr;) {
                        wc -= cpr;
                        if (++i == d) {
                            i = 0;
                            if (++a < n)
                                base = (const char*)ld_const(
                                    tab + __builtin_amdgcn_readfirstlane((uint32_t)ctl->moe_list[a]));
                        }
                    }
                }
            } else if (MOE && in.op == OP_EGU) {
                // selected expert slot a, chunk w of its (gate, up) row pairs; the slot's
                // matrices come from the expert table (rows interleaved as in GATEUP)
                const uint32_t n = lds_ld(&ctl->moe_n), nx = (uint32_t)(P.n_shared + P.E);
                const uint32_t rb = (uint32_t)P.d * 2u;
                const uint32_t per = 2u * in.count * rb / kChunk;
                const uint16_t* const* tab = P.eptr + (size_t)in.layer * 3u * nx;
                auto slot_stream = [&](uint32_t a, Stream& X) {
                    const uint32_t x = __builtin_amdgcn_readfirstlane((uint32_t)ctl->moe_list[a]);
                    X.attn = X.sliced = false;
                    X.end0 = X.end1 = 0xFFFFFFFFu;
                    X.p1 = X.p2 = X.head = nullptr;
                    X.p0 = (const char*)(ld_const(tab + x) + (size_t)in.begin * P.d);
                    X.p1 = (const char*)(ld_const(tab + nx + x) + (size_t)in.begin * P.d);
                    X.per_shift = (uint32_t)__builtin_ctz(rb / kChunk);
                    X.inter = true;
                };
                if (P.x_slices > 1) {
                    // sliced input: slice-major over every selected slot: slice s of
                    // slot a's (gate, up) row pairs, cps chunks per row slice
                    const uint32_t sb = rb / (uint32_t)P.x_slices, cps = sb / kChunk, pss = 2u * in.count * cps;
                    uint32_t x0 = c - cb, s0 = x0 / (n * pss);
                    x0 -= s0 * n * pss;
                    uint32_t a = x0 / pss, w = x0 - a * pss;
                    for (; c < ce; ) {
                        if (c >= limit && !make_room()) {
                            stop = true;
                            break;
                        }
                        const uint32_t xs_ = __builtin_amdgcn_readfirstlane((uint32_t)ctl->moe_list[a]);
                        const uint32_t j = w / (2u * cps), half = (w / cps) & 1u, within = w % cps;
                        const char* base = (const char*)ld_const(tab + (half ? nx : 0u) + xs_);
                        const uint32_t voff = (in.begin + j) * rb + s0 * sb + within * kChunk + (uint32_t)lane_id() * 16u;
                        dma_chunk_s(uniform_ptr(base), voff, slot);
                        advance();
                        for (w += NL; w >= pss;) {
                            w -= pss;
                            if (++a == n) {
                                a = 0;
                                ++s0;
                            }
                        }
                    }
                    cb = ce;
                    continue;
                }
                uint32_t a = (c - cb) / per, w = (c - cb) - a * per;
                if (a < n) slot_stream(a, S);
                for (; c < ce; ) {
                    if (c >= limit && !make_room()) {
                        stop = true;
                        break;
                    }
                    uint32_t voff;
                    const char* base = uniform_ptr(stream_chunk<HD>(S, w, voff));
                    dma_chunk_s(base, voff, slot);
                    advance();
                    for (w += NL; w >= per && a < n; w -= per)
                        if (++a < n) slot_stream(a, S);
                }
            } else if (setup_stream<HD>(P, in, Lw, ctx, S)) {
                for (; c < ce; ) {
                    if (c >= limit && !make_room()) {
                        stop = true;
                        break;
                    }
                    uint32_t voff;
                    const char* base = uniform_ptr(stream_chunk<HD>(S, c - cb, voff));
                    dma_chunk_s(base, voff, slot);
                    advance();
                }
            } else {
                for (; c < ce; ) {
                    if (c >= limit && !make_room()) {
                        stop = true;
                        break;
                    }
                    dma_chunk(chunk_src<HD>(P, in, Lw, c - cb, ctx), slot);
                    advance();
                }
            }
        }
        cb = ce;
    }
    wait_vmcnt<0>();
    landed = issued;
    lds_st(&ctl->landed[k], 0xFFFFFFFFu);  // every chunk of this loader is resident
    const uint32_t last = head_at < q1 ? head_at : q1 - 1;
    if (k == 0 && P.trace && q1 > q0 && lane_id() == 0) {
        P.trace[((size_t)blockIdx.x * P.trace_stride + (last - q0)) * kTraceWords + 5] = (uint32_t)now_ticks();
        P.trace[((size_t)blockIdx.x * P.trace_stride + (last - q0)) * kTraceWords + 7] = stall;
    }
    return stop ? q1 : head_at;
}

// ------------------------------------------------------------------------------------------------
// compute waves
// ------------------------------------------------------------------------------------------------
// Wait until the loader has `need` chunks resident; adds the ticks spent waiting
// to `waited` (read only by the trace).
__device__ __forceinline__ bool wait_landed(const Params& P, Ctl* ctl, uint32_t need, uint32_t& waited) {
    if (landed_prefix(ctl) >= need) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        return true;
    }
    const uint64_t t0 = now_ticks();
    uint32_t polls = 0;
    bool ok = true;
    while (landed_prefix(ctl) < need) {
        if (lds_ld(&ctl->abort)) {
            ok = false;
            break;
        }
        if ((++polls & 255u) == 0 && now_ticks() - t0 > P.spin_ticks) {
            raise_error_impl(P.state, P.host_err, &ctl->abort, DERR_TIMEOUT, 0xFFFFFFFFu, need);
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(0);
    }
    waited += (uint32_t)(now_ticks() - t0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return ok;
}

__device__ __forceinline__ void set_consumed(Ctl* ctl, int wave, uint32_t chunk) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    lds_st(&ctl->consumed[wave], chunk);
}

// Barrier of the compute waves only (the loader wave never joins s_barrier).
// False when the workgroup aborted or the watchdog expired.
struct CwBarrier {
    Ctl* ctl;
    const Params* P;
    uint32_t gen;
    __device__ __forceinline__ bool operator()() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane_id() == 0) __hip_atomic_fetch_add(&ctl->bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t target = (++gen) * (uint32_t)kComputeWaves;
        const uint64_t t0 = now_ticks();
        uint32_t polls = 0;
        while (lds_ld(&ctl->bar) < target) {
            if (lds_ld(&ctl->abort)) return false;
            if ((++polls & 255u) == 0 && now_ticks() - t0 > P->spin_ticks) {
                raise_error_impl(P->state, P->host_err, &ctl->abort, DERR_TIMEOUT, 0xFFFFFFFEu, target);
                return false;
            }
            __builtin_amdgcn_s_sleep(0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        return true;
    }
};

// A wave leaving a region of the stream (one GEMV over a column slice, one
// expert's rows) moves its mark to the region's end before any barrier that
// follows inside the same instruction: it needs nothing before it again.
// Without this a wave that had no rows in the region (fewer row batches than
// waves) would keep its mark at the region's start, and since the loader only
// reuses ring slots below the smallest mark, the waves with rows would wait for
// chunks the loader may not issue once the instruction is longer than the ring.
// The chunk holding the end byte stays protected.  (Called by the instruction
// code, not inside the GEMV loops: there the extra live values pushed the VALU
// kernel past its 256 registers into scratch.)
__device__ __forceinline__ void release_region(Ctl* ctl, int wave, uint32_t end_byte) {
    set_consumed(ctl, wave, end_byte / kChunk);
}

// Ring byte address of stream byte x.
__device__ __forceinline__ uint32_t ring_addr(uint32_t x, uint32_t nchunks) {
    return ((x >> 10) % nchunks) * kChunk + (x & (kChunk - 1u));
}

// Rows [0, nrows) of the current instruction from the ring in batches of R
// consecutive rows; batch t goes to compute wave t mod kComputeWaves, so the
// four waves work on neighbouring rows and the ring span stays small.
template <int B, int R, class Epi>
__device__ __forceinline__ bool gemv_ring(const Params& P, Ctl* ctl, const char* ring, uint32_t S, uint32_t rb,
                                          uint32_t nrows, const XLds& x, int wave, uint32_t& lw, Epi& epi) {
    const int np = (int)(rb >> 4);
    const uint32_t ring_bytes = P.ring_chunks * kChunk;
    for (uint32_t r0 = (uint32_t)wave * R; r0 < nrows; r0 += (uint32_t)R * kComputeWaves) {
        const uint32_t nr = min((uint32_t)R, nrows - r0);
        const uint32_t off = S + r0 * rb;
        set_consumed(ctl, wave, off / kChunk);
        if (!wait_landed(P, ctl, (off + nr * rb + kChunk - 1u) / kChunk, lw)) return false;
        const RingBatch rows{ring, ring_addr(off, P.ring_chunks), rb, ring_bytes};
        float res[R][B];
        rows_dot<B, R>(rows, np, x, res);
        epi(r0, nr, res);
    }
    return true;
}

// Long rows at small batches stream through the ring in segments: a wave waits
// for kSegBytes of its row, accumulates them and frees them, so the four waves
// hold four segments rather than four whole rows (at 8 to 28 KB a row, most of
// the ring) and start on a row's first segment while the loader streams the rest.
// Each lane still accumulates its pieces in ascending order, so every row's value
// is the one rows_dot gives.  R = 2 (GATEUP): the wave takes the gate row, then
// the up row of its pair.
template <int B, int R, class Epi>
__device__ __forceinline__ bool gemv_ring_seg(const Params& P, Ctl* ctl, const char* ring, uint32_t S, uint32_t rb,
                                              uint32_t nrows, const XLds& x, int wave, uint32_t& lw, Epi& epi) {
    const uint32_t ring_bytes = P.ring_chunks * kChunk;
    const uint32_t np = rb >> 4, lane = (uint32_t)lane_id();
    constexpr uint32_t SP = kSegBytes / 16u;  // pieces per segment (a multiple of 64)
    for (uint32_t r0 = (uint32_t)wave * R; r0 < nrows; r0 += (uint32_t)R * kComputeWaves) {
        float res[R][B];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint32_t off = S + (r0 + (uint32_t)i) * rb;
            const RingBatch row{ring, ring_addr(off, P.ring_chunks), rb, ring_bytes};
            float acc[B];
#pragma unroll
            for (int b = 0; b < B; ++b) acc[b] = 0.f;
            for (uint32_t s0 = 0; s0 < np; s0 += SP) {
                const uint32_t s1 = min(np, s0 + SP);
                set_consumed(ctl, wave, (off + s0 * 16u) / kChunk);
                if (!wait_landed(P, ctl, (off + s1 * 16u + kChunk - 1u) / kChunk, lw)) return false;
#pragma unroll 2
                for (uint32_t p = s0 + lane; p < s1; p += 64u) {
                    const uint4 w = row.piece(0u, p);
                    float4 xa[B], xb[B];
#pragma unroll
                    for (int b = 0; b < B; ++b) x.piece(b, p, xa[b], xb[b]);
#pragma unroll
                    for (int b = 0; b < B; ++b) acc[b] = dot8(w, xa[b], xb[b], acc[b]);
                }
            }
            wave_total_n<B>(acc);
#pragma unroll
            for (int b = 0; b < B; ++b) res[i][b] = acc[b];
        }
        epi(r0, (uint32_t)R, res);
    }
    return true;
}

// Batch 1, rows of 64 NPL pieces (NPL = 4: 4 KB, the hidden size of 2048): each
// lane only ever reads the NPL pieces lane, lane + 64, ... of x, so they stay in
// registers for the whole instruction (32 floats), and a row batch reads only
// weights from the ring: all R x NPL pieces are requested at once, so a batch
// waits on the LDS once instead of once per piece pair.  Each lane accumulates
// its pieces in ascending order and wave_total reduces in its fixed tree: the
// same bits as rows_dot.  Used for the QKV and O rows; the (gate, up) pairs keep
// gemv_ring, which measured faster there (the pair stream is loader bound, and
// this loop's tighter polling of the ring slowed it).
template <int R, int NPL, class Epi>
__device__ __forceinline__ bool gemv_ring_xreg(const Params& P, Ctl* ctl, const char* ring, uint32_t S, uint32_t rb,
                                               uint32_t nrows, const XLds& x, int wave, uint32_t& lw, Epi& epi) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t ring_bytes = P.ring_chunks * kChunk;
    float4 xa[NPL], xb[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) x.piece(0, lane + 64u * (uint32_t)k, xa[k], xb[k]);
    for (uint32_t r0 = (uint32_t)wave * R; r0 < nrows; r0 += (uint32_t)R * kComputeWaves) {
        const uint32_t nr = min((uint32_t)R, nrows - r0);
        const uint32_t off = S + r0 * rb;
        set_consumed(ctl, wave, off / kChunk);
        if (!wait_landed(P, ctl, (off + nr * rb + kChunk - 1u) / kChunk, lw)) return false;
        const RingBatch rows{ring, ring_addr(off, P.ring_chunks), rb, ring_bytes};
        uint4 w[R][NPL];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int k = 0; k < NPL; ++k) w[i][k] = rows.piece((uint32_t)i, lane + 64u * (uint32_t)k);
        float acc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < NPL; ++k)
#pragma unroll
            for (int i = 0; i < R; ++i) acc[i] = dot8(w[i][k], xa[k], xb[k], acc[i]);
        wave_total_n<R>(acc);
        float res[R][1];
#pragma unroll
        for (int i = 0; i < R; ++i) res[i][0] = acc[i];
        epi(r0, nr, res);
    }
    return true;
}

// Batch size by row length; GATEUP keeps a (gate, up) pair inside one batch.
template <int B, class Epi>
__device__ __forceinline__ bool gemv_ring_auto(const Params& P, Ctl* ctl, const char* ring, uint32_t S, uint32_t rb,
                                               uint32_t nrows, const XLds& x, int wave, uint32_t& lw, Epi& epi,
                                               bool pairs) {
    if (segmented_rows(rb, B)) {
        if (pairs) return gemv_ring_seg<B, 2>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
        return gemv_ring_seg<B, 1>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
    }
    const int R = ring_batch_rows(rb, B, pairs);
    if constexpr (B == 1) {
        if (rb == 64u * 4u * 16u && R == 2 && !pairs)
            return gemv_ring_xreg<2, 4>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
    }
    if (R == 4) return gemv_ring<B, 4>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
    if (R == 2) return gemv_ring<B, 2>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
    return gemv_ring<B, 1>(P, ctl, ring, S, rb, nrows, x, wave, lw, epi);
}

// ------------------------------------------------------------------------------------------------
// LM head, streamed straight into registers by all eight waves of the CU (the
// four loader waves join the four compute waves).  The head has no dependency
// edge inside it, so the LDS ring, which exists to keep the weight stream going
// while instructions wait on other compute units, buys nothing here, and its
// coupling of loader and consumers capped the head near 4.5 TB/s.  Wave hw of 8
// takes rows hw, hw + 8, ... of the instruction in 4 KB segments; lane l loads
// pieces l, l + 64, l + 128, l + 192 of each segment with non-temporal loads,
// four segments ahead at batch 1, two at batch 2 and 8 (dense), one at batch 4 and
// for the MoE kernels at 8 (where the registers hold the batch's accumulators and
// activations; a second one measured 10 us slower per step at dense batch 4 and 17 us
// faster at dense batch 8), so 128 KB (64, 32 KB) stream per CU at once.  Each lane accumulates
// its pieces in ascending order and wave_total reduces in its fixed tree: the
// logits are bit for bit those of the ring GEMV (rows_dot).  The first segments
// are issued before `ready()`, which waits for the staged final-norm input and
// supplies its RMSNorm scales.  One instantiation serves every hidden size
// (segments per row at run time): one per size pushed the persistent kernel
// past its registers.
// ------------------------------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int B, bool MOE, class Ready>
__device__ __forceinline__ bool head_direct(const Params& P, const StepArgs& A, const float* xs, const Instr& in, int hw,
                                            Spin& spin, Ready& ready) {
    constexpr int NW = kComputeWaves + kLoaderWaves;
    constexpr int G = 4;  // pieces per lane of one 4 KB segment of a row
    constexpr int D = B == 1 ? 4 : (B == 4 || (MOE && B == 8)) ? 1 : 2;  // segments in flight per wave (measured)
    const uint32_t d = (uint32_t)P.d, np = d >> 3, lane = (uint32_t)lane_id();
    const uint32_t nseg = (np + 64u * G - 1u) / (64u * G);  // segments per row
    const uint32_t nrow = in.count > (uint32_t)hw ? (in.count - (uint32_t)hw + NW - 1u) / NW : 0u;
    const uint32_t nu = nrow * nseg;                          // this wave's (row, segment) units
    const uint4* base = (const uint4*)(P.head + ((size_t)in.begin + (uint32_t)hw) * d);
    const size_t row_stride = (size_t)NW * np;  // uint4 between this wave's consecutive rows
    uint4 w[D][G];
    // unit u = (row t, segment sg): pieces sg * 64 G + 64 g + lane of the row
    auto issue = [&](uint32_t u, uint4 (&dst)[G]) {
        const uint32_t t = u / nseg, sg = u - t * nseg;
        const uint4* rp = base + (size_t)t * row_stride;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t p = sg * (64u * G) + 64u * (uint32_t)g + lane;
            dst[g] = ld_nt16(rp + (p < np ? p : 0u));  // lanes past a short row re-read its start
        }
    };
    float r[B];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if ((uint32_t)i < nu) issue((uint32_t)i, w[i]);
    if (!ready(r)) return false;
    const XLds x{xs, d};
    float best_v[B], acc[B];
    int32_t best_i[B];
    bool nan_seen = false;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        best_v[b] = -INFINITY;
        best_i[b] = 0x7FFFFFFF;
        acc[b] = 0.f;
    }
    for (uint32_t u0 = 0; u0 < nu; u0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {  // (no break: w must stay register-indexed)
            const uint32_t u = u0 + (uint32_t)i;
            if (u < nu) {
                uint4 cur[G];
#pragma unroll
                for (int g = 0; g < G; ++g) cur[g] = w[i][g];
                if (u + D < nu) issue(u + D, w[i]);
                const uint32_t t = u / nseg, sg = u - t * nseg;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint32_t p = sg * (64u * G) + 64u * (uint32_t)g + lane;
                    if (p < np) {
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            float4 xa, xb;
                            x.piece(b, p, xa, xb);
                            acc[b] = dot8(cur[g], xa, xb, acc[b]);
                        }
                    }
                }
                if (sg + 1u == nseg) {  // the row is complete
                    wave_total_n<B>(acc);
                    const int32_t row = (int32_t)(in.begin + (uint32_t)hw + t * NW);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float v = acc[b] * r[b];
                        if (v != v) nan_seen = true;
                        if (head_better(v, row, best_v[b], best_i[b])) {
                            best_v[b] = v;
                            best_i[b] = row;
                        }
                    }
                    if (lane < B) A.logits[(size_t)lane * P.V + row] = pick<B>(acc, lane) * pick<B>(r, lane);
#pragma unroll
                    for (int b = 0; b < B; ++b) acc[b] = 0.f;
                }
            }
        }
    }
    if (nan_seen) {
#pragma unroll
        for (int b = 0; b < B; ++b) best_v[b] = __int_as_float(0x7FC00000);
    }
    return head_publish<B>(P, A, in.slot * (uint32_t)NW + (uint32_t)hw, best_v, best_i, spin);
}

// Matrix-core GEMV over one column slice of an instruction whose tile-major
// chunks start at stream byte S0.  Full groups: wave w owns tile 4 g + w and
// every k-unit of it.  The last group of m tiles is shared: wave w takes the
// units v = w, w + 4, ... (v = ku m + tile) and the four partial tiles are added
// in wave order through `red` (behind a barrier of the compute waves); a partial
// tile's unit has fewer chunks, and the rows past the end read whatever follows
// (their sums are never stored).  epi(t, v) gets tile t's sums (combine_parts
// layout).  Units are taken kMfmaBatchUnits at a time: one wait for the last of
// their chunks, all operand reads issued together, and alternate k-blocks go to
// two accumulators, so neither the LDS latency nor the accumulation chain is
// paid per k-block.
constexpr uint32_t kMfmaBatchKb = 8;
constexpr uint32_t kMfmaBatchUnits = kMfmaBatchKb >= kMfmaUnitKb ? kMfmaBatchKb / kMfmaUnitKb : 1u;

// Operand A of k-block e of the unit whose first chunk sits at ring slot s0 (of
// N): this lane's tile row r = l % 16 in chunk r / R, piece 4 e + l / 16 at its
// XOR-swizzled slot.
__device__ __forceinline__ uint4 unit_a(const char* ring, uint32_t s0, uint32_t N, uint32_t e) {
    const uint32_t l = (uint32_t)lane_id(), r = l & 15u, p = e * 4u + (l >> 4);
    uint32_t ci = s0 + r / kMfmaChunkRows;
    ci = ci >= N ? ci - N : ci;
    const uint32_t slot = (r % kMfmaChunkRows) * kMfmaPiecesPerRow + (p ^ (r % kMfmaPiecesPerRow));
    return *(const uint4*)(ring + ci * kChunk + slot * 16u);
}

template <int B, int PRT, class Epi>
__device__ __forceinline__ bool gemv_mfma_ring(const Params& P, Ctl* ctl, const char* ring, uint32_t S0,
                                               const MfmaGeo& g, const char* area, char* red, int wave, uint32_t& lw,
                                               Epi& epi, CwBarrier& barrier) {
    constexpr uint32_t PB = (uint32_t)(PRT * B), PBP = (uint32_t)parts_pitch(B);
    constexpr uint32_t U = kMfmaBatchUnits, KBU = kMfmaUnitKb, NC = kMfmaUnitChunks;
    const uint32_t c0 = S0 / kChunk, N = P.ring_chunks;
    for (uint32_t grp = 0; grp < g.G4; ++grp) {
        floatx4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0;
        const uint32_t cb = c0 + NC * (grp * 4u * g.KU + (uint32_t)wave);  // first chunk of k-unit 0
        for (uint32_t k0 = 0; k0 < g.KU; k0 += U) {
            const uint32_t n = min(U, g.KU - k0);
            set_consumed(ctl, wave, cb + k0 * 4u * NC);
            if (!wait_landed(P, ctl, cb + (k0 + n - 1u) * 4u * NC + NC, lw)) return false;
            uint4 a[U * KBU];
            bf16x8_t b[U * KBU];
#pragma unroll
            for (uint32_t u = 0; u < U; ++u)
                if (u < n) {
                    const uint32_t s0 = (cb + (k0 + u) * 4u * NC) % N;
#pragma unroll
                    for (uint32_t e = 0; e < KBU; ++e) {
                        a[u * KBU + e] = unit_a(ring, s0, N, e);
                        b[u * KBU + e] = load_parts(area, (k0 + u) * KBU + e, PB, PBP);
                    }
                }
#pragma unroll
            for (uint32_t u = 0; u < U; ++u)
                if (u < n) {
#pragma unroll
                    for (uint32_t e = 0; e < KBU; ++e) {
                        if (e & 1u) d1 = mfma_acc(a[u * KBU + e], b[u * KBU + e], d1);
                        else d0 = mfma_acc(a[u * KBU + e], b[u * KBU + e], d0);
                    }
                }
        }
        epi(grp * 4u + (uint32_t)wave, combine_parts<PRT>(d0 + d1));
    }
    const uint32_t m = g.m;
    if (m) {
        floatx4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0, d2 = d0, d3 = d0;
        const uint32_t base = c0 + g.full_chunks(), total = m * g.KU;  // units of the last group
        // first chunk and chunk count of unit v (k-unit v / m, tile v % m)
        auto ustart = [&](uint32_t v, uint32_t& cnt) -> uint32_t {
            const uint32_t ku = v / m, t = v - ku * m;
            cnt = min(NC, g.CR - t * NC);
            return base + ku * g.CR + t * NC;
        };
        for (uint32_t v0 = (uint32_t)wave; v0 < total; v0 += 4u * U) {
            const uint32_t n = min(U, (total - v0 + 3u) / 4u);  // units v0, v0 + 4, ... below total
            uint32_t cnt0, cntl;
            const uint32_t first = ustart(v0, cnt0), lastc = ustart(v0 + 4u * (n - 1u), cntl);
            set_consumed(ctl, wave, first);
            if (!wait_landed(P, ctl, lastc + cntl, lw)) return false;
            uint4 a[U * KBU];
            bf16x8_t b[U * KBU];
#pragma unroll
            for (uint32_t i = 0; i < U; ++i)
                if (i < n) {
                    const uint32_t v = v0 + 4u * i, ku = v / m;
                    uint32_t cnt;
                    const uint32_t s0 = ustart(v, cnt) % N;
#pragma unroll
                    for (uint32_t e = 0; e < KBU; ++e) {
                        a[i * KBU + e] = unit_a(ring, s0, N, e);
                        b[i * KBU + e] = load_parts(area, ku * KBU + e, PB, PBP);
                    }
                }
#pragma unroll
            for (uint32_t i = 0; i < U; ++i)
                if (i < n) {
                    const uint32_t v = v0 + 4u * i, t = v - (v / m) * m;
                    floatx4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
#pragma unroll
                    for (uint32_t e = 0; e < KBU; ++e) {
                        if (e & 1u) x1 = mfma_acc(a[i * KBU + e], b[i * KBU + e], x1);
                        else x0 = mfma_acc(a[i * KBU + e], b[i * KBU + e], x0);
                    }
                    const floatx4_t x = x0 + x1;
                    if (t == 0) d0 += x;
                    else if (t == 1) d1 += x;
                    else if (t == 2) d2 += x;
                    else d3 += x;
                }
        }
        red_store<B, PRT>(red, wave, 0, combine_parts<PRT>(d0));
        if (m > 1) red_store<B, PRT>(red, wave, 1, combine_parts<PRT>(d1));
        if (m > 2) red_store<B, PRT>(red, wave, 2, combine_parts<PRT>(d2));
        if (m > 3) red_store<B, PRT>(red, wave, 3, combine_parts<PRT>(d3));
        release_region(ctl, wave, (c0 + g.slice_chunks()) * kChunk);  // before the barrier: no wave may hold the slice
        if (!barrier()) return false;
        if ((uint32_t)wave < m) epi(4u * g.G4 + (uint32_t)wave, red_sum<B, PRT>(red, (uint32_t)wave));
    }
    release_region(ctl, wave, (c0 + g.slice_chunks()) * kChunk);
    return true;
}

// Lane of a combined tile: holds rows 4 (lane / 16) + r of batch row b when it is
// the part-0 lane of b (column PRT b).
template <int B, int PRT>
__device__ __forceinline__ bool mfma_lane(int& b, uint32_t& row4) {
    const uint32_t l = (uint32_t)lane_id(), j = l & 15u;
    b = (int)(j / (uint32_t)PRT);
    row4 = (l >> 4) * 4u;
    return j % (uint32_t)PRT == 0u && j < (uint32_t)(PRT * B);
}

// One GEMV instruction (QKV, O, GATEUP, DOWN or the LM head) on the matrix cores:
// the staged activations land as bf16 parts at the start of the activation
// area, the cross-wave partial tiles at its end.  Same epilogues as the VALU
// path; each used lane of a combined tile owns four consecutive rows of one
// batch row.
template <int B, int HD>
__device__ __forceinline__ bool mfma_instr(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                        int wave, const Instr& in, uint32_t S, Spin& spin, CwBarrier& barrier,
                                        uint32_t& land_wait, uint32_t* tr) {
    constexpr int PRT = mfma_parts(B);
    constexpr uint32_t PB = (uint32_t)(PRT * B);
    const int lane = lane_id();
    const int layer = in.layer;
    const DevLayer Lw = ld_const(P.layers + (layer < P.L ? layer : 0));
    char* area = (char*)xs;
    char* red = (char*)xs + P.x_bytes - mfma_red_bytes(B);
    const MfmaGeo g = mfma_geo<HD>(P, in);
    int lb;
    uint32_t row4;
    const bool lane_ok = mfma_lane<B, PRT>(lb, row4);
    lb = lb < B ? lb : B - 1;
    if (in.op == OP_O || in.op == OP_DOWN) {
        const bool is_o = in.op == OP_O;
        const uint32_t K = is_o ? (uint32_t)(P.Hq * HD) : (uint32_t)P.F;
        const uint32_t tag_x = is_o ? phase_tag(A.tag0, layer, 1) : phase_tag(A.tag0, layer, 3);
        const uint32_t tag_res = is_o ? phase_tag(A.tag0, layer - 1, 4) : phase_tag(A.tag0, layer, 2);
        const uint32_t tag_out = is_o ? phase_tag(A.tag0, layer, 2) : phase_tag(A.tag0, layer, 4);
        const uint32_t ns = g.slices, Ks = K / ns;
        float* hres = (float*)(area + parts_bytes(B, (int)Ks));  // [B][count] residual rows
        float* part = hres + B * in.count;                        // [B][count] partial sums
        for (uint32_t ks = 0; ks < ns; ++ks) {
            if (ks > 0 && !barrier()) return false;
            float ss[1] = {0.f};
            const StageSeg sx = {(is_o ? P.attn : P.act) + ks * Ks, (float*)area, nullptr, Ks, (uint32_t)B, K, Ks,
                                 tag_x, (uint32_t)PRT};
            if (ks > 0) {
                const StageSeg sg[1] = {sx};
                if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
            } else if (is_o && layer == 0) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    stage_bf16(P.embed + token_row(A, b, P.V) * P.d + in.begin, in.count,
                               hres + b * in.count, nullptr, wave, kComputeWaves, ss[0]);
                const StageSeg sg[1] = {sx};
                if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
            } else {
                const StageSeg sg[2] = {sx, {P.h + in.begin, hres, nullptr, in.count, (uint32_t)B, (uint32_t)P.d,
                                             in.count, tag_res, 0u}};
                if (!stage_segs<kStagePassWordsWide, 1, 2>(sg, wave, kComputeWaves, spin, ss)) return false;
            }
            if (!barrier()) return false;
            if (tr && lane == 0 && ks == 0) tr[2] = (uint32_t)now_ticks();
            const bool last = ks + 1 == ns;
            auto epi = [&](uint32_t t, floatx4_t v) {
                if (!lane_ok) return;
#pragma unroll
                for (uint32_t r = 0; r < 4u; ++r) {
                    const uint32_t j = t * 16u + row4 + r;
                    if (j < in.count) {
                        float x = v[r];
                        if (ks > 0) x = part[lb * in.count + j] + x;
                        if (!last) part[lb * in.count + j] = x;
                        else st_tagged(P.h + (size_t)lb * P.d + in.begin + j, hres[lb * in.count + j] + x, tag_out);
                    }
                }
            };
            if (!gemv_mfma_ring<B, PRT>(P, ctl, ring, S + ks * g.slice_chunks() * kChunk, g, area, red, wave, land_wait,
                                        epi, barrier))
                return false;
        }
        return true;
    }
    // QKV, GATEUP, HEAD: RMSNorm of the residual stream, then the rows
    const uint16_t* gain = in.op == OP_QKV ? Lw.attn_norm : in.op == OP_GATEUP ? Lw.mlp_norm : P.final_norm;
    const uint32_t tag_in = in.op == OP_QKV      ? phase_tag(A.tag0, layer - 1, 4)
                            : in.op == OP_GATEUP ? phase_tag(A.tag0, layer, 2)
                                                 : phase_tag(A.tag0, P.L - 1, 4);
    const uint32_t d = (uint32_t)P.d;
    float ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = 0.f;
    if (in.op == OP_QKV && layer == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b)
            stage_bf16_parts<PRT>(P.embed + token_row(A, b, P.V) * d, d, area, (uint32_t)b,
                                  (uint32_t)parts_pitch(B), gain, wave, kComputeWaves, ss[b]);
    } else {
        const StageSeg sg[1] = {{P.h, (float*)area, gain, d, (uint32_t)B, d, d, tag_in, (uint32_t)PRT}};
        if (!stage_segs<kStagePassWords, B, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
    }
    wave_total_n<B>(ss);
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) ctl->ss[b][wave] = ss[b];
    }
    if (!barrier()) return false;
    float r[B];
#pragma unroll
    for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
    const float rl = pick<B>(r, lb);
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    if (in.op == OP_QKV) {
        const uint32_t tag_out = phase_tag(A.tag0, layer, 0);
        auto epi = [&](uint32_t t, floatx4_t v) {
            if (!lane_ok) return;
#pragma unroll
            for (uint32_t rr = 0; rr < 4u; ++rr) {
                const uint32_t j = t * 16u + row4 + rr;
                if (j < g.nrows) st_tagged(P.qkv + (size_t)lb * P.qkv_rows + in.begin + j, v[rr] * rl, tag_out);
            }
        };
        return gemv_mfma_ring<B, PRT>(P, ctl, ring, S, g, area, red, wave, land_wait, epi, barrier);
    }
    if (in.op == OP_GATEUP) {
        const uint32_t tag_out = phase_tag(A.tag0, layer, 3);
        auto epi = [&](uint32_t t, floatx4_t v) {
            if (!lane_ok) return;
#pragma unroll
            for (uint32_t pr = 0; pr < 2u; ++pr) {
                const uint32_t j = t * 16u + row4 + 2u * pr;  // gate row j, up row j + 1
                if (j + 1u < g.nrows)
                    st_tagged(P.act + (size_t)lb * P.F + in.begin + j / 2u,
                              silu_mul(v[2 * pr] * rl, v[2 * pr + 1] * rl), tag_out);
            }
        };
        return gemv_mfma_ring<B, PRT>(P, ctl, ring, S, g, area, red, wave, land_wait, epi, barrier);
    }
    // LM head: logits, and each lane's best row of its batch row
    float bv = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    bool nan_seen = false;
    auto epi = [&](uint32_t t, floatx4_t v) {
        if (!lane_ok) return;
#pragma unroll
        for (uint32_t rr = 0; rr < 4u; ++rr) {
            const uint32_t j = t * 16u + row4 + rr;
            if (j < g.nrows) {
                const float x = v[rr] * rl;
                const int32_t row = (int32_t)(in.begin + j);
                if (x != x) nan_seen = true;
                if (head_better(x, row, bv, bi)) {
                    bv = x;
                    bi = row;
                }
                A.logits[(size_t)lb * P.V + row] = x;
            }
        }
    };
    if (!gemv_mfma_ring<B, PRT>(P, ctl, ring, S, g, area, red, wave, land_wait, epi, barrier)) return false;
    // the four lanes of a column (lane % 16) hold disjoint rows of one batch row
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
        const float ov = __shfl_xor(bv, msk, 64);
        const int32_t oi = __shfl_xor(bi, msk, 64);
        if (head_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    float best_v[B];
    int32_t best_i[B];
    const bool any_nan = __any(nan_seen);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        best_v[b] = any_nan ? __int_as_float(0x7FC00000)
                            : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), PRT * b));
        best_i[b] = __builtin_amdgcn_readlane(bi, PRT * b);
    }
    return head_publish<B>(P, A, in.slot * kComputeWaves + (uint32_t)wave, best_v, best_i, spin);
}

// ------------------------------------------------------------------------------------------------
// MoE FFN (the synthetic MoE decoder's layers): router logits (OP_ROUTE), then on
// every CU the selected experts' (gate, up) rows of its f-range (OP_EGU) and
// their down rows of its output rows (OP_EDOWN).  Each CU routes for itself from
// the router logits, so every CU derives the same selected set; only the
// selected experts' rows are streamed.
// ------------------------------------------------------------------------------------------------

// Top-k routing of one sequence; lane e < E holds the router logit of expert e.
// Probabilities are the softmax evaluated in double and rounded to fp32; the k
// largest are selected, ties to the lower expert index (NaN never wins).
// Returns the selected-expert mask; `prob` = this lane's probability.
__device__ __forceinline__ uint64_t route_topk(float z, int E, int K, float& prob) {
    const int lane = lane_id();
    const bool valid = lane < E;
    float m = valid ? z : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const double ex = valid ? exp((double)z - (double)m) : 0.0;
    double Z = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Z += __shfl_xor(Z, o, 64);
    prob = valid ? (float)(ex / Z) : -1.0f;
    const uint64_t valid_mask = E >= 64 ? ~0ull : ((1ull << E) - 1ull);
    uint64_t sel = 0;
    for (int t = 0; t < K; ++t) {
        const float v = ((sel >> lane) & 1ull) || !valid ? -2.0f : prob;
        float best = v;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) best = fmaxf(best, __shfl_xor(best, o, 64));
        uint64_t cand = __ballot(v == best) & valid_mask & ~sel;
        if (!cand) cand = valid_mask & ~sel;  // NaN probabilities: the lowest index not yet taken
        sel |= 1ull << __builtin_ctzll(cand);
    }
    return sel;
}

// Routes the B sequences from the router logits at zeta [B][E] (LDS); returns the
// union of the selected sets and, per sequence, the mask and this lane's
// probability.  Wave 0 publishes the expert-table slots of the union (shared
// first) for the loaders and the other waves; the caller's barrier orders it.
template <int B>
__device__ __forceinline__ uint32_t moe_route(const Params& P, Ctl* ctl, const float* zeta, int wave, uint32_t qi,
                                              uint64_t (&sel)[B], float (&prob)[B]) {
    const int lane = lane_id();
    uint64_t U = 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float z = lane < P.E ? zeta[b * P.E + lane] : 0.f;
        sel[b] = route_topk(z, P.E, P.top_k, prob[b]);
        U |= sel[b];
    }
    const uint32_t n = (uint32_t)P.n_shared + (uint32_t)__builtin_popcountll(U);
    if (wave == 0 && lane == 0) {
        uint32_t a = 0;
        for (int x = 0; x < P.n_shared; ++x) ctl->moe_list[a++] = (uint8_t)x;
        for (uint64_t u = U; u; u &= u - 1ull) ctl->moe_list[a++] = (uint8_t)(P.n_shared + __builtin_ctzll(u));
        ctl->moe_n = n;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        lds_st(&ctl->moe_seq, qi + 1u);
    }
    return n;
}

// OP_EGU: x = RMSNorm(h after O) * g; route; then for every selected slot the
// CU's (gate, up) row pairs of f-range [begin, begin + count): SwiGLU outputs.
template <int B>
__device__ __forceinline__ bool moe_egu(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                        int wave, const Instr& in, uint32_t qi, uint32_t S, Spin& spin,
                                        CwBarrier& barrier, uint32_t& land_wait, uint32_t* tr, uint32_t& bytes) {
    const int lane = lane_id();
    const int layer = in.layer;
    const DevLayer Lw = ld_const(P.layers + layer);
    const uint32_t d = (uint32_t)P.d, E = (uint32_t)P.E;
    const uint32_t tag_o = phase_tag(A.tag0, layer, 2);
    float* zeta = xs + B * d;
    float ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = 0.f;
    const StageSeg sg[2] = {{P.h, xs, Lw.mlp_norm, d, (uint32_t)B, d, d, tag_o, 0u},
                            {P.route, zeta, nullptr, E, (uint32_t)B, E, E, tag_o, 0u}};
    if (!stage_segs<stage_words<B>(), B, 2>(sg, wave, kComputeWaves, spin, ss)) return false;
    wave_total_n<B>(ss);
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) ctl->ss[b][wave] = ss[b];
    }
    if (!barrier()) return false;
    float r[B];
#pragma unroll
    for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
    uint64_t sel[B];
    float prob[B];
    const uint32_t n = moe_route<B>(P, ctl, zeta, wave, qi, sel, prob);
    // the instruction holding the layer's first expert rows counts the slots the
    // layer streams (every CU derives the same set)
    if (in.begin == 0 && wave == 0 && lane == 0)
        __hip_atomic_fetch_add(&P.state->moe_slots, (unsigned long long)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!barrier()) return false;  // the slot list is visible
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    bytes = moe_bytes(P, in, n);
    const uint32_t per = 2u * in.count, tag_out = phase_tag(A.tag0, layer, 3);
    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
        #pragma unroll
        for (uint32_t i = 0; i + 1 < (uint32_t)(sizeof(res) / sizeof(res[0])); i += 2) {
            if (i + 1 >= nr) break;
            const uint32_t j = r0 + i, a = j / per, f = in.begin + (j - a * per) / 2u;
            const uint32_t x = ctl->moe_list[a];
            if (lane < B) {
                const float rr = pick<B>(r, lane);
                st_tagged(P.eact + ((size_t)x * P.B + lane) * P.Fe + f,
                          silu_mul(pick<B>(res[i], lane) * rr, pick<B>(res[i + 1], lane) * rr), tag_out);
            }
        }
    };
    return gemv_ring_auto<B>(P, ctl, ring, S, d * 2u, n * per, XLds{xs, d}, wave, land_wait, epi, true);
}

// QKV or router rows over column slices of their RMSNorm input (MoE models whose
// B x hidden fp32 input does not fit next to the weight ring: hidden 4096 at batch
// 8).  Per slice the compute waves stage h * g of the slice (the sums of squares
// accumulate over the slices) and add every row's dot product over the slice to
// its partial sum in LDS; after the last slice the rows are scaled by the RMSNorm
// factor and stored.  The stream is slice-major (the rows' first slices, then
// their second, ...).  The dot product of a row is the slice sums added in slice
// order: the same value as the unsliced GEMV up to fp32 rounding order.
template <int B>
__device__ __forceinline__ bool norm_gemv_sliced(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring,
                                                 float* xs, int wave, const Instr& in, uint32_t S, Spin& spin,
                                                 CwBarrier& barrier, uint32_t& land_wait, uint32_t* tr) {
    const int lane = lane_id();
    const int layer = in.layer;
    const DevLayer Lw = ld_const(P.layers + layer);
    const bool qkv = in.op == OP_QKV;
    const uint16_t* gain = uniform_p(qkv ? Lw.attn_norm : Lw.mlp_norm);
    const uint32_t tag_in = qkv ? phase_tag(A.tag0, layer - 1, 4) : phase_tag(A.tag0, layer, 2);
    const uint32_t tag_out = qkv ? phase_tag(A.tag0, layer, 0) : phase_tag(A.tag0, layer, 2);
    const uint32_t d = (uint32_t)P.d, ns = (uint32_t)P.x_slices, Ks = d / ns, cnt = in.count;
    float* part = xs + B * Ks;  // [B][cnt] partial sums
    float ss[B], r[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = r[b] = 0.f;
    for (uint32_t ks = 0; ks < ns; ++ks) {
        if (ks > 0 && !barrier()) return false;  // every wave is done with the previous slice
        if (qkv && layer == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b)
                stage_bf16(P.embed + token_row(A, b, P.V) * d + ks * Ks, Ks, xs + b * Ks,
                           gain + ks * Ks, wave, kComputeWaves, ss[b]);
        } else {
            const StageSeg sg[1] = {{P.h + ks * Ks, xs, gain + ks * Ks, Ks, (uint32_t)B, d, Ks, tag_in}};
            if (!stage_segs<stage_words<B>(), B, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
        }
        const bool last = ks + 1 == ns;
        if (last) {
            wave_total_n<B>(ss);
            if (lane == 0) {
#pragma unroll
                for (int b = 0; b < B; ++b) ctl->ss[b][wave] = ss[b];
            }
        }
        if (!barrier()) return false;
        if (tr && lane == 0 && ks == 0) tr[2] = (uint32_t)now_ticks();
        if (last) {
#pragma unroll
            for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
        }
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i) {
                if (i >= nr) break;
                const uint32_t j = r0 + i;
                if (lane < B) {
                    float v = pick<B>(res[i], lane);
                    if (ks > 0) v = part[lane * cnt + j] + v;
                    if (!last) {
                        part[lane * cnt + j] = v;
                    } else {
                        uint64_t* dst = qkv ? P.qkv + (size_t)lane * P.qkv_rows : P.route + (size_t)lane * P.E;
                        st_tagged(dst + in.begin + j, v * pick<B>(r, lane), tag_out);
                    }
                }
            }
        };
        if (!gemv_ring_auto<B>(P, ctl, ring, S + ks * cnt * Ks * 2u, Ks * 2u, cnt, XLds{xs, Ks}, wave, land_wait, epi,
                               false))
            return false;
        release_region(ctl, wave, S + (ks + 1u) * cnt * Ks * 2u);
    }
    return true;
}

// OP_EGU over column slices of x (see norm_gemv_sliced): slice 0 also stages the
// router logits and routes; per slice every selected slot's (gate, up) row pairs
// add their dot products over the slice to partial sums in LDS; after the last
// slice the SwiGLU outputs are stored.  The stream is slice-major over the slots.
template <int B>
__device__ __forceinline__ bool moe_egu_sliced(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring,
                                               float* xs, int wave, const Instr& in, uint32_t qi, uint32_t S,
                                               Spin& spin, CwBarrier& barrier, uint32_t& land_wait, uint32_t* tr,
                                               uint32_t& bytes) {
    const int lane = lane_id();
    const int layer = in.layer;
    const DevLayer Lw = ld_const(P.layers + layer);
    const uint32_t d = (uint32_t)P.d, E = (uint32_t)P.E, ns = (uint32_t)P.x_slices, Ks = d / ns;
    const uint32_t tag_o = phase_tag(A.tag0, layer, 2), tag_out = phase_tag(A.tag0, layer, 3);
    const uint16_t* gain = uniform_p(Lw.mlp_norm);
    float* zeta = xs + B * Ks;     // [B][E] router logits
    float* part = zeta + B * E;    // [row][B] partial sums of every selected slot's rows
    const uint32_t per = 2u * in.count;
    float ss[B], r[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = r[b] = 0.f;
    uint32_t n = 0;
    for (uint32_t ks = 0; ks < ns; ++ks) {
        if (ks > 0 && !barrier()) return false;  // every wave is done with the previous slice
        const StageSeg sx = {P.h + ks * Ks, xs, gain + ks * Ks, Ks, (uint32_t)B, d, Ks, tag_o, 0u};
        if (ks == 0) {
            const StageSeg sg[2] = {sx, {P.route, zeta, nullptr, E, (uint32_t)B, E, E, tag_o, 0u}};
            if (!stage_segs<stage_words<B>(), B, 2>(sg, wave, kComputeWaves, spin, ss)) return false;
        } else {
            const StageSeg sg[1] = {sx};
            if (!stage_segs<stage_words<B>(), B, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
        }
        const bool last = ks + 1 == ns;
        if (last) {
            wave_total_n<B>(ss);
            if (lane == 0) {
#pragma unroll
                for (int b = 0; b < B; ++b) ctl->ss[b][wave] = ss[b];
            }
        }
        if (!barrier()) return false;
        if (ks == 0) {
            uint64_t sel[B];
            float prob[B];
            n = moe_route<B>(P, ctl, zeta, wave, qi, sel, prob);
            if (in.begin == 0 && wave == 0 && lane == 0)
                __hip_atomic_fetch_add(&P.state->moe_slots, (unsigned long long)n, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (!barrier()) return false;  // the slot list is visible
            if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
            bytes = moe_bytes(P, in, n);
        }
        if (last) {
#pragma unroll
            for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
        }
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i + 1 < (uint32_t)(sizeof(res) / sizeof(res[0])); i += 2) {
                if (i + 1 >= nr) break;
                const uint32_t j = r0 + i;
                if (lane < B) {
                    float g = pick<B>(res[i], lane), u = pick<B>(res[i + 1], lane);
                    if (ks > 0) {
                        g = part[j * B + lane] + g;
                        u = part[(j + 1u) * B + lane] + u;
                    }
                    if (!last) {
                        part[j * B + lane] = g;
                        part[(j + 1u) * B + lane] = u;
                    } else {
                        const uint32_t a = j / per, f = in.begin + (j - a * per) / 2u;
                        const uint32_t x = ctl->moe_list[a];
                        const float rr = pick<B>(r, lane);
                        st_tagged(P.eact + ((size_t)x * P.B + lane) * P.Fe + f, silu_mul(g * rr, u * rr), tag_out);
                    }
                }
            }
        };
        const uint32_t sl = n * per * Ks * 2u;  // stream bytes of one slice over every slot
        if (!gemv_ring_auto<B>(P, ctl, ring, S + ks * sl, Ks * 2u, n * per, XLds{xs, Ks}, wave, land_wait, epi, true))
            return false;
        release_region(ctl, wave, S + (ks + 1u) * sl);
    }
    return true;
}

// OP_EPART: route again (same logits, same result; the loader waits for the slot
// list, so the weight stream starts before the SwiGLU outputs are ready); then for
// each selected slot a in the CU's share of the (slot, down row) pairs: stage the
// slot's SwiGLU rows and store the unweighted down rows' outputs epart[a][b][row].
// A CU stages the inputs of the few slots its share touches, not of every slot.
template <int B>
__device__ __forceinline__ bool moe_epart(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                          int wave, const Instr& in, uint32_t qi, uint32_t S, Spin& spin,
                                          CwBarrier& barrier, uint32_t& land_wait, uint32_t* tr, uint32_t& bytes) {
    const int lane = lane_id();
    const int layer = in.layer;
    const uint32_t E = (uint32_t)P.E, Fe = (uint32_t)P.Fe, d = (uint32_t)P.d;
    const uint32_t tag_o = phase_tag(A.tag0, layer, 2), tag_a = phase_tag(A.tag0, layer, 3);
    float* zeta = xs + B * Fe;  // [B][E] router logits, after one slot's SwiGLU rows
    {
        float ss[1] = {0.f};
        const StageSeg sg[1] = {{P.route, zeta, nullptr, E, (uint32_t)B, E, E, tag_o, 0u}};
        if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
    }
    if (!barrier()) return false;
    uint32_t n;
    {
        uint64_t sel[B];
        float prob[B];
        n = moe_route<B>(P, ctl, zeta, wave, qi, sel, prob);
    }
    if (!barrier()) return false;  // the slot list is visible
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    uint32_t t0, t1;
    moe_part_range(n, d, P.n_cu, (int)in.begin, &t0, &t1);
    bytes = (t1 - t0) * Fe * 2u;
    const uint32_t rb = Fe * 2u;
    uint32_t off = S;
    for (uint32_t t = t0; t < t1;) {
        const uint32_t a = t / d, i0 = t - a * d, nr = min(d, t1 - a * d) - i0;
        const uint32_t x = __builtin_amdgcn_readfirstlane((uint32_t)ctl->moe_list[a]);
        if (t > t0 && !barrier()) return false;  // every wave is done with the previous slot's rows
        float ss[1] = {0.f};
        const StageSeg sa[1] = {{P.eact + (size_t)x * P.B * Fe, xs, nullptr, Fe, (uint32_t)B, Fe, Fe, tag_a, 0u}};
        if (!stage_segs<kStagePassWordsWide, 1, 1>(sa, wave, kComputeWaves, spin, ss)) return false;
        if (!barrier()) return false;
        uint64_t* dst = P.epart + (size_t)a * B * d + i0;
        auto epi = [&](uint32_t r0, uint32_t nrr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i) {
                if (i >= nrr) break;
                if (lane < B) st_tagged(dst + (size_t)lane * d + r0 + i, pick<B>(res[i], lane), tag_a);
            }
        };
        if (!gemv_ring_auto<B>(P, ctl, ring, off, rb, nr, XLds{xs, Fe}, wave, land_wait, epi, false)) return false;
        off += nr * rb;
        release_region(ctl, wave, off);
        t += nr;
    }
    return true;
}

// Stages rows [0, nrows) x columns [0, cnt) (cnt <= 16) of the tagged words at
// src (row stride `stride` words) into dst [nrows][cnt] once each carries `tag`.
// Lane l of compute wave w takes column l % 16 of rows 4 w + l / 16 + 16 k: K
// rows per lane per pass, any number of rows (the generic staging resolves at
// most kMaxBatch rows per segment).
// OP_EDOWN: route again; for output rows [begin, begin + count) stage every
// selected slot's outputs (epart) and add them in slot order (shared, then
// ascending experts), weighted by the sequence's probability (1 for the shared
// expert; slots the sequence did not select are skipped); then h += the sum.
template <int B>
__device__ __forceinline__ bool moe_ered(const Params& P, const StepArgs& A, Ctl* ctl, float* xs, int wave,
                                         const Instr& in, uint32_t qi, Spin& spin, CwBarrier& barrier, uint32_t* tr) {
    const int lane = lane_id();
    const int layer = in.layer;
    const uint32_t E = (uint32_t)P.E, d = (uint32_t)P.d, cnt = in.count;
    const uint32_t tag_o = phase_tag(A.tag0, layer, 2), tag_a = phase_tag(A.tag0, layer, 3);
    const uint32_t smax = (uint32_t)P.n_shared + min(E, (uint32_t)(B * P.top_k));
    float* zeta = xs;                    // [B][E] router logits
    float* wtab = zeta + B * E;          // [slot][B] weights of the selected slots
    float* hres = wtab + (smax + 1u) * B;  // [B][cnt] residual rows after O
    float* part = hres + B * cnt;        // [slot][B][cnt] the slots' outputs of the rows
    {
        float ss[1] = {0.f};
        const StageSeg sg[2] = {{P.route, zeta, nullptr, E, (uint32_t)B, E, E, tag_o, 0u},
                                {P.h + in.begin, hres, nullptr, cnt, (uint32_t)B, d, cnt, tag_o, 0u}};
        if (!stage_segs<kStagePassWordsWide, 1, 2>(sg, wave, kComputeWaves, spin, ss)) return false;
    }
    if (!barrier()) return false;
    uint32_t n;
    {
        uint64_t sel[B];
        float prob[B];
        n = moe_route<B>(P, ctl, zeta, wave, qi, sel, prob);
        if (wave == 0) {
            // weight of slot a for sequence b: 1 (shared), its probability where b
            // selected the expert, else 0; lane e writes expert e's slot
            uint64_t U = 0;
#pragma unroll
            for (int b = 0; b < B; ++b) U |= sel[b];
            const bool mine = lane < P.E && ((U >> lane) & 1ull);
            const uint32_t slot = (uint32_t)P.n_shared + (uint32_t)__builtin_popcountll(U & ((1ull << lane) - 1ull));
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (mine) wtab[slot * B + b] = ((sel[b] >> lane) & 1ull) ? prob[b] : 0.f;
                if (lane < P.n_shared) wtab[lane * B + b] = 1.0f;
            }
        }
    }
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    // row a * B + b of the staged outputs is epart row a * B + b
    if (!stage_grid<kStagePassWordsWide>(nullptr, 0u, 0u, P.epart + in.begin, n * (uint32_t)B, tag_a, d, cnt, part,
                                         wave, kComputeWaves, spin))
        return false;
    if (!barrier()) return false;  // the weights and the staged outputs are visible
    const uint32_t tag_out = phase_tag(A.tag0, layer, 4);
    for (uint32_t i = (uint32_t)(wave * 64 + lane); i < B * cnt; i += 64u * kComputeWaves) {
        const uint32_t b = i / cnt, j = i - b * cnt;
        float acc = 0.f;
        for (uint32_t a = 0; a < n; ++a) {
            const float wv = wtab[a * B + b];
            if (wv != 0.f) acc += wv * part[(a * B + b) * cnt + j];
        }
        st_tagged(P.h + (size_t)b * d + in.begin + j, hres[i] + acc, tag_out);
    }
    return true;
}

// Transposed Wdown rows of an OP_DPART instruction in the ring: get(f, q) gives
// this lane's 16 bytes of rows f .. f + kDpartRowsPerGet - 1 of the current part
// (rows taken in order from f = 0; `cur` is the ring byte of the lane's piece of
// the next row), once they have landed; the wave's mark moves to row f first.
struct DpartRingRows {
    const Params* P;
    Ctl* ctl;
    const char* ring;
    uint32_t base, rb, ring_bytes, cur;  // stream byte of the part's first row, row bytes, ring bytes
    int wave;
    bool on;  // the lane has outputs (its piece lies inside the row)
    uint32_t* lw;
    __device__ __forceinline__ bool get(uint32_t f, uint4 (&q)[kDpartRowsPerGet]) {
        const uint32_t s0 = base + f * rb;
        set_consumed(ctl, wave, s0 / kChunk);
        if (!wait_landed(*P, ctl, (s0 + (uint32_t)kDpartRowsPerGet * rb + kChunk - 1u) / kChunk, *lw)) return false;
#pragma unroll
        for (int u = 0; u < kDpartRowsPerGet; ++u) {
            q[u] = on ? *(const uint4*)(ring + cur) : make_uint4(0u, 0u, 0u, 0u);
            cur += rb;
            if (cur >= ring_bytes) cur -= ring_bytes;
        }
        return true;
    }
};

// OP_DPART (split down projection): parts [begin, begin + count) of F.  The
// compute waves stage the parts' SwiGLU inputs (a CU's parts are normally its own
// GATEUP outputs: no wait on other CUs), then every wave reads every transposed
// row of the parts from the ring, lane l of wave w the outputs 8 (64 w + l) ..
// + 7; each part's partial outputs of all rows go through LDS to dpart[part][b][row],
// tagged (dpart_store).
template <int B>
__device__ __forceinline__ bool dpart_instr(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                            int wave, const Instr& in, uint32_t S, Spin& spin, CwBarrier& barrier,
                                            uint32_t& land_wait, uint32_t* tr) {
    const int lane = lane_id();
    const uint32_t d = (uint32_t)P.d, np = in.count, nf = np * kDownPart, f0 = in.begin * kDownPart;
    const uint32_t tag_a = phase_tag(A.tag0, in.layer, 3);
    float* out = xs + B * nf;  // [B][d] one part's outputs, after the staged inputs [B][nf]
    {
        float ss[1] = {0.f};
        const StageSeg sg[1] = {{P.act + f0, xs, nullptr, nf, (uint32_t)B, (uint32_t)P.F, nf, tag_a, 0u}};
        if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kComputeWaves, spin, ss)) return false;
    }
    if (!barrier()) return false;
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    const uint32_t rb = d * 2u, lo = 16u * (uint32_t)(wave * 64 + lane);
    DpartRingRows rows{&P, ctl, ring, S, rb, P.ring_chunks * kChunk, 0u, wave, lo < rb, &land_wait};
    for (uint32_t j = 0; j < np; ++j) {
        rows.base = S + j * kDownPart * rb;
        rows.cur = ring_addr(rows.base + lo, P.ring_chunks);
        float acc[B][8];
        if (!dpart_acc<B>(rows, xs + j * kDownPart, nf, acc)) return false;
        release_region(ctl, wave, rows.base + kDownPart * rb);
        if (j > 0 && !barrier()) return false;  // every wave has stored the previous part's outputs
        if (rows.on) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float* o = out + (size_t)b * d + lo / 2u;
                *(float4*)o = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
                *(float4*)(o + 4) = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
            }
        }
        if (!barrier()) return false;
        dpart_store<B>(P, out, in.begin + j, tag_a, wave, kComputeWaves);
    }
    return true;
}

// OP_DRED (split down projection): output rows [begin, begin + count): stage the
// residual rows after O and every part's partials of the rows, then h = hres +
// the partials added in part order.
template <int B>
__device__ __forceinline__ bool dred_instr(const Params& P, const StepArgs& A, float* xs, int wave, const Instr& in,
                                           Spin& spin, CwBarrier& barrier, uint32_t* tr) {
    const uint32_t d = (uint32_t)P.d, cnt = in.count, np = (uint32_t)P.F / kDownPart;
    float* hres = xs;             // [B][cnt]
    float* part = hres + B * cnt;  // [part][B][cnt]
    // the residual rows after O, then every part's partials of the rows (one round trip)
    if (!stage_grid<kStagePassWordsWide>(P.h + in.begin, (uint32_t)B, phase_tag(A.tag0, in.layer, 2),
                                         P.dpart + in.begin, np * (uint32_t)B, phase_tag(A.tag0, in.layer, 3), d, cnt,
                                         xs, wave, kComputeWaves, spin))
        return false;
    if (!barrier()) return false;
    if (tr && lane_id() == 0) tr[2] = (uint32_t)now_ticks();
    dred_out<B>(P, part, hres, in.begin, cnt, np, phase_tag(A.tag0, in.layer, 4), wave, kComputeWaves);
    return true;
}

// One attention item (sequence, KV head, split) as an instruction.
template <int B, int HD, bool CH>
__device__ __forceinline__ bool attn_instr(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                           int wave, const Instr& in, uint32_t S, Spin& spin, CwBarrier& barrier,
                                           uint32_t& land_wait, uint32_t* tr, const int32_t* ctx) {
    const int lane = lane_id();
    const AttnItem it = attn_item_of(P, in.begin);
    const int b = it.b, g = it.g, s = it.s;
    // stream: [RoPE row 1 KB][group 0: K 1 KB, V 1 KB][group 1] ...
    const RingKV<HD> kv{ring, S + kChunk, P.ring_chunks};
    auto need = [&](int t) -> bool {  // group t resident (K and V chunks); t = -1: the RoPE row
        return wait_landed(P, ctl, (S + kChunk + (uint32_t)(t + 1) * 2048u) / kChunk, land_wait);
    };
    auto release = [&](int t) {  // groups before t no longer needed by this wave
        set_consumed(ctl, wave, (S + kChunk + (uint32_t)t * 2048u) / kChunk);
    };
    if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
    auto mark = [&](int m) {
        if (tr && lane == 0) tr[9 + m] = (uint32_t)now_ticks();
    };
    const int pc = ctx_of(ctx, b);
    // (decode kernels take the one-position values at compile time)
    return attn_item<HD, CH>(P, A.tag0, in.layer, b, g, s, it.h0, it.gh, CH ? attn_pos(P, pc, b) : pc, pc,
                             CH ? b + 1 : 1, CH ? kv_seq(P, b) : b, !CH || b < A.tok_rows, kv, need, release, barrier,
                             xs, wave,
                         kComputeWaves, spin, mark);
}

// Returns the queue index of the LM-head instruction once its input is staged
// and published (the caller runs its rows: head_instr), or q1 (none in this kind,
// or the workgroup stopped).
// The down projection at batch 1 with F = 8192, by column quarters (down_q_partial):
// compute wave q stages quarter q of the input (wave 0 also the residual rows), keeps
// it in registers and, row by row, waits for that row's quarter in the ring (4 KB),
// reduces it and leaves the value in LDS; after a barrier wave 0 adds each row's
// quarters in order and the residual.
__device__ __forceinline__ bool down_q_instr(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xs,
                                             int wave, const Instr& in, uint32_t S, Spin& spin, CwBarrier& barrier,
                                             uint32_t& land_wait, uint32_t* tr) {
    const uint32_t lane = (uint32_t)lane_id(), K = (uint32_t)P.F, layer = in.layer;
    float* hres = xs + K;                 // [count] residual rows
    float* part = hres + kMaxResidRows;   // [count][4] quarter values
    float ss[1] = {0.f};
    // each wave stages only its own quarter of the input (the one it reads), wave 0
    // also the residual rows (read only by wave 0, after the closing barrier): no
    // wave reads what another staged before that barrier
    const uint32_t qw = K / 4u, qoff = (uint32_t)wave * qw;
    const StageSeg sg[2] = {{P.act + qoff, xs + qoff, nullptr, qw, 1u, qw, qw, phase_tag(A.tag0, layer, 3)},
                            {P.h + in.begin, hres, nullptr, wave == 0 ? in.count : 0u, 1u, (uint32_t)P.d, in.count,
                             phase_tag(A.tag0, layer, 2)}};
    if (!stage_segs<stage_words_wide<1>(), 1, 2>(sg, 0, 1, spin, ss)) return false;
    if (tr && lane == 0 && wave == 0) tr[2] = (uint32_t)now_ticks();
    const XLds x{xs, K};
    float4 xa[4], xb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x.piece(0, (uint32_t)wave * kDownQPieces + lane + 64u * (uint32_t)k, xa[k], xb[k]);
    // two rows at a time: one wait, all eight pieces requested together, the two
    // reductions interleaved (each row's value is the one down_q_partial gives)
    const uint32_t rb = K * 2u, ring_bytes = P.ring_chunks * kChunk, qb = kDownQPieces * 16u;
    for (uint32_t j = 0; j < in.count; j += 2u) {
        const uint32_t nr = min(2u, in.count - j);
        const uint32_t off = S + j * rb + (uint32_t)wave * qb;
        set_consumed(ctl, wave, off / kChunk);
        if (!wait_landed(P, ctl, (off + (nr - 1u) * rb + qb + kChunk - 1u) / kChunk, land_wait)) return false;
        uint4 w[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // (a lone last row reads its own quarter twice)
            const RingBatch q{ring, ring_addr(off + (i < (int)nr ? (uint32_t)i : 0u) * rb, P.ring_chunks), rb, ring_bytes};
#pragma unroll
            for (int k = 0; k < 4; ++k) w[i][k] = q.piece(0u, lane + 64u * (uint32_t)k);
        }
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = dot8(w[i][k], xa[k], xb[k], acc[i]);
        wave_total_n<2>(acc);
        if (lane == 0) {
            part[j * 4u + (uint32_t)wave] = acc[0];
            if (nr > 1u) part[(j + 1u) * 4u + (uint32_t)wave] = acc[1];
        }
    }
    if (!barrier()) return false;
    if (wave == 0) {
        const uint32_t tag_out = phase_tag(A.tag0, layer, 4);
        for (uint32_t j = lane; j < in.count; j += 64u)
            st_tagged(P.h + in.begin + j, hres[j] + down_q_row(part + j * 4u), tag_out);
    }
    return true;
}

template <int B, int HD, bool MF, bool MOE, bool CH>
__device__ __forceinline__ uint32_t compute_wave(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring,
                                                 float* xs, int wave, uint32_t q0, uint32_t q1, const int32_t* ctx) {
    const int lane = lane_id();
    uint32_t S = 0, k = 0;
    Spin spin(&P, &ctl->abort);
    CwBarrier barrier{ctl, &P, 0u};
    uint32_t head_qi = q1;
    uint32_t gu_expect = 0;  // loader reads of staged (gate, up) inputs seen so far (gu_loader)
    uint32_t o_expect = 0;   // loader completions of O instructions seen so far (o_loader)
    for (uint32_t qi = q0; qi < q1; ++qi, ++k) {
        const Instr in = ld_const(P.instrs + qi);
        uint32_t bytes = instr_bytes<HD, MF, B == 1 && !MF && !MOE && HD == 128>(P, in, ctx);  // MoE expert instructions set it once routed
        uint32_t* tr =
            (P.trace && wave == 0) ? P.trace + ((size_t)blockIdx.x * P.trace_stride + k) * kTraceWords : nullptr;
        if (tr && lane == 0) {
            tr[0] = (uint32_t)in.op | ((uint32_t)in.layer << 16);
            tr[1] = (uint32_t)now_ticks();
        }
        // every wave has finished reading the previous instruction's staged inputs
        if (!barrier()) return q1;
        if (tr && lane == 0) tr[8] = (uint32_t)now_ticks();
        if constexpr (B == 1 && !MOE) {  // (read only by gu_loader)
            if (wave == 0 && lane == 0) lds_st(&ctl->prog, 2u * qi + 1u);
        }
        uint32_t land_wait = 0;
        const int layer = in.layer;
        const DevLayer Lw = ld_const(P.layers + (layer < P.L ? layer : 0));
        bool ok = true;
        // (the matrix-core kernel carries no VALU GEMV code: a smaller kernel)
        if constexpr (MF) {
            if (is_gemv(in.op)) ok = mfma_instr<B, HD>(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr);
            else if (in.op == OP_ATTN) ok = attn_instr<B, HD, CH>(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr, ctx);
        } else switch (in.op) {
            case OP_EGU:
                if constexpr (MOE && B == kMaxBatch) {
                    if (P.x_slices > 1) {
                        ok = moe_egu_sliced<B>(P, A, ctl, ring, xs, wave, in, qi, S, spin, barrier, land_wait, tr, bytes);
                        break;
                    }
                }
                if constexpr (MOE) ok = moe_egu<B>(P, A, ctl, ring, xs, wave, in, qi, S, spin, barrier, land_wait, tr, bytes);
                break;
            case OP_EPART:
                if constexpr (MOE) ok = moe_epart<B>(P, A, ctl, ring, xs, wave, in, qi, S, spin, barrier, land_wait, tr, bytes);
                break;
            case OP_EDOWN:
                if constexpr (MOE) ok = moe_ered<B>(P, A, ctl, xs, wave, in, qi, spin, barrier, tr);
                break;
            case OP_DPART:
                if constexpr (!MOE) ok = dpart_instr<B>(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr);
                break;
            case OP_DRED:
                if constexpr (!MOE) ok = dred_instr<B>(P, A, xs, wave, in, spin, barrier, tr);
                break;
            case OP_QKV:
            case OP_GATEUP:
            case OP_ROUTE:
            case OP_HEAD: {
                if constexpr (MOE && B == kMaxBatch) {
                    if (P.x_slices > 1 && in.op != OP_HEAD) {
                        ok = norm_gemv_sliced<B>(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr);
                        break;
                    }
                }
                // (the gain pointer is chosen on the scalar unit: a plain select of the
                // loaded pointers was lowered through a private array, i.e. scratch memory)
                const uint16_t* gain =
                    uniform_p(in.op == OP_QKV ? Lw.attn_norm : in.op == OP_HEAD ? P.final_norm : Lw.mlp_norm);
                const uint32_t tag_in = in.op == OP_QKV    ? phase_tag(A.tag0, layer - 1, 4)
                                        : in.op == OP_HEAD ? phase_tag(A.tag0, P.L - 1, 4)
                                                           : phase_tag(A.tag0, layer, 2);
                const uint32_t d = (uint32_t)P.d;
                float ss[B];
#pragma unroll
                for (int b = 0; b < B; ++b) ss[b] = 0.f;
                if (in.op == OP_QKV && layer == 0) {
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        stage_bf16(P.embed + token_row(A, b, P.V) * d, d, xs + b * d, gain, wave,
                                   kComputeWaves, ss[b]);
                } else {
                    float* xd = xs;
                    if constexpr (MOE && B == kMaxBatch) {
                        if (in.op == OP_HEAD && P.x_slices > 1) {
                            // the LM-head input is wider than the staging area: it goes
                            // over the weight ring, idle once every loader has retired
                            // its last chunk (the loaders stop streaming at the head)
                            if (!wait_landed(P, ctl, 0xFFFFFFFFu, land_wait)) return q1;
                            xd = (float*)const_cast<char*>(ring);
                        }
                    }
                    const StageSeg sg[1] = {{P.h, xd, gain, d, (uint32_t)B, d, d, tag_in}};
                    if (!stage_segs<stage_words<B>(), B, 1>(sg, wave, kComputeWaves, spin, ss)) return q1;
                }
                wave_total_n<B>(ss);
                if (lane == 0) {
#pragma unroll
                    for (int b = 0; b < B; ++b) ctl->ss[b][wave] = ss[b];
                }
                if (!barrier()) return q1;
                float r[B];
#pragma unroll
                for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
                if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
                if constexpr (B == 1 && !MOE && HD == 128) {  // (read only by o_loader)
                    if (in.op == OP_QKV && wave == 0 && lane == 0) lds_st(&ctl->qkv_layer, (uint32_t)layer + 1u);
                }
                if (in.op == OP_HEAD) {
                    // the LM-head input is staged: publish it to the loader waves; all
                    // eight waves stream the rows after the loop (head_instr)
                    if (wave == 0 && lane == 0) {
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                        lds_st(&ctl->head_seq, qi + 1u);
                    }
                    head_qi = qi;
                    break;
                }
                const uint32_t rb = d * 2u;
                const XLds x{xs, d};
                const uint32_t nrows = in.op == OP_GATEUP ? 2u * in.count : in.count;
                if (in.op == OP_QKV) {
                    const uint32_t tag_out = phase_tag(A.tag0, layer, 0);
                    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                        #pragma unroll
                        for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i)
                            if (i < nr && lane < B)
                                st_tagged(P.qkv + (size_t)lane * P.qkv_rows + in.begin + r0 + i,
                                          pick<B>(res[i], lane) * pick<B>(r, lane), tag_out);
                    };
                    ok = gemv_ring_auto<B>(P, ctl, ring, S, rb, nrows, x, wave, land_wait, epi, false);
                } else if (in.op == OP_ROUTE) {
                    // router logits of experts begin.., tagged like the residual after O
                    const uint32_t tag_out = phase_tag(A.tag0, layer, 2);
                    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                        #pragma unroll
                        for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i)
                            if (i < nr && lane < B)
                                st_tagged(P.route + (size_t)lane * P.E + in.begin + r0 + i,
                                          pick<B>(res[i], lane) * pick<B>(r, lane), tag_out);
                    };
                    ok = gemv_ring_auto<B>(P, ctl, ring, S, rb, nrows, x, wave, land_wait, epi, false);
                } else if (in.op == OP_GATEUP) {
                    const uint32_t tag_out = phase_tag(A.tag0, layer, 3);
                    if (B == 1 && !MOE && P.gu_direct) {  // (B is a template constant)
                        // the loader waves compute the rows (gu_loader): publish the input,
                        // then wait until every loader has stored its outputs
                        if (wave == 0 && lane == 0) {
                            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                            lds_st(&ctl->gu_seq, qi + 1u);
                        }
                        gu_expect += (uint32_t)kLoaderWaves;
                        ok = wait_lds_at_least(P, ctl, &ctl->gu_done, gu_expect, 0xFFFFFFFAu);
                        break;
                    }
                    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                        #pragma unroll
                        for (uint32_t i = 0; i + 1 < (uint32_t)(sizeof(res) / sizeof(res[0])); i += 2) {
                            if (i + 1 >= nr) break;
                            const uint32_t f = in.begin + (r0 + i) / 2u;
                            if (lane < B) {
                                const float rr = pick<B>(r, lane);
                                st_tagged(P.act + (size_t)lane * P.F + f,
                                          silu_mul(pick<B>(res[i], lane) * rr, pick<B>(res[i + 1], lane) * rr),
                                          tag_out);
                            }
                        }
                    };
                    ok = gemv_ring_auto<B>(P, ctl, ring, S, rb, nrows, x, wave, land_wait, epi, true);
                }
                break;
            }
            case OP_O:
            case OP_DOWN: {
                const bool is_o = in.op == OP_O;
                if constexpr (B == 1 && !MOE) {
                    if (!is_o && P.down_q) {
                        ok = down_q_instr(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr);
                        break;
                    }
                }
                const uint32_t K = is_o ? (uint32_t)(P.Hq * HD) : (uint32_t)P.F;
                const uint32_t tag_x = is_o ? phase_tag(A.tag0, layer, 1) : phase_tag(A.tag0, layer, 3);
                const uint32_t tag_res = is_o ? phase_tag(A.tag0, layer - 1, 4) : phase_tag(A.tag0, layer, 2);
                const uint32_t tag_out = is_o ? phase_tag(A.tag0, layer, 2) : phase_tag(A.tag0, layer, 4);
                // O runs over P.x_slices and DOWN over P.down_slices column slices of its input (the stream is
                // slice-major); partial sums of the rows wait in LDS between slices
                const uint32_t ns = is_o ? (uint32_t)P.x_slices : (uint32_t)P.down_slices, Ks = K / ns;
                float* hres = xs + B * Ks;         // [B][count] residual rows before this op
                float* part = hres + B * in.count;  // [B][count] partial sums
                for (uint32_t ks = 0; ks < ns && ok; ++ks) {
                    if (ks > 0 && !barrier()) return q1;  // every wave is done with the previous slice
                    float ss[1] = {0.f};
                    const StageSeg sx = {(is_o ? P.attn : P.act) + ks * Ks, xs, nullptr, Ks, (uint32_t)B, K, Ks,
                                         tag_x};
                    if (ks > 0) {
                        const StageSeg sg[1] = {sx};
                        if (!stage_segs<stage_words_wide<B>(), 1, 1>(sg, wave, kComputeWaves, spin, ss)) return q1;
                    } else if (is_o && layer == 0) {
                        // the residual is the token embedding: no wait
#pragma unroll
                        for (int b = 0; b < B; ++b)
                            stage_bf16(P.embed + token_row(A, b, P.V) * P.d + in.begin,
                                       in.count, hres + b * in.count, nullptr, wave, kComputeWaves, ss[0]);
                        const StageSeg sg[1] = {sx};
                        if (!stage_segs<stage_words_wide<B>(), 1, 1>(sg, wave, kComputeWaves, spin, ss)) return q1;
                    } else {
                        const StageSeg sg[2] = {sx, {P.h + in.begin, hres, nullptr, in.count, (uint32_t)B,
                                                     (uint32_t)P.d, in.count, tag_res}};
                        if (!stage_segs<stage_words_wide<B>(), 1, 2>(sg, wave, kComputeWaves, spin, ss)) return q1;
                    }
                    if (!barrier()) return q1;
                    if (tr && lane == 0 && ks == 0) tr[2] = (uint32_t)now_ticks();
                    if constexpr (B == 1 && !MOE) {
                        if (is_o && ks == 0 && wave == 0 && lane == 0) lds_st(&ctl->prog, 2u * qi + 2u);
                        if (HD == 128 && is_o && P.o_direct) {
                            // the loader waves compute the rows (o_loader); xs is reused
                            // only once every loader is done
                            o_expect += (uint32_t)kLoaderWaves;
                            ok = wait_lds_at_least(P, ctl, &ctl->o_done, o_expect, 0xFFFFFFF5u);
                            break;
                        }
                    }
                    const XLds x{xs, Ks};
                    const bool last = ks + 1 == ns;
                    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                        #pragma unroll
                        for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i) {
                            if (i >= nr) break;
                            const uint32_t j = r0 + i;
                            if (lane < B) {
                                float v = pick<B>(res[i], lane);
                                if (ks > 0) v = part[lane * in.count + j] + v;
                                if (!last) {
                                    part[lane * in.count + j] = v;
                                } else {
                                    st_tagged(P.h + (size_t)lane * P.d + in.begin + j, hres[lane * in.count + j] + v,
                                              tag_out);
                                }
                            }
                        }
                    };
                    ok = gemv_ring_auto<B>(P, ctl, ring, S + ks * in.count * Ks * 2u, Ks * 2u, in.count, x, wave,
                                           land_wait, epi, false);
                    if (ns > 1) release_region(ctl, wave, S + (ks + 1u) * in.count * Ks * 2u);
                }
                break;
            }
            case OP_ATTN: ok = attn_instr<B, HD, CH>(P, A, ctl, ring, xs, wave, in, S, spin, barrier, land_wait, tr, ctx); break;
            default: break;
        }
        if (!ok || lds_ld(&ctl->abort)) return q1;
        if (head_qi < q1) break;  // the head's rows run after the loop
        if (tr && lane == 0) {
            tr[3] = (uint32_t)now_ticks();
            tr[6] = land_wait;
        }
        // the other waves' compute ends (for (gate, up) rows computed by the loaders,
        // loader 0 writes these words: rows requested, input seen, rows done)
        if (P.trace && wave > 0 && in.op != OP_ATTN && !(in.op == OP_GATEUP && P.gu_direct) && lane == 0)
            P.trace[((size_t)blockIdx.x * P.trace_stride + k) * kTraceWords + 8 + wave] = (uint32_t)now_ticks();
        S += bytes;
        set_consumed(ctl, wave, S / kChunk);
        if (tr && lane == 0) tr[4] = (uint32_t)now_ticks();
    }
    return head_qi;
}

// The LM-head instruction (VALU and MoE kinds): the compute waves have staged its
// input in their instruction loop (the staging shared with QKV and GATEUP) and
// published it; then all eight waves stream its rows, in one inlined copy of the
// code for both wave kinds (the kernel is far larger than the instruction cache
// already).  The rows run outside the compute waves' instruction loop: their
// loads are issued ahead, and inside the loop the compiler would have to assume
// some may still be in flight at the back edge, guarding every later write of
// their registers (in the GEMV row loops) with a vmcnt wait.
template <int B, bool MOE>
__device__ __forceinline__ void head_instr(const Params& P, const StepArgs& A, Ctl* ctl, float* xs, int wave,
                                           uint32_t q0, uint32_t qi) {
    const Instr in = ld_const(P.instrs + qi);
    Spin spin(&P, &ctl->abort);
    auto ready = [&](float (&r)[B]) -> bool {
        // The loader waves wait for the input.  Like their other waits this ends on
        // the workgroup's own abort flag or the watchdog, not on an error latched by
        // an earlier step (it spans most of the step, long enough to see one), and
        // the watchdog counts from the compute waves' last barrier: it measures a
        // lack of progress, not the step.
        uint64_t t0 = now_ticks();
        uint32_t polls = 0, seen = lds_ld(&ctl->bar);
        while (lds_ld(&ctl->head_seq) != qi + 1u) {
            if (lds_ld(&ctl->abort)) return false;
            if ((++polls & 255u) == 0) {
                const uint32_t b = lds_ld(&ctl->bar);
                if (b != seen) {
                    seen = b;
                    t0 = now_ticks();
                } else if (now_ticks() - t0 > P.spin_ticks) {
                    raise_error_impl(P.state, P.host_err, &ctl->abort, DERR_TIMEOUT, 0xFFFFFFFBu, qi);
                    return false;
                }
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
        for (int b = 0; b < B; ++b) r[b] = rms_scale(ctl->ss[b], kComputeWaves, P.d, P.eps);
        return true;
    };
    const bool ok = head_direct<B, MOE>(P, A, xs, in, wave, spin, ready);
    if (ok && P.trace && wave == 0 && lane_id() == 0) {  // compute end and end of the head's record
        uint32_t* tr = P.trace + ((size_t)blockIdx.x * P.trace_stride + (qi - q0)) * kTraceWords;
        tr[3] = tr[4] = (uint32_t)now_ticks();
    }
}

template <int B, int HD, bool MF, bool MOE, bool CH = false>
__global__ void __launch_bounds__(kThreads, 1) mk_megakernel(Params P, StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ Ctl ctl;
    char* ring = lds;
    float* xs = (float*)(lds + (size_t)P.ring_chunks * kChunk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (threadIdx.x == 0) {
        for (int k = 0; k < kLoaderWaves; ++k) ctl.landed[k] = (uint32_t)k;
        for (int w = 0; w < kComputeWaves; ++w) ctl.consumed[w] = 0;
        ctl.bar = 0;
        ctl.abort = 0;
        ctl.moe_seq = 0;
        ctl.moe_n = 0;
        ctl.head_seq = 0;
        ctl.gu_seq = 0;
        ctl.gu_done = 0;
        ctl.prog = 0;
        if constexpr (B == 1 && !MF && !MOE && HD == 128) {  // (o_loader)
            ctl.o_done = 0;
            ctl.qkv_layer = 0;
        }
    }
    // context lengths at launch (a multi-position step: every row sees the sequence's cached length)
    if (threadIdx.x < kMaxBatch)
        ctl.ctx[threadIdx.x] = (int)threadIdx.x < B ? P.ctx_len[P.chunk ? P.chunk_seq : (int)threadIdx.x] : 0;
    __syncthreads();
    // this launch's part of the CU's queue (all of it unless the step is cut into several launches)
    const uint32_t* qr = P.cut_q ? P.cut_q + 2u * blockIdx.x : P.queue_off + blockIdx.x;
    const uint32_t q0 = ld_const(qr), q1 = ld_const(qr + 1);
    uint32_t hi;
    if (wave >= kComputeWaves) {
        hi = loader_wave<B, HD, MF, MOE>(P, &ctl, ring, wave - kComputeWaves, q0, q1, ctl.ctx, xs, A.tag0);
    } else {
        hi = compute_wave<B, HD, MF, MOE, CH>(P, A, &ctl, ring, xs, wave, q0, q1, ctl.ctx);
    }
    if constexpr (!MF) {
        float* hx = xs;
        if constexpr (MOE && B == kMaxBatch) hx = P.x_slices > 1 ? (float*)ring : xs;  // staged over the ring
        if (hi < q1) head_instr<B, MOE>(P, A, &ctl, hx, wave, q0, hi);
    }
}

// ------------------------------------------------------------------------------------------------
// host-side launch
// ------------------------------------------------------------------------------------------------
// Kernel of one kind for batch B and head_dim hd (nullptr if not built).
template <bool MF, bool MOE>
const void* kernel_of(int B, int hd) {
    if (hd == 64) {
        if (B == 1) return (const void*)mk_megakernel<1, 64, MF, MOE>;
        if (B == 2) return (const void*)mk_megakernel<2, 64, MF, MOE>;
        if (B == 4) return (const void*)mk_megakernel<4, 64, MF, MOE>;
        if (B == 8) return (const void*)mk_megakernel<8, 64, MF, MOE>;
    } else if (hd == 128) {
        if (B == 1) return (const void*)mk_megakernel<1, 128, MF, MOE>;
        if (B == 2) return (const void*)mk_megakernel<2, 128, MF, MOE>;
        if (B == 4) return (const void*)mk_megakernel<4, 128, MF, MOE>;
        if (B == 8) return (const void*)mk_megakernel<8, 128, MF, MOE>;
    }
    return nullptr;
}

// Multi-position kernel (kChunkRows rows of one sequence, VALU GEMVs) for head_dim hd.
template <bool MOE>
const void* kernel_of_chunk(int hd) {
    if (hd == 64) return (const void*)mk_megakernel<kChunkRows, 64, false, MOE, true>;
    if (hd == 128) return (const void*)mk_megakernel<kChunkRows, 128, false, MOE, true>;
    return nullptr;
}

}  // namespace mk
