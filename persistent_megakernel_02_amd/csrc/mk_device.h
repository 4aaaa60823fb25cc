// Device tile functions shared by the persistent megakernel and the
// one-kernel-per-op path.  Both paths call the same functions with the same
// lane-to-data mapping, so they perform identical fp32 operations in identical
// order and produce bitwise-identical results.
//
// Ops (page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "Megakernel：从零设计的深度融合方案": the composite instructions fuse RMSNorm, the
// QKV projection and RoPE; attention; the MLP).  The textbook definitions they
// follow: RMSNorm (Zhang and Sennrich 2019), rotary embedding with rotate-half
// pairs (Su et al.), grouped-query attention (Ainslie et al. 2023), SwiGLU
// (Shazeer 2020).  Precision: weights and the K/V cache are bf16; every
// activation (normed x, q, attention output, SwiGLU product, residual) is fp32;
// every product of a matrix and a vector accumulates in fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Load through the constant address space: uniform, read-only data (schedule,
// layer pointer table) then travels through scalar loads and never occupies the
// vector-memory counters.
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
    static_assert(sizeof(T) % 4 == 0, "word-sized records only");
    typedef const __attribute__((address_space(4))) uint32_t cword;
    const cword* q = (const cword*)p;
    uint32_t w[sizeof(T) / 4];
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i) w[i] = q[i];
    T out;
    __builtin_memcpy(&out, w, sizeof(T));
    return out;
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f_to_bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f_to_bf(lo) | (f_to_bf(hi) << 16); }

// acc + sum over the 8 bf16 weights of w times the 8 fp32 activations (xa, xb),
// one fused multiply-add each, in a fixed order.
__device__ __forceinline__ float dot8(uint4 w, float4 xa, float4 xb, float acc) {
    acc = fmaf(bf_lo(w.x), xa.x, acc);
    acc = fmaf(bf_hi(w.x), xa.y, acc);
    acc = fmaf(bf_lo(w.y), xa.z, acc);
    acc = fmaf(bf_hi(w.y), xa.w, acc);
    acc = fmaf(bf_lo(w.z), xb.x, acc);
    acc = fmaf(bf_hi(w.z), xb.y, acc);
    acc = fmaf(bf_lo(w.w), xb.z, acc);
    acc = fmaf(bf_hi(w.w), xb.w, acc);
    return acc;
}

// Total over the 64 lanes with DPP, in a fixed tree: quad butterflies, half-row
// and row mirrors (16-lane sums), then row broadcasts accumulate rows 0..3 into
// lane 63.  The value of lane 63 is returned to every lane (scalar).
__device__ __forceinline__ float wave_total(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);  // row_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// wave_total of N values at once: the same tree, one DPP step applied to every
// value before the next step, so consecutive DPP reads never depend on each
// other (no wait states between them).  Each result is bit-identical to
// wave_total of that value alone.
template <int N>
__device__ __forceinline__ void wave_total_n(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0xB1, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x4E, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x141, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x140, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x142, 0xA, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x143, 0xC, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Token ids come from device memory; clamp so a bad id cannot index outside the
// embedding table.
__device__ __forceinline__ size_t token_row(const StepArgs& A, int b, int V) {
    const int r = b < A.tok_rows ? b : A.tok_rows - 1;  // rows past the given tokens repeat the last
    const int t = A.tok_in[r * A.tok_stride];
    return (size_t)(t < 0 ? 0 : (t >= V ? V - 1 : t));
}

// ---------------------------------------------------------------------------------------------
// Tagged activation words {fp32 value (low half), tag (high half)}.  Stores and
// loads are single 8-byte accesses at agent scope: the store writes through to
// the device coherence point and the load reads it there, so a word whose tag
// matches carries the matching value.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void st_tagged(uint64_t* p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tv_val(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t tv_tag(uint64_t w) { return (uint32_t)(w >> 32); }

// Device error: the first code wins the state word and is mirrored to the
// pinned host word; the workgroup's abort flag (LDS) stops its other waves.
__device__ __noinline__ void raise_error_impl(DevState* state, HostErr* herr, uint32_t* abort_flag, uint32_t code,
                                             uint32_t a, uint32_t b) {
    if (abort_flag) __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((threadIdx.x & 63) == 0) {
        uint32_t expected = 0;
        if (__hip_atomic_compare_exchange_strong(&state->error, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
            state->err_info[0] = a;
            state->err_info[1] = b;
            state->err_info[2] = blockIdx.x;
            if (herr) {
                __hip_atomic_store(&herr->info[0], a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(&herr->info[1], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(&herr->info[2], blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(&herr->code, code, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
}

// Bounded spin of one wave: again() sleeps briefly and answers whether to keep
// polling.  It gives up when the workgroup aborted, when another workgroup
// latched a device error, or (raising DERR_TIMEOUT) when the watchdog expires.
struct Spin {
    const Params* P;
    uint32_t* abort_flag;  // LDS flag of the workgroup, or nullptr
    uint64_t t0;
    uint32_t polls;
    __device__ Spin(const Params* p, uint32_t* ab) : P(p), abort_flag(ab), t0(0), polls(0) {}
    __device__ __forceinline__ bool aborted() const {
        return abort_flag && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
    }
    __device__ __forceinline__ void start() { polls = 0; }  // begin a new wait
    __device__ __forceinline__ bool again(uint32_t a, uint32_t b) {
        if (polls == 0) t0 = now_ticks();
        ++polls;
        __builtin_amdgcn_s_sleep(1);
        if (aborted()) return false;
        if ((polls & 63u) == 0) {
            if (__hip_atomic_load(&P->state->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                if (abort_flag) __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                return false;
            }
            if (now_ticks() - t0 > P->spin_ticks) {
                raise_error_impl(P->state, P->host_err, abort_flag, DERR_TIMEOUT, a, b);
                return false;
            }
        }
        return true;
    }
};

// ---------------------------------------------------------------------------------------------
// GEMV on the matrix cores (v_mfma_f32_16x16x32_bf16).  A tile is 16 consecutive
// rows of an instruction's row sequence; a k-block is 32 columns.  Operand A is
// the weights: lane l holds row l % 16, columns 8 (l / 16) .. + 7 of the k-block
// (16 bytes).  Operand B holds the activations split into PRT bf16 parts
// x = x_1 + x_2 (+ x_3), each exact as a bf16 product with a weight: column
// j = PRT b + p of B is part p of batch row b (lanes with j >= PRT B hold zeros).
// D[i][j] (lane l: rows 4 (l / 16) + r, column l % 16) summed over the parts of
// batch row b is the dot product of row i with x_b, accumulated in fp32.
// Three parts carry 24 mantissa bits (the fp32 value up to rounding of the sum);
// two parts, used from batch 6 on where 3 B columns exceed 16, carry 16.
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Row j of an instruction's row sequence: QKV [Wq; Wk; Wv] rows from `begin`;
// GATEUP gate row, up row of f = begin + j / 2; the others rows from `begin`.
template <int OP>
__device__ __forceinline__ const uint16_t* gemv_row_ptr(const Params& P, const DevLayer& Lw, uint32_t begin,
                                                        uint32_t j) {
    if (OP == OP_QKV) {
        const uint32_t row = begin + j, nq = (uint32_t)(P.Hq * P.hd), nk = (uint32_t)(P.Hkv * P.hd);
        return row < nq ? Lw.wq + (size_t)row * P.d
             : row < nq + nk ? Lw.wk + (size_t)(row - nq) * P.d
                             : Lw.wv + (size_t)(row - nq - nk) * P.d;
    } else if (OP == OP_GATEUP) {
        return ((j & 1u) ? Lw.w_up : Lw.w_gate) + (size_t)(begin + (j >> 1)) * P.d;
    } else if (OP == OP_HEAD) {
        return P.head + (size_t)(begin + j) * P.d;
    } else if (OP == OP_O) {
        return Lw.wo + (size_t)(begin + j) * (P.Hq * P.hd);
    } else {
        return Lw.w_down + (size_t)(begin + j) * P.F;
    }
}

// Byte offset in the activation-parts area of column j (part p of batch row b is
// column PRT b + p) of element k: [k-block][k-group of 8][slot j < pitch][8 bf16].
__device__ __forceinline__ uint32_t part_offset(uint32_t k, uint32_t j, uint32_t pitch) {
    return ((((k >> 5) * 4u + ((k >> 3) & 3u)) * pitch + j) * 8u + (k & 7u)) * 2u;
}

// Splits v into PRT bf16 parts (round to nearest even at each step) and stores
// them for element k of batch row b.
template <int PRT>
__device__ __forceinline__ void store_parts(char* area, uint32_t k, uint32_t b, uint32_t pitch, float v) {
    float rem = v;
#pragma unroll
    for (int p = 0; p < PRT; ++p) {
        const uint32_t h = f_to_bf(rem);
        *(uint16_t*)(area + part_offset(k, (uint32_t)PRT * b + (uint32_t)p, pitch)) = (uint16_t)h;
        rem = rem - __uint_as_float(h << 16);
    }
}

// store_parts for a pair of lanes (2 l, 2 l + 1) holding elements k, k + 1 of one
// batch row (staging hands consecutive elements to consecutive lanes, and a parts
// segment has an even number of elements per row): each part is converted with
// the hardware round-to-nearest-even, the odd lane's value moves over with a DPP
// row shift and the even lane stores both as one 32-bit word.  Both lanes of a
// pair must be active.
__device__ __forceinline__ void store_parts_pair(char* area, uint32_t k, uint32_t b, uint32_t pitch, uint32_t prt,
                                                 float v) {
    const bool even = (lane_id() & 1) == 0;
    float rem = v;
#pragma unroll
    for (uint32_t p = 0; p < 3u; ++p) {
        if (p < prt) {
            const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rem);
            rem = rem - __uint_as_float(h << 16);
            const uint32_t hn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x101, 0xF, 0xF, false);  // row_shl:1
            if (even) *(uint32_t*)(area + part_offset(k, prt * b + p, pitch)) = h | (hn << 16);
        }
    }
}

// Operand B of k-block kb for this lane (zeros past the PB used columns).
__device__ __forceinline__ bf16x8_t load_parts(const char* area, uint32_t kb, uint32_t PB, uint32_t pitch) {
    const uint32_t l = (uint32_t)lane_id(), j = l & 15u, kg = l >> 4;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (j < PB) u = *(const uint4*)(area + (((kb * 4u + kg) * pitch + j) * 16u));
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ floatx4_t mfma_acc(uint4 a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b, c, 0, 0, 0);
}

// Sum of the PRT part columns into the lane of part 0 (lanes j = PRT b): the
// neighbours' values come over with DPP row shifts.  Other lanes hold partial sums.
template <int PRT>
__device__ __forceinline__ floatx4_t combine_parts(floatx4_t d) {
    floatx4_t s;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float v1 = __builtin_amdgcn_update_dpp(0.0f, d[r], 0x101, 0xF, 0xF, false);  // row_shl:1
        float t = d[r] + v1;
        if (PRT == 3) t += __builtin_amdgcn_update_dpp(0.0f, d[r], 0x102, 0xF, 0xF, false);  // row_shl:2
        s[r] = t;
    }
    return s;
}

// Tile-major chunks of a matrix-core GEMV instruction, column slice by column
// slice.  A chunk holds R = kMfmaChunkRows rows of a tile, each row's 1024 / R
// bytes whole (the weight loads read whole 128-byte lines and longer runs of a
// row).  Within a slice:
//  - full groups: four full tiles (16 rows) in step, one per wave.  A unit is one
//    tile's 16 rows x kMfmaUnitCols columns (16 / R chunks); units run
//    k-unit-major, then tile of the group;
//  - the last group: the remaining nrows - 64 G4 rows (up to four tiles, the last
//    one partial), k-unit-major, CR = ceil(rows / R) chunks per k-unit holding
//    the group's rows in order, so no row past the end is streamed (a chunk may
//    end past it: those rows re-read the last row).
// In a chunk, piece p (16 bytes) of its row rr (tile row r) sits at slot
// rr * PPR + (p ^ (r % PPR)), PPR = pieces per chunk row: the XOR spreads the
// sixteen lanes that read one column of pieces over different LDS banks.
constexpr uint32_t kMfmaPiecesPerRow = 64u / kMfmaChunkRows;
constexpr uint32_t kMfmaUnitChunks = 16u / kMfmaChunkRows;
constexpr uint32_t kMfmaUnitKb = kMfmaPiecesPerRow / 4u;  // k-blocks of 32 columns per unit
// 4 or 8 chunks per unit: a loader (every fourth chunk) takes one or two of each
static_assert(kMfmaChunkRows == 2 || kMfmaChunkRows == 4, "chunk rows");

struct MfmaGeo {
    uint32_t nrows, KU, slices, K;  // rows, k-units per slice, slices, row length
    uint32_t G4;                    // full groups of four full tiles
    uint32_t m;                     // tiles of the last group (0 to 4, the last may be partial)
    uint32_t CR;                    // chunks per k-unit of the last group
    __device__ __forceinline__ uint32_t full_chunks() const { return G4 * 4u * KU * kMfmaUnitChunks; }
    __device__ __forceinline__ uint32_t slice_chunks() const { return full_chunks() + KU * CR; }
    __device__ __forceinline__ uint32_t chunks() const { return slices * slice_chunks(); }
};

template <int HD>
__device__ __forceinline__ MfmaGeo mfma_geo(const Params& P, const Instr& in) {
    MfmaGeo g;
    g.nrows = in.op == OP_GATEUP ? 2u * in.count : in.count;
    g.K = in.op == OP_O ? (uint32_t)(P.Hq * HD) : in.op == OP_DOWN ? (uint32_t)P.F : (uint32_t)P.d;
    g.slices = in.op == OP_DOWN ? (uint32_t)P.down_slices : 1u;
    g.KU = g.K / g.slices / (32u * kMfmaUnitKb);
    g.G4 = g.nrows / 64u;
    const uint32_t rest = g.nrows - 64u * g.G4;
    g.m = (rest + 15u) / 16u;
    g.CR = (rest + kMfmaChunkRows - 1u) / kMfmaChunkRows;
    return g;
}

// Row j of instruction `in`'s row sequence, by op.
__device__ __forceinline__ const uint16_t* gemv_row(const Params& P, const DevLayer& Lw, const Instr& in, uint32_t j) {
    switch (in.op) {
        case OP_QKV: return gemv_row_ptr<OP_QKV>(P, Lw, in.begin, j);
        case OP_GATEUP: return gemv_row_ptr<OP_GATEUP>(P, Lw, in.begin, j);
        case OP_O: return gemv_row_ptr<OP_O>(P, Lw, in.begin, j);
        case OP_DOWN: return gemv_row_ptr<OP_DOWN>(P, Lw, in.begin, j);
        default: return gemv_row_ptr<OP_HEAD>(P, Lw, in.begin, j);
    }
}

// Partial tile t of wave w after combine_parts: the part-0 lane of each batch row
// stores its 4 sums; the owner adds the four waves' partials in wave order.
template <int B, int PRT>
__device__ __forceinline__ void red_store(char* red, int w, uint32_t t, floatx4_t d) {
    const uint32_t l = (uint32_t)lane_id(), j = l & 15u, kg = l >> 4;
    if (j % (uint32_t)PRT == 0u && j < (uint32_t)(PRT * B))
        *(floatx4_t*)(red + ((((uint32_t)w * 4u + t) * 4u + kg) * B + j / PRT) * 16u) = d;
}
template <int B, int PRT>
__device__ __forceinline__ floatx4_t red_sum(const char* red, uint32_t t) {
    const uint32_t l = (uint32_t)lane_id(), j = l & 15u, kg = l >> 4;
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
    if (j % (uint32_t)PRT == 0u && j < (uint32_t)(PRT * B)) {
#pragma unroll
        for (uint32_t w = 0; w < 4u; ++w) {
            const floatx4_t v = *(const floatx4_t*)(red + (((w * 4u + t) * 4u + kg) * B + j / PRT) * 16u);
            s = w == 0 ? v : s + v;
        }
    }
    return s;
}

// ---------------------------------------------------------------------------------------------
// Staging of tagged activations into LDS.  A segment is `rows` rows of n tagged
// words (row r at src + r * src_stride) that land as fp32 at dst + r * dst_stride,
// optionally times a bf16 gain g[i] (the RMSNorm weight).  The segments of one
// instruction are numbered as one sequence; wave w of nw takes elements
// e = 64 (w + nw k) + lane, K words per lane per pass.  Every load of a pass
// is issued at once (the gains with the words), and the next pass is issued
// before the current one is checked, so a staging costs about one memory round
// trip however many segments and passes it has.  Words whose tag does not match
// yet are re-read until it does (bounded by the watchdog).
// ---------------------------------------------------------------------------------------------
struct StageSeg {
    const uint64_t* src;
    float* dst;
    const uint16_t* g;  // gain, or nullptr
    uint32_t n, rows, src_stride, dst_stride;
    uint32_t tag;       // tag the words must carry
    uint32_t parts;     // 0: fp32 rows at dst; 2 or 3: bf16 parts for the matrix cores in the area at dst
};

// Element e of the concatenated segments resolved to its row's source, target,
// gain and tag.  The segment fields are wave-uniform; only the choice between
// them is per lane, made by selects (no indexing of the segment array by a
// per-lane value, which would move it to scratch memory).
struct StageLoc {
    const uint64_t* src;  // the tagged word
    float* dst;           // where its value lands (fp32 rows), or the parts area
    const uint16_t* g;    // its gain, or nullptr
    uint32_t tag;
    uint32_t row;
    uint32_t idx;         // element index within the row
    uint32_t parts;       // 0, or the number of bf16 parts (area of parts * rows columns)
    uint32_t pitch;       // slots per row of the parts area
};

template <class T>
__device__ __forceinline__ T* uniform_p(T* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (T*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t uniform_u(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

template <int NS>
struct StageMap {
    // the segment fields as wave-uniform register values (read once)
    const uint64_t* src[NS];
    float* dst[NS];
    const uint16_t* g[NS];
    uint32_t n[NS], rows[NS], ss[NS], ds[NS], tag[NS], end[NS], parts[NS];
    uint32_t total;
    __device__ __forceinline__ explicit StageMap(const StageSeg (&s)[NS]) {
        uint32_t t = 0;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            src[i] = uniform_p(s[i].src);
            dst[i] = uniform_p(s[i].dst);
            g[i] = uniform_p(s[i].g);
            n[i] = uniform_u(s[i].n);
            ss[i] = uniform_u(s[i].src_stride);
            ds[i] = uniform_u(s[i].dst_stride);
            tag[i] = uniform_u(s[i].tag);
            parts[i] = uniform_u(s[i].parts);
            rows[i] = uniform_u(s[i].rows);
            t += n[i] * rows[i];
            end[i] = t;
        }
        total = t;
    }
    __device__ __forceinline__ StageLoc locate(uint32_t e) const {
        const uint64_t* sp = src[0];
        float* dp = dst[0];
        const uint16_t* gp = g[0];
        uint32_t nn = n[0], nr = rows[0], s1 = ss[0], d1 = ds[0], tg = tag[0], pt = parts[0], e0 = 0;
#pragma unroll
        for (int k = 1; k < NS; ++k) {
            const bool in = e >= end[k - 1];
            sp = in ? src[k] : sp;
            dp = in ? dst[k] : dp;
            gp = in ? g[k] : gp;
            nn = in ? n[k] : nn;
            nr = in ? rows[k] : nr;
            s1 = in ? ss[k] : s1;
            d1 = in ? ds[k] : d1;
            tg = in ? tag[k] : tg;
            pt = in ? parts[k] : pt;
            e0 = in ? end[k - 1] : e0;
        }
        // row of element x of the segment by comparisons (at most kMaxBatch rows):
        // no integer division per element
        const uint32_t x = e - e0;
        uint32_t r = 0;
#pragma unroll
        for (int k = 1; k < kMaxBatch; ++k) r += ((uint32_t)k < nr && x >= (uint32_t)k * nn) ? 1u : 0u;
        const uint32_t i = x - r * nn;
        return StageLoc{sp + (size_t)r * s1 + i, pt ? dp : dp + (size_t)r * d1 + i, gp ? gp + i : nullptr, tg, r, i,
                        pt, (pt * nr) | 1u};
    }
};

// ss[r] gets the lane's sum of squares of the raw values of row r of the gained
// segments, in ascending element order (RMSNorm statistics).
template <int K, int R, int NS>
__device__ __forceinline__ bool stage_segs(const StageSeg (&sg)[NS], int w, int nw, Spin& spin, float (&ss)[R]) {
    const StageMap<NS> map(sg);
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t step = 64u * (uint32_t)nw;
    const uint32_t per_pass = step * (uint32_t)K;
    const uint32_t total = map.total;
    // loads of the pass starting at p0 (elements past the end re-read element 0)
    auto issue = [&](uint32_t p0, uint64_t (&v)[K], uint32_t (&gv)[K]) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
            const StageLoc L = map.locate(e < total ? e : 0u);
            v[k] = ld_tagged(L.src);
            gv[k] = *(L.g ? L.g : (const uint16_t*)L.src);
        }
    };
    // wait for, check and store the pass starting at p0
    auto finish = [&](uint32_t p0, uint64_t (&v)[K], const uint32_t (&gv)[K]) -> bool {
        spin.start();
        for (;;) {
            bool ok = true;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
                ok &= e >= total || tv_tag(v[k]) == map.locate(e).tag;
            }
            if (__all(ok)) break;
            if (!spin.again(map.tag[0], p0)) return false;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
                if (e < total) {
                    const StageLoc L = map.locate(e);
                    if (tv_tag(v[k]) != L.tag) v[k] = ld_tagged(L.src);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
            if (e < total) {
                const StageLoc L = map.locate(e);
                const float x = tv_val(v[k]);
                float y = x;
                if (L.g) {
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
                        if (rr == (int)L.row) ss[rr] = fmaf(x, x, ss[rr]);
                    y = x * bf_to_f((uint16_t)gv[k]);
                }
                if (L.parts) store_parts_pair((char*)L.dst, L.idx, L.row, L.pitch, L.parts, y);
                else *L.dst = y;
            }
        }
        return true;
    };
    // A pass is issued only when it will be read, and the exit retires every load
    // explicitly (vmcnt(0), cheap since nothing unread is in flight): the compiler's
    // wait analysis cannot tie the `more` tests together, so without the explicit
    // wait it would take loads into these registers as possibly pending wherever
    // they are next written, and inside the GEMV row loops that follow it would
    // guard such writes with a vmcnt wait on every row batch, which also waits for
    // the previous batch's write-through result stores.
    uint64_t va[K], vb[K];
    uint32_t ga[K], gb[K];
    issue(0u, va, ga);
    for (uint32_t p0 = 0;; p0 += 2u * per_pass) {
        const bool more = p0 + per_pass < total;
        if (more) issue(p0 + per_pass, vb, gb);
        if (!finish(p0, va, ga)) return false;
        if (!more) break;
        const bool more2 = p0 + 2u * per_pass < total;
        if (more2) issue(p0 + 2u * per_pass, va, ga);
        if (!finish(p0 + per_pass, vb, gb)) return false;
        if (!more2) break;
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
    return true;
}

// Stages a grid of tagged words into dst [n0 + n1][cnt]: rows [0, n0) from src0
// carrying tag0, then rows [0, n1) from src1 carrying tag1 (row stride `stride`
// words in both, columns [0, cnt)), once each word carries its tag.  Element
// e = r cnt + c is lane e mod 64 of wave (e / 64) mod nw's passes, K per lane per
// pass and two passes in flight, like stage_segs, but for any number of rows
// (StageSeg resolves at most kMaxBatch rows per segment).  The row of e is
// e * ceil(2^32 / cnt) >> 32, exact for e < 2^32 / cnt.
template <int K>
__device__ __forceinline__ bool stage_grid(const uint64_t* src0, uint32_t n0, uint32_t tag0, const uint64_t* src1,
                                           uint32_t n1, uint32_t tag1, uint32_t stride, uint32_t cnt, float* dst,
                                           int w, int nw, Spin& spin) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t step = 64u * (uint32_t)nw, per_pass = step * (uint32_t)K, total = (n0 + n1) * cnt;
    const uint64_t magic = ((1ull << 32) + cnt - 1u) / cnt;
    const uint32_t e1 = n0 * cnt;  // first element of the second block
    auto word = [&](uint32_t e) -> const uint64_t* {
        const uint32_t r = (uint32_t)(((uint64_t)e * magic) >> 32), c = e - r * cnt;
        return r < n0 ? src0 + (size_t)r * stride + c : src1 + (size_t)(r - n0) * stride + c;
    };
    auto tag_of = [&](uint32_t e) { return e < e1 ? tag0 : tag1; };
    auto issue = [&](uint32_t p0, uint64_t (&v)[K]) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
            v[k] = ld_tagged(word(e < total ? e : 0u));
        }
    };
    auto finish = [&](uint32_t p0, uint64_t (&v)[K]) -> bool {
        spin.start();
        for (;;) {
            bool ok = true;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
                ok &= e >= total || tv_tag(v[k]) == tag_of(e);
            }
            if (__all(ok)) break;
            if (!spin.again(tag1, p0)) return false;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
                if (e < total && tv_tag(v[k]) != tag_of(e)) v[k] = ld_tagged(word(e));
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t e = p0 + 64u * (uint32_t)w + lane + step * (uint32_t)k;
            if (e < total) dst[e] = tv_val(v[k]);
        }
        return true;
    };
    if (total == 0) return true;
    uint64_t va[K], vb[K];
    issue(0u, va);
    for (uint32_t p0 = 0;; p0 += 2u * per_pass) {
        const bool more = p0 + per_pass < total;
        if (more) issue(p0 + per_pass, vb);
        if (!finish(p0, va)) return false;
        if (!more) break;
        const bool more2 = p0 + 2u * per_pass < total;
        if (more2) issue(p0 + 2u * per_pass, va);
        if (!finish(p0 + per_pass, vb)) return false;
        if (!more2) break;
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
    return true;
}

// Split down projection, one part: acc[b][e] = sum over the part's kDownPart
// SwiGLU outputs f, in ascending order, of x[b][f] * WT[f][o + e] (fp32 fma), where
// o = 8 (64 w + l) is this lane's first output row and WT the transposed Wdown
// rows of the part.  `rows.get(f, q)` supplies this lane's 16 bytes of rows f ..
// f + kDpartRowsPerGet - 1 (after any wait); x is [B][xstride] in LDS from the
// part's first column.
// Both the persistent kernel (rows from the LDS ring) and the one-kernel-per-op
// path (rows from HBM) call it, so their partials are the same bits.
template <int B, class Rows>
__device__ __forceinline__ bool dpart_acc(Rows& rows, const float* x, uint32_t xstride, float (&acc)[B][8]) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
    for (uint32_t f = 0; f < kDownPart; f += kDpartRowsPerGet) {
        uint4 q[kDpartRowsPerGet];
        if (!rows.get(f, q)) return false;
        static_assert(kDpartRowsPerGet == 4, "one float4 of inputs per batch row and get");
        float4 xv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xv[b] = *(const float4*)(x + (size_t)b * xstride + f);
#pragma unroll
        for (int u = 0; u < kDpartRowsPerGet; ++u) {
            const float wv[8] = {bf_lo(q[u].x), bf_hi(q[u].x), bf_lo(q[u].y), bf_hi(q[u].y),
                                 bf_lo(q[u].z), bf_hi(q[u].z), bf_lo(q[u].w), bf_hi(q[u].w)};
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float a = u == 0 ? xv[b].x : u == 1 ? xv[b].y : u == 2 ? xv[b].z : xv[b].w;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(a, wv[e], acc[b][e]);
            }
        }
    }
    return true;
}

// Split down projection, rows [begin, begin + cnt): h[b][row] = hres + the sum of
// the parts' partials, from the staged partials part[(j B + b) cnt + i] and
// residual rows hres[b cnt + i] in LDS.  Output k = b cnt + i goes to wave k mod
// nw: lane l adds the partials of parts l, l + 64, ... in ascending order, then
// wave_total adds the 64 lane sums in its fixed tree (four outputs at a time).
template <int B>
__device__ __forceinline__ void dred_out(const Params& P, const float* part, const float* hres, uint32_t begin,
                                         uint32_t cnt, uint32_t np, uint32_t tag, int w, int nw) {
    const uint32_t lane = (uint32_t)lane_id(), total = (uint32_t)B * cnt, step = (uint32_t)nw;
    for (uint32_t k0 = (uint32_t)w; k0 < total; k0 += 4u * step) {
        float s[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t k = k0 + (uint32_t)t * step;
            s[t] = 0.f;
            if (k < total) {
                const uint32_t b = k / cnt, i = k - b * cnt;
                for (uint32_t p = lane; p < np; p += 64u) s[t] += part[(p * B + b) * cnt + i];
            }
        }
        wave_total_n<4>(s);
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t k = k0 + (uint32_t)t * step;
                if (k < total) {
                    const uint32_t b = k / cnt, i = k - b * cnt;
                    st_tagged(P.h + (size_t)b * P.d + begin + i, hres[k] + s[t], tag);
                }
            }
        }
    }
}

// Split down projection: one part's partial outputs out[b][row] (LDS, written by
// dpart_acc's lanes 8 rows each) stored to dpart with consecutive lanes on
// consecutive words (a lane's own 8 rows are 64 bytes apart from its
// neighbour's: stored directly, every store would touch 64 cache lines).
template <int B>
__device__ __forceinline__ void dpart_store(const Params& P, const float* out, uint32_t part, uint32_t tag, int w,
                                            int nw) {
    const uint32_t n = (uint32_t)B * (uint32_t)P.d;
    uint64_t* dst = P.dpart + (size_t)part * n;
    for (uint32_t i = (uint32_t)(w * 64 + lane_id()); i < n; i += 64u * (uint32_t)nw) st_tagged(dst + i, out[i], tag);
}

// Same from a bf16 row that needs no wait (the token embedding of layer 0);
// g == nullptr copies without a gain.
__device__ __forceinline__ void stage_bf16(const uint16_t* __restrict__ src, uint32_t n, float* __restrict__ dst,
                                           const uint16_t* __restrict__ g, int w, int nw, float& ss) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t step = 64u * (uint32_t)nw;
    for (uint32_t e = 64u * (uint32_t)w + lane; e < n; e += step) {
        const float x = bf_to_f(src[e]);
        ss = fmaf(x, x, ss);
        dst[e] = g ? x * bf_to_f(g[e]) : x;
    }
}

// As stage_bf16, into the bf16 parts of batch row b for the matrix cores.
template <int PRT>
__device__ __forceinline__ void stage_bf16_parts(const uint16_t* __restrict__ src, uint32_t n, char* area, uint32_t b,
                                                 uint32_t pitch, const uint16_t* __restrict__ g, int w, int nw,
                                                 float& ss) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t step = 64u * (uint32_t)nw;
    for (uint32_t e = 64u * (uint32_t)w + lane; e < n; e += step) {
        const float x = bf_to_f(src[e]);
        ss = fmaf(x, x, ss);
        store_parts<PRT>(area, e, b, pitch, g ? x * bf_to_f(g[e]) : x);
    }
}

// RMSNorm statistics: wave w stored its total wave_total(ss) in part[w]; every
// wave forms r = 1 / sqrt(mean + eps) from the four partials in order 0..3.
__device__ __forceinline__ float rms_scale(const float* part, int nw, int d, float eps) {
    float s = part[0];
    for (int w = 1; w < nw; ++w) s += part[w];
    return 1.0f / sqrtf(s / (float)d + eps);
}

// ---------------------------------------------------------------------------------------------
// Row sources: piece p (16 bytes = 8 bf16) of row i of the current batch.
// ---------------------------------------------------------------------------------------------
struct RingBatch {  // rows back to back in the LDS ring starting at byte `base`
    const char* ring;
    uint32_t base, rb, ring_bytes;
    __device__ __forceinline__ uint4 piece(uint32_t i, uint32_t p) const {
        uint32_t a = base + i * rb + p * 16u;
        a = a >= ring_bytes ? a - ring_bytes : a;
        return *(const uint4*)(ring + a);
    }
};

// Activation source (fp32 in LDS): the 8 values of piece p of batch row b.
struct XLds {
    const float* x;
    uint32_t k;
    __device__ __forceinline__ void piece(int b, uint32_t p, float4& a, float4& c) const {
        const float* q = x + (size_t)b * k + 8 * p;
        a = *(const float4*)q;
        c = *(const float4*)(q + 4);
    }
};

// out[i][b] = dot(row i, x_b) for the R rows of a batch.  Lane l accumulates
// pieces p = l, l + 64, ... in ascending order, then wave_total reduces in its
// fixed tree; a row's value never depends on R or on the other rows.  (Issuing
// four pieces' loads ahead of their use measured slower in the persistent
// kernel: the extra registers cost more than the latency they hide.)
template <int B, int R, class Rows, class X>
__device__ __forceinline__ void rows_dot(const Rows& rows, int np, const X& x, float (&out)[R][B]) {
    const int lane = lane_id();
    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.f;
#pragma unroll 2
    for (int p = lane; p < np; p += 64) {
        uint4 w[R];
#pragma unroll
        for (int i = 0; i < R; ++i) w[i] = rows.piece((uint32_t)i, (uint32_t)p);
        float4 xa[B], xb[B];
#pragma unroll
        for (int b = 0; b < B; ++b) x.piece(b, (uint32_t)p, xa[b], xb[b]);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[i][b] = dot8(w[i], xa[b], xb[b], acc[i][b]);
    }
    float t[R * B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) t[i * B + b] = acc[i][b];
    wave_total_n<R * B>(t);
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) out[i][b] = t[i * B + b];
}

// Quarter q of a down-projection row (batch 1, F = 8192): this lane's 4 pieces
// lane + 64 k of the quarter against the matching x pieces (in registers), in
// ascending order, then the fixed wave_total tree.  The row is the four quarters'
// values added in order (down_q_row).
__device__ __forceinline__ float down_q_partial(const uint4 (&w)[4], const float4 (&xa)[4], const float4 (&xb)[4]) {
    float acc[1] = {0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[0] = dot8(w[k], xa[k], xb[k], acc[0]);
    wave_total_n<1>(acc);
    return acc[0];
}
__device__ __forceinline__ float down_q_row(const float* q4) { return ((q4[0] + q4[1]) + q4[2]) + q4[3]; }

// a[i] for a per-lane i < B.  The empty asm between the selects keeps the chain
// of v_cndmask: folded into a table lookup it would index a private array.
template <int B>
__device__ __forceinline__ float pick(const float (&a)[B], int i) {
    float v = a[0];
#pragma unroll
    for (int b = 1; b < B; ++b) {
        v = (i == b) ? a[b] : v;
        asm volatile("" : "+v"(v));
    }
    return v;
}

__device__ __forceinline__ float silu_mul(float z, float u) { return z / (1.0f + expf(-z)) * u; }

// q . k over 8 dims: fp32 query, bf16 key.
__device__ __forceinline__ float qk8(const float* q, uint4 k) {
    float a = 0.f;
    a = fmaf(q[0], bf_lo(k.x), a);
    a = fmaf(q[1], bf_hi(k.x), a);
    a = fmaf(q[2], bf_lo(k.y), a);
    a = fmaf(q[3], bf_hi(k.y), a);
    a = fmaf(q[4], bf_lo(k.z), a);
    a = fmaf(q[5], bf_hi(k.z), a);
    a = fmaf(q[6], bf_lo(k.w), a);
    a = fmaf(q[7], bf_hi(k.w), a);
    return a;
}

// Greedy order: larger logit first, ties to the lower token id (first maximum).
__device__ __forceinline__ bool head_better(float v, int32_t i, float bv, int32_t bi) {
    return v > bv || (v == bv && i < bi);
}

// ---------------------------------------------------------------------------------------------
// Attention of one (sequence b, KV head g, split s) over the positions of that split.
//
// The G query heads of a KV head read the same keys and values, so each of the
// four compute waves takes a quarter of the positions (every fourth group of
// PPW positions) and scores all G heads on them; each wave keeps its own online
// softmax (running maximum, sum, weighted V) per head, and the four wave
// partials are merged at the end in wave order, as split partials are merged in
// split order.
//
// Score pass: lane -> (position slot ps = lane / LPP, dims dl .. dl + 7 with
// dl = 8 * (lane % LPP)); the per-position dot is summed over the slot's lanes
// with DPP.  Value pass: lane -> dims lane * DPL .. + DPL - 1, one position at a
// time, so no reduction across lanes is needed.
// ---------------------------------------------------------------------------------------------
// Attention item id -> (sequence b, KV head g, split s, q heads h0 .. h0 + gh - 1):
// item = ((b * Hkv + g) * nsplit + s) * hsplit + q-head group.
struct AttnItem {
    int b, g, s, h0, gh;
};
__device__ __forceinline__ AttnItem attn_item_of(const Params& P, uint32_t item) {
    const int hs = (int)item % P.hsplit, it = (int)item / P.hsplit, per_b = P.Hkv * P.nsplit;
    AttnItem r;
    r.b = it / per_b;
    r.g = (it % per_b) / P.nsplit;
    r.s = it % P.nsplit;
    r.gh = P.G / P.hsplit;
    r.h0 = hs * r.gh;
    return r;
}

template <int HD>
struct AttnGeom {
    static constexpr int LPP = HD / 8;    // lanes per position (score pass)
    static constexpr int PPW = 64 / LPP;  // positions per 1 KB group
    static constexpr int DPL = HD / 64;   // dims per lane (value pass)
};

// bf16 values of dims lane * DPL .. + DPL - 1 read from an address (2 or 4 bytes).
template <int DPL>
__device__ __forceinline__ void load_vdims(const char* p, float (&v)[DPL]) {
    if constexpr (DPL == 1) {
        v[0] = bf_to_f(*(const uint16_t*)p);
    } else {
        const uint32_t u = *(const uint32_t*)p;
        v[0] = bf_lo(u);
        v[1] = bf_hi(u);
    }
}

// K/V groups of an attention item in the LDS ring: block(t0) gives the groups
// from t0 on (at most kAttnBlockGroups of them, so one wrap at most).
template <int HD>
struct RingKV {
    const char* ring;
    uint32_t S, nchunks;  // stream byte of the item's first group (group t = [K 1 KB][V 1 KB]), ring size
    struct Block {
        const char* ring;
        uint32_t base, ring_bytes;  // ring byte of group t0
        __device__ __forceinline__ uint32_t addr(uint32_t off) const {
            const uint32_t a = base + off;
            return a >= ring_bytes ? a - ring_bytes : a;
        }
        // this lane's 16-byte piece of K in group t (score-pass mapping)
        __device__ __forceinline__ uint4 k(int t) const {
            return *(const uint4*)(ring + addr((uint32_t)t * 2048u + lane_id() * 16u));
        }
        // this lane's 16-byte piece of V in group t (score-pass mapping)
        __device__ __forceinline__ uint4 vp(int t) const {
            return *(const uint4*)(ring + addr((uint32_t)t * 2048u + 1024u + lane_id() * 16u));
        }
        // this lane's dims of V at position slot `slot` of group t (value-pass mapping)
        __device__ __forceinline__ void v(int t, int slot, float (&out)[AttnGeom<HD>::DPL]) const {
            constexpr int DPL = AttnGeom<HD>::DPL;
            load_vdims<DPL>(ring + addr((uint32_t)t * 2048u + 1024u + (uint32_t)slot * (HD * 2u) +
                                        (uint32_t)lane_id() * (DPL * 2u)),
                            out);
        }
    };
    __device__ __forceinline__ Block block(int t0) const {
        const uint32_t x = S + (uint32_t)t0 * 2048u;
        return Block{ring, ((x >> 10) % nchunks) * 1024u + (x & 1023u), nchunks * 1024u};
    }
    // (cos, sin) entry i of the position's RoPE row (the chunk before group 0)
    __device__ __forceinline__ float2 rope_at(int i) const {
        const uint32_t x = S - 1024u;
        return *(const float2*)(ring + ((x >> 10) % nchunks) * 1024u + (uint32_t)i * 8u);
    }
};

// RoPE table row of one position read straight from the table.
struct GlobalRope {
    const float2* row;
    __device__ __forceinline__ float2 rope_at(int i) const { return row[i]; }
};

// Own position of row b of a step whose rows see `cached` positions: the cached
// length in a decode step; cached + b in a multi-position step, clamped to the
// cache (only ignored rows of a short chunk can pass its end).
__device__ __forceinline__ int attn_pos(const Params& P, int cached, int b) {
    const int p = cached + (P.chunk ? b : 0);
    return p < P.S ? p : P.S - 1;
}
// KV-cache row (sequence) of step row b.
__device__ __forceinline__ int kv_seq(const Params& P, int b) { return P.chunk ? P.chunk_seq : b; }

template <int HD>
struct GlobalKV {
    const uint16_t *kb, *vb;  // cache rows of (layer, b, g): [S][HD]
    int s0, last;             // first position of the split, last valid cached position
    const float2* rope_row;   // (cos, sin) row of the position
    __device__ __forceinline__ int pos(int t, int slot) const {
        int j = s0 + t * AttnGeom<HD>::PPW + slot;
        if (j > last) j = last;
        if (j < 0) j = 0;
        return j;
    }
    __device__ __forceinline__ float2 rope_at(int i) const { return rope_row[i]; }
    struct Block {
        const GlobalKV* kv;
        int t0;
        __device__ __forceinline__ uint4 k(int t) const {
            constexpr int LPP = AttnGeom<HD>::LPP;
            return *(const uint4*)(kv->kb + (size_t)kv->pos(t0 + t, lane_id() / LPP) * HD + 8 * (lane_id() % LPP));
        }
        __device__ __forceinline__ uint4 vp(int t) const {
            constexpr int LPP = AttnGeom<HD>::LPP;
            return *(const uint4*)(kv->vb + (size_t)kv->pos(t0 + t, lane_id() / LPP) * HD + 8 * (lane_id() % LPP));
        }
        __device__ __forceinline__ void v(int t, int slot, float (&out)[AttnGeom<HD>::DPL]) const {
            constexpr int DPL = AttnGeom<HD>::DPL;
            load_vdims<DPL>((const char*)(kv->vb + (size_t)kv->pos(t0 + t, slot) * HD + lane_id() * DPL), out);
        }
    };
    __device__ __forceinline__ Block block(int t0) const { return Block{this, t0}; }
};

// Split geometry of item s for a context of n = p + 1 positions.
struct SplitRange {
    int s0, s1, ncached, ngroups;
    bool has_new;
};
template <int HD>
__device__ __forceinline__ SplitRange split_range(int p, int s, int nsplit) {
    const int n = p + 1;
    const int len = (n + nsplit - 1) / nsplit;
    SplitRange r;
    r.s0 = min(s * len, n);
    r.s1 = min(r.s0 + len, n);
    const int ce = min(r.s1, p);
    r.ncached = max(0, ce - r.s0);
    r.ngroups = (r.ncached + AttnGeom<HD>::PPW - 1) / AttnGeom<HD>::PPW;
    r.has_new = (r.s0 <= p) && (p < r.s1);
    return r;
}

// Merge the softmax partial (m2, l2, acc2) into (m, l, acc); empty partials
// (maximum -inf) contribute nothing.
template <int N>
__device__ __forceinline__ void lse_merge(float& m, float& l, float (&acc)[N], float m2, float l2,
                                          const float (&acc2)[N]) {
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;  // both empty
    const float c1 = (m == -INFINITY) ? 0.f : expf(m - mm);
    const float c2 = (m2 == -INFINITY) ? 0.f : expf(m2 - mm);
    l = l * c1 + l2 * c2;
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    m = mm;
}

// Rotate-half RoPE of dim i of one head whose raw fp32 values start at `raw`
// (LDS): pair (i, i + HD/2) turns by the angle of table entry i mod HD/2.  Every
// read is issued on both halves' paths (no branch around a load), so the reads
// of all dims overlap.
template <int HD, class KV>
__device__ __forceinline__ float rope_dim(const float* raw, const KV& kv, int i) {
    constexpr int half = HD / 2;
    const float x = raw[i], y = raw[i ^ half];  // i ^ half: the partner dim
    const float2 cs = kv.rope_at(i & (half - 1));
    return i < half ? fmaf(x, cs.x, -(y * cs.y)) : fmaf(y, cs.y, x * cs.x);
}

// Sum over the groups of `LPP` consecutive lanes (8 or 16) with DPP: quad
// butterflies, then the half-row mirror (and the row mirror for 16); partners
// add the same two values, so every lane of a group ends with identical bits.
template <int LPP>
__device__ __forceinline__ float group_sum_dpp(float v) {
    static_assert(LPP == 8 || LPP == 16, "8 or 16 lanes per position");
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    if (LPP == 16) v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return v;
}

// group_sum_dpp of N values at once (steps interleaved, results identical).
template <int LPP, int N>
__device__ __forceinline__ void group_sum_dpp_n(float (&v)[N]) {
    static_assert(LPP == 8 || LPP == 16, "8 or 16 lanes per position");
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0xB1, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x4E, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x141, 0xF, 0xF, false);
    if (LPP == 16) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += __builtin_amdgcn_update_dpp(0.0f, v[i], 0x140, 0xF, 0xF, false);
    }
}

// wave_maxf of N values at once (steps interleaved, results identical).
template <int N>
__device__ __forceinline__ void wave_max_n(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0xB1, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0x4E, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0x141, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0x140, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0x142, 0xA, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], __builtin_amdgcn_update_dpp(-INFINITY, v[i], 0x143, 0xC, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// Maximum over the 64 lanes (DPP tree as wave_total), returned to every lane.
__device__ __forceinline__ float wave_maxf(float v) {
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0xB1, 0xF, 0xF, false));
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0x4E, 0xF, 0xF, false));
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0x141, 0xF, 0xF, false));
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0x140, 0xF, 0xF, false));
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0x142, 0xA, 0xF, false));
    v = fmaxf(v, __builtin_amdgcn_update_dpp(-INFINITY, v, 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

static_assert(kAttnBlockGroups % (2 * kComputeWaves) == 0, "groups of a block (full or half) are dealt evenly to the waves");

// Runs one attention item (sequence b, KV head g, split s) with the nw == 4 compute
// waves of the workgroup, which all call it.
//  1. stage the raw q (G heads), k and v of the position (tagged words);
//  2. wave h rotates q head h, wave 0 also k; the new K (rotated) and V are
//     rounded to bf16, appended to the cache and kept in LDS;
//  3. block by block (kAttnBlockGroups groups, half that when the split is
//     longer), wave w scores groups t0 + w, t0 + w + 4, ... for every head as
//     they land, exponentiates against its running maximum and accumulates the
//     weighted V (the new position is one extra group);
//  4. the four wave partials of head h are merged by wave h, in wave order.
// `need(t)` waits for ring group t; `release(t)` frees ring groups before t;
// `barrier()` synchronises the waves.  Writes the attention output (tagged) or,
// when split, the item's (max, sum, output) partial; the last split to arrive
// merges all partials in split order.
// Positions: p is the row's own position (RoPE of q, where its K/V is appended),
// pc the cached positions it attends to from the cache (the context length at
// launch), and the nnew new positions pc, pc + 1, ..., p are the rows b - nnew + 1
// .. b of the step (one, p = pc, in a decode step; rows 0 .. b of one sequence in
// a multi-position step), taken from this step's projections rather than the
// cache; kvb is the cache row (sequence) and `append` says whether the row stores
// its K/V.  CH: compiled for multi-position steps (nnew up to kChunkRows); the
// decode kernels keep one new position and its smaller register and LDS footprint.
template <int HD, bool CH, class KV, class Need, class Release, class Barrier, class Mark>
__device__ __forceinline__ bool attn_item(const Params& P, uint32_t tag0, int layer, int b, int g, int s, int h0, int gh, int p,
                                          int pc, int nnew, int kvb, bool append, const KV& kv, Need& need,
                                          Release& release, Barrier& barrier, float* xs, int wave, int nw, Spin& spin,
                                          Mark& mark) {
    using Geo = AttnGeom<HD>;
    constexpr int LPP = Geo::LPP, PPW = Geo::PPW, DPL = Geo::DPL;
    constexpr int GW = kAttnBlockGroups / kComputeWaves;  // groups per wave per block
    static_assert(GW * PPW <= kAttnWavePositions, "a wave's positions of one block fit its score area");
    const int lane = lane_id();
    const int ps = lane / LPP;
    const int dl = 8 * (lane % LPP);
    const int G = gh;  // q heads h0 .. h0 + gh - 1 of the KV head's P.G
    const SplitRange R = split_range<HD>(pc, s, P.nsplit);
    constexpr int NM = CH ? kChunkRows : 1;                       // new-position rows the LDS layout holds
    constexpr int NGM = CH ? (kChunkRows + PPW - 1) / PPW : 1;    // groups of new positions at most
    static_assert(NGM <= 2, "new positions fill at most two groups");
    if constexpr (!CH) nnew = 1;
    const int NG = (nnew + PPW - 1) / PPW;  // groups of new positions
    const float scale = P.attn_scale;
    const uint32_t tag_in = phase_tag(tag0, layer, 0) ^ ((P.inject && layer == 0) ? 0x80000000u : 0u);
    const uint32_t tag_out = phase_tag(tag0, layer, 1);
    const uint32_t stride = HD + 2;

    // LDS: raw q [G][HD], k [NM][HD], v [NM][HD]; rotated q [G][HD]; new K and V
    // (bf16, [NM][HD]); scores [wave][64][4]; wave partials [wave][G][2 + 4 HD];
    // split partials [split][G][HD + 2].
    float* q_raw = xs;
    float* k_raw = q_raw + G * HD;
    float* v_raw = k_raw + NM * HD;
    float* q_rot = v_raw + NM * HD;
    uint16_t* k_new = (uint16_t*)(q_rot + G * HD);
    uint16_t* v_new = k_new + NM * HD;
    float* sc = (float*)(v_new + NM * HD) + wave * kAttnWavePositions * kMaxGroup;
    float* wpart = (float*)(v_new + NM * HD) + kComputeWaves * kAttnWavePositions * kMaxGroup;
    float* spart = wpart + kComputeWaves * G * (4 * HD + 2);
    uint32_t* flag = (uint32_t*)(spart + P.nsplit * G * stride);

    // the (cos, sin) row of position p (for the ring: the item's first chunk)
    if (!need(-1)) return false;
    {
        const uint64_t* row = P.qkv + (size_t)b * P.qkv_rows;
        const uint64_t* row0 = P.qkv + (size_t)(b - nnew + 1) * P.qkv_rows;  // first new-position row
        const uint32_t nr = (uint32_t)nnew, qs = (uint32_t)P.qkv_rows;
        float ss[1] = {0.f};
        const StageSeg sg[3] = {{row + (size_t)(g * P.G + h0) * HD, q_raw, nullptr, (uint32_t)(G * HD), 1u, 0u, 0u, tag_in},
                                {row0 + (size_t)(P.Hq + g) * HD, k_raw, nullptr, (uint32_t)HD, nr, qs, (uint32_t)HD, tag_in},
                                {row0 + (size_t)(P.Hq + P.Hkv + g) * HD, v_raw, nullptr, (uint32_t)HD, nr, qs, (uint32_t)HD,
                                 tag_in}};
        if (!stage_segs<kStagePassWords, 1, 3>(sg, wave, nw, spin, ss)) return false;
    }
    if (!barrier()) return false;
    mark(0);

    // rotations (lane -> dims lane * DPL + j) and the KV append
    if (wave < G) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int i = lane * DPL + j;
            q_rot[wave * HD + i] = rope_dim<HD>(q_raw + wave * HD, kv, i);
        }
    }
    if (wave == 0) {
        uint32_t kw = 0, vw = 0;
        if constexpr (CH) {
            // earlier new positions of a multi-position step: K rotated at position
            // pc + r (table rows read directly; the ring carries the row of p only)
            for (int r = 0; r + 1 < nnew; ++r) {
                const GlobalRope grp{P.rope + (size_t)min(pc + r, P.S - 1) * (HD / 2)};
#pragma unroll
                for (int j = 0; j < DPL; ++j) {
                    const int i = lane * DPL + j;
                    k_new[r * HD + i] = (uint16_t)f_to_bf(rope_dim<HD>(k_raw + r * HD, grp, i));
                    v_new[r * HD + i] = (uint16_t)f_to_bf(v_raw[r * HD + i]);
                }
            }
        }
        const int own = nnew - 1;  // this row's new position
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int i = lane * DPL + j;
            const uint32_t kb16 = f_to_bf(rope_dim<HD>(k_raw + own * HD, kv, i));
            const uint32_t vb16 = f_to_bf(v_raw[own * HD + i]);
            k_new[own * HD + i] = (uint16_t)kb16;
            v_new[own * HD + i] = (uint16_t)vb16;
            kw |= kb16 << (16 * j);
            vw |= vb16 << (16 * j);
        }
        if (R.has_new && h0 == 0 && append) {  // KV append at position p (read by later steps), once per KV head
            const size_t row = ((((size_t)layer * P.kv_b + kvb) * P.Hkv + g) * P.S + p) * HD + lane * DPL;
            if constexpr (DPL == 1) {
                P.kcache[row] = (uint16_t)kw;
                P.vcache[row] = (uint16_t)vw;
            } else {
                *(uint32_t*)(P.kcache + row) = kw;
                *(uint32_t*)(P.vcache + row) = vw;
            }
        }
    }
    if (!barrier()) return false;

    // this lane's 8 dims of every rotated q head, and of the new K and V
    float q[kMaxGroup][8];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        const int hh = h < G ? h : 0;
        const float4 a = *(const float4*)(q_rot + hh * HD + dl);
        const float4 c = *(const float4*)(q_rot + hh * HD + dl + 4);
        q[h][0] = a.x; q[h][1] = a.y; q[h][2] = a.z; q[h][3] = a.w;
        q[h][4] = c.x; q[h][5] = c.y; q[h][6] = c.z; q[h][7] = c.w;
    }
    // this lane's slot of the new positions' groups (slots past nnew repeat the last)
    uint4 kn[NGM], vn[NGM];
#pragma unroll
    for (int n = 0; n < NGM; ++n) {
        const int r = min(n * PPW + ps, nnew - 1);
        kn[n] = *(const uint4*)(k_new + r * HD + dl);
        vn[n] = *(const uint4*)(v_new + r * HD + dl);
    }

    const int ngr = R.ngroups + (R.has_new ? NG : 0);  // ring groups, then the new positions' groups
    // running maximum and sum per head (wave-uniform), weighted V per (slot, 8 dims)
    float m_run[kMaxGroup], l_run[kMaxGroup], acc[kMaxGroup][8];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    // A split of at most kAttnBlockGroups groups is one block (one rescale); a
    // longer one goes in half-size blocks, so the ring holds the next block
    // streaming in while the waves work on the current one.
    const int bg = ngr <= kAttnBlockGroups ? kAttnBlockGroups : kAttnBlockGroups / 2;
    for (int t0 = 0; t0 < ngr; t0 += bg) {
        const int t1 = min(ngr, t0 + bg);
        const auto blk = kv.block(t0);
        // this wave's groups of the block: t0 + wave + 4 i, i < ngw
        const int first = t0 + wave;
        const int ngw = first < t1 ? (t1 - first + kComputeWaves - 1) / kComputeWaves : 0;
        const int own_last = first + kComputeWaves * (ngw - 1);
        // scores of every head, two groups per step.  Each step first waits for its
        // own ring groups only: the loader fills a block in stream order, so a wave
        // starts on the groups that have landed while the rest arrive.  Loads are
        // issued for every step, from the wave's last group when the step is past
        // its groups (so they read resident data) or from the new position's slot,
        // and the values selected afterwards.
        float mx[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) mx[h] = -INFINITY;
        for (int i = 0; i < ngw; i += 2) {
            const int tl = min(first + kComputeWaves * min(i + 1, ngw - 1), R.ngroups - 1);
            if (tl >= t0 && !need(tl)) return false;
            uint4 kp[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = first + kComputeWaves * (i + u);
                const uint4 kr = blk.k(min(tt, own_last) - t0);
                kp[u] = (tt < R.ngroups) ? kr : (tt == R.ngroups ? kn[0] : kn[NGM - 1]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = first + kComputeWaves * (i + u);
                const bool valid = (i + u < ngw) && (tt >= R.ngroups ? (tt - R.ngroups) * PPW + ps < nnew
                                                                      : tt * PPW + ps < R.ncached);
                float v4[kMaxGroup];
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h) v4[h] = qk8(q[h], kp[u]);
                group_sum_dpp_n<LPP, kMaxGroup>(v4);
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h) {
                    const float v = (valid && h < G) ? v4[h] * scale : -INFINITY;
                    v4[h] = v;
                    mx[h] = fmaxf(mx[h], v);
                }
                if (dl == 0 && i + u < ngw)
                    *(float4*)(sc + ((i + u) * PPW + ps) * kMaxGroup) = make_float4(v4[0], v4[1], v4[2], v4[3]);
            }
        }
        const int npw = ngw * PPW;  // this wave's positions in the block
        float m_new[kMaxGroup], c[kMaxGroup];
        wave_max_n<kMaxGroup>(mx);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            m_new[h] = fmaxf(m_run[h], mx[h]);
            c[h] = m_run[h] == -INFINITY ? 0.f : expf(m_run[h] - m_new[h]);
        }
        // weights against the running maximum (lane = position), and their sums
        float l_blk[kMaxGroup];
        {
            float4 e4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (lane < npw) {
                const float4 v = *(const float4*)(sc + lane * kMaxGroup);
                e4.x = v.x == -INFINITY ? 0.f : expf(v.x - m_new[0]);
                e4.y = v.y == -INFINITY ? 0.f : expf(v.y - m_new[1]);
                e4.z = v.z == -INFINITY ? 0.f : expf(v.z - m_new[2]);
                e4.w = v.w == -INFINITY ? 0.f : expf(v.w - m_new[3]);
                *(float4*)(sc + lane * kMaxGroup) = e4;
            }
            l_blk[0] = e4.x;
            l_blk[1] = e4.y;
            l_blk[2] = e4.z;
            l_blk[3] = e4.w;
            wave_total_n<kMaxGroup>(l_blk);
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            l_run[h] = l_run[h] * c[h] + l_blk[h];
            m_run[h] = m_new[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= c[h];
        }
        // weighted V: lane (slot, 8 dims) takes its slot's position of each group
        for (int i = 0; i < ngw; i += 2) {
            uint4 vp[2];
            float4 w4[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tt = first + kComputeWaves * (i + u);
                const uint4 vr = blk.vp(min(tt, own_last) - t0);
                const float4 w = *(const float4*)(sc + (min(i + u, ngw - 1) * PPW + ps) * kMaxGroup);
                vp[u] = (tt < R.ngroups) ? vr : (tt == R.ngroups ? vn[0] : vn[NGM - 1]);
                w4[u] = (i + u < ngw) ? w : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float wv[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
                const float v8[8] = {bf_lo(vp[u].x), bf_hi(vp[u].x), bf_lo(vp[u].y), bf_hi(vp[u].y),
                                     bf_lo(vp[u].z), bf_hi(vp[u].z), bf_lo(vp[u].w), bf_hi(vp[u].w)};
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wv[h], v8[e], acc[h][e]);
            }
        }
        release(min(t1, R.ngroups));
    }
    mark(1);

    // Wave partials -> LDS: the slots of a 16-lane row are summed with DPP (8
    // lanes per position: the two slots of the row), then each row's 8-dim pieces
    // are stored; [wave][head]: maximum, sum, 4 rows of HD.
    constexpr uint32_t wstride = 2 + 4 * HD;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (LPP == 8) acc[h][e] += __builtin_amdgcn_update_dpp(0.0f, acc[h][e], 0x128, 0xF, 0xF, false);  // row_ror:8
    const int row = lane >> 4;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
            float* dst = wpart + (size_t)(wave * G + h) * wstride;
            if (lane == 0) {
                dst[0] = m_run[h];
                dst[1] = l_run[h];
            }
            if (LPP == 16 || (lane & 8) == 0) {
                float* r = dst + 2 + row * HD + dl;
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = acc[h][e];
            }
        }
    }
    if (!barrier()) return false;
    const int j = wave;  // q head this wave merges and writes (lane -> dims lane * DPL + e)
    float mm = -INFINITY, ll = 0.f, aa[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) aa[e] = 0.f;
    if (j < G) {
        float pm[kComputeWaves], pl[kComputeWaves], pa[kComputeWaves][DPL];
#pragma unroll
        for (int w = 0; w < kComputeWaves; ++w) {
            const float* src = wpart + (size_t)(w * G + j) * wstride;
            pm[w] = src[0];
            pl[w] = src[1];
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane * DPL + e;
                pa[w][e] = (src[2 + d] + src[2 + HD + d]) + (src[2 + 2 * HD + d] + src[2 + 3 * HD + d]);
            }
        }
        // one common maximum, then every wave's share scaled to it (waves whose
        // maximum is -inf saw no position and contribute nothing)
#pragma unroll
        for (int w = 0; w < kComputeWaves; ++w) mm = fmaxf(mm, pm[w]);
        if (mm != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kComputeWaves; ++w) {
                const float cw = pm[w] == -INFINITY ? 0.f : expf(pm[w] - mm);
                ll = fmaf(pl[w], cw, ll);
#pragma unroll
                for (int e = 0; e < DPL; ++e) aa[e] = fmaf(pa[w][e], cw, aa[e]);
            }
        }
    }
    uint64_t* out_b = P.attn + (size_t)b * P.Hq * HD;
    if (P.nsplit == 1) {
        if (j < G) {
            const float inv = 1.0f / ll;
            uint64_t* o = out_b + (size_t)(g * P.G + h0 + j) * HD + lane * DPL;
#pragma unroll
            for (int e = 0; e < DPL; ++e) st_tagged(o + e, aa[e] * inv, tag_out);
        }
        mark(2);
        return true;
    }
    // split: publish the partial; the last split to arrive merges all of them
    const size_t pstride = (size_t)G * stride;
    uint64_t* part = P.attn_part + (((size_t)b * P.Hkv + g) * P.nsplit) * pstride;
    uint32_t* tk = P.attn_ticket + (((size_t)layer * P.B + b) * P.Hkv + g) * kCtrStride;
    if (j < G) {
        uint64_t* dst = part + (size_t)s * pstride + (size_t)j * stride;
        if (lane == 0) {
            st_tagged(dst, mm, tag_out);
            st_tagged(dst + 1, ll, tag_out);
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) st_tagged(dst + 2 + lane * DPL + e, aa[e], tag_out);
    }
    if (!barrier()) return false;  // every head's partial is issued
    if (wave == 0) {
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0, 64);
        if (lane == 0) *flag = (old == (uint32_t)P.nsplit - 1u) ? 1u : 0u;
    }
    if (!barrier()) return false;
    if (*flag == 0u) {
        mark(2);
        return true;
    }
    // last arrival: every wave stages the partials, wave j merges head j in split order
    {
        float ss[1] = {0.f};
        const StageSeg sg[1] = {{part, spart, nullptr, (uint32_t)(P.nsplit * pstride), 1u, 0u, 0u, tag_out}};
        if (!stage_segs<kStagePassWords, 1, 1>(sg, wave, nw, spin, ss)) return false;
    }
    if (!barrier()) return false;
    if (j < G) {
        const float* s0p = spart + (size_t)j * stride;
        float m2 = s0p[0], l2 = s0p[1], a2[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) a2[e] = s0p[2 + lane * DPL + e];
        for (int sp = 1; sp < P.nsplit; ++sp) {
            const float* src = spart + (size_t)sp * pstride + (size_t)j * stride;
            float a3[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) a3[e] = src[2 + lane * DPL + e];
            lse_merge(m2, l2, a2, src[0], src[1], a3);
        }
        const float inv = 1.0f / l2;
        uint64_t* o = out_b + (size_t)(g * P.G + h0 + j) * HD + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) st_tagged(o + e, a2[e] * inv, tag_out);
    }
    if (wave == 0 && lane == 0) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mark(2);
    return true;
}

// ---------------------------------------------------------------------------------------------
// LM head: every compute wave publishes its argmax partial (value, index) tagged;
// the last wave to arrive on the ticket reduces all partials, writes the greedy
// tokens and advances the context lengths.  A NaN logit travels as a NaN partial.
// ---------------------------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ bool head_publish(const Params& P, const StepArgs& A, uint32_t slot, const float (&bv)[B],
                                             const int32_t (&bi)[B], Spin& spin) {
    const int lane = lane_id();
    const uint32_t tag = phase_tag(A.tag0, P.L, 0);
    if (lane < B) {
        uint64_t* dst = P.head_part + ((size_t)slot * P.B + lane) * 2;
        int32_t i = bi[0];
#pragma unroll
        for (int b = 1; b < B; ++b) {
            i = (lane == b) ? bi[b] : i;
            asm volatile("" : "+v"(i));
        }
        st_tagged(dst, pick<B>(bv, lane), tag);
        st_tagged(dst + 1, __int_as_float(i), tag);
    }
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(P.head_ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != P.n_head_slots - 1u) return true;
    // last wave of the step
    bool nan_seen = false;
    for (int b = 0; b < B; ++b) {
        float best = -INFINITY;
        int32_t besti = 0x7FFFFFFF;
        for (uint32_t k0 = 0; k0 < P.n_head_slots; k0 += 64u * kStageWords / 2) {
            uint64_t w[kStageWords];
#pragma unroll
            for (int i = 0; i < kStageWords; ++i) {
                const uint32_t k = k0 + (uint32_t)lane + 64u * (uint32_t)(i / 2);
                w[i] = k < P.n_head_slots ? ld_tagged(P.head_part + ((size_t)k * P.B + b) * 2 + (i & 1))
                                          : ((uint64_t)tag << 32);
            }
            spin.start();
            for (;;) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < kStageWords; ++i) ok &= tv_tag(w[i]) == tag;
                if (__all(ok)) break;
                if (!spin.again(tag, k0)) return false;
#pragma unroll
                for (int i = 0; i < kStageWords; ++i) {
                    const uint32_t k = k0 + (uint32_t)lane + 64u * (uint32_t)(i / 2);
                    if (tv_tag(w[i]) != tag) w[i] = ld_tagged(P.head_part + ((size_t)k * P.B + b) * 2 + (i & 1));
                }
            }
#pragma unroll
            for (int i = 0; i < kStageWords; i += 2) {
                const uint32_t k = k0 + (uint32_t)lane + 64u * (uint32_t)(i / 2);
                if (k < P.n_head_slots) {
                    const float v = tv_val(w[i]);
                    const int32_t idx = __float_as_int(tv_val(w[i + 1]));
                    if (v != v) nan_seen = true;
                    if (head_better(v, idx, best, besti)) {
                        best = v;
                        besti = idx;
                    }
                }
            }
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
            const float ov = __shfl_xor(best, msk, 64);
            const int32_t oi = __shfl_xor(besti, msk, 64);
            if (head_better(ov, oi, best, besti)) {
                best = ov;
                besti = oi;
            }
        }
        if (lane == 0) A.tok_out[b] = besti;
    }
    if (P.chunk) {
        if (lane == 0) P.ctx_len[P.chunk_seq] = P.ctx_len[P.chunk_seq] + A.tok_rows;
    } else if (lane < B) {
        P.ctx_len[lane] = P.ctx_len[lane] + 1;
    }
    if (lane == 0) __hip_atomic_store(P.head_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__any(nan_seen)) raise_error_impl(P.state, P.host_err, spin.abort_flag, DERR_NAN, 0, 0);
    return true;
}

}  // namespace mk
