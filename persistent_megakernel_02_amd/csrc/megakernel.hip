// The persistent decode megakernel: one launch runs a whole decode step.
//
// Design (page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "Megakernel：从零设计的深度融合方案", re-made for CDNA4):
//  - one workgroup per compute unit walks that CU's instruction queue, built on
//    the host before launch (the per-SM plan);
//  - shared memory cut into pages lets the next instructions' weights load while
//    the current one computes: here one LOADER wave streams the CU's weight and
//    KV bytes HBM -> LDS with 16-byte-per-lane direct-to-LDS loads
//    (global_load_lds_dwordx4) into a 128 KB ring, ahead of the four COMPUTE
//    waves, and keeps streaming while they wait on dependencies;
//  - dependencies are global-memory counters: the last wave of a CU to finish an
//    instruction releases its results and increments the instruction's counter;
//    a dependant spins (one relaxed agent-scope load per poll, s_sleep between
//    polls) until counter >= epoch * producers, then acquires.  Counters are
//    monotonic across steps, so nothing is reset between launches;
//  - every spin is bounded by a watchdog (s_memrealtime, 100 MHz): on expiry the
//    CU records an error and all waves leave, so a launch always terminates.
//
// The loader's vector-memory instructions are only these LDS loads, so its
// vmcnt counter counts exactly the chunks in flight; it publishes progress in
// LDS after `s_waitcnt vmcnt(N)`.  Compute waves publish, per wave, the first
// ring chunk they still need; the loader reuses ring space below the minimum.
#include <hip/hip_runtime.h>

#include "mk_device.h"

namespace mk {

struct Ctl {
    uint32_t landed;                     // chunks of the stream resident in the ring
    uint32_t consumed[kComputeWaves];    // first chunk each compute wave still needs
    uint32_t done;                       // instruction completions (monotonic, per wave)
    uint32_t bar;                        // compute-wave barrier arrivals (monotonic)
    uint32_t abort;                      // set when a wave gives up (error)
    int32_t ctx[kMaxBatch];              // context lengths at launch
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

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

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t align_chunk(uint32_t b) { return (b + kChunk - 1u) & ~(kChunk - 1u); }

// Bytes of the CU stream that instruction `in` consumes.
template <int HD>
__device__ __forceinline__ uint32_t instr_bytes(const Params& P, const Instr& in, const int32_t* ctx) {
    switch (in.op) {
        case OP_QKV:
        case OP_HEAD: return align_chunk(in.count * (uint32_t)P.d * 2u);
        case OP_O: return align_chunk(in.count * (uint32_t)(P.Hq * HD) * 2u);
        case OP_GATEUP: return align_chunk(2u * in.count * (uint32_t)P.d * 2u);
        case OP_DOWN: return align_chunk(in.count * (uint32_t)P.F * 2u);
        case OP_ATTN: {
            const int per_b = P.Hkv * P.nsplit;
            const int b = (int)in.begin / per_b, s = (int)in.begin % P.nsplit;
            const SplitRange R = split_range<HD>(ctx[b], s, P.nsplit);
            return (uint32_t)R.ngroups * 2u * kChunk;
        }
        default: return 0;
    }
}

// Global source address of this lane's 16 bytes of chunk c of instruction `in`.
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
        case OP_HEAD: {
            const uint32_t rb = (uint32_t)P.d * 2u;
            uint32_t r = off / rb, col = off - r * rb;
            if (r >= in.count) { r = 0; col = 0; }
            return (const char*)(P.head + (size_t)(in.begin + r) * P.d) + col;
        }
        case OP_ATTN: {
            constexpr uint32_t rbkv = HD * 2u;
            const int per_b = P.Hkv * P.nsplit;
            const int b = (int)in.begin / per_b, g = ((int)in.begin % per_b) / P.nsplit, s = (int)in.begin % P.nsplit;
            const SplitRange R = split_range<HD>(ctx[b], s, P.nsplit);
            const uint32_t t = off >> 11, w = off & 2047u, inner = w & 1023u;
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
__device__ __forceinline__ void dma_chunk(const char* src, uint32_t lds_addr) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
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
        "global_load_lds_dwordx4 %0, %1 offset:0"
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
//    `per` chunks of each in turn;
//  - the K and V blocks of consecutive position groups interleaved (ATTN), one
//    chunk each, lanes past the cached positions re-reading the block start.
// Only pointers and chunk counts, all wave-uniform, so the loop runs on SGPRs.
struct Stream {
    const char* p[3];
    uint32_t n[3];    // chunks per range (ranges), or pairs (interleaved)
    uint32_t per;     // interleaved: chunks of each matrix per turn; 0 = ranges
    int ncached;      // ATTN: valid positions of the split
    bool attn;
};

template <int HD>
__device__ __forceinline__ bool setup_stream(const Params& P, const Instr& in, const DevLayer& Lw, const int32_t* ctx,
                                             Stream& S) {
    S.per = 0;
    S.attn = false;
    S.ncached = 0;
    S.n[1] = S.n[2] = 0;
    S.p[1] = S.p[2] = nullptr;
    uint32_t rb = 0;
    switch (in.op) {
        case OP_QKV: {
            rb = (uint32_t)P.d * 2u;
            const uint32_t nq = (uint32_t)(P.Hq * HD), nk = (uint32_t)(P.Hkv * HD);
            const uint32_t r0 = in.begin, r1 = in.begin + in.count;
            const uint32_t q0 = min(r0, nq), q1 = min(r1, nq);
            const uint32_t k0 = min(max(r0, nq), nq + nk) - nq, k1 = min(max(r1, nq), nq + nk) - nq;
            const uint32_t v0 = max(r0, nq + nk) - nq - nk, v1 = max(r1, nq + nk) - nq - nk;
            S.p[0] = (const char*)Lw.wq + (size_t)q0 * rb; S.n[0] = q1 - q0;
            S.p[1] = (const char*)Lw.wk + (size_t)k0 * rb; S.n[1] = k1 - k0;
            S.p[2] = (const char*)Lw.wv + (size_t)v0 * rb; S.n[2] = v1 - v0;
            break;
        }
        case OP_O:
            rb = (uint32_t)(P.Hq * HD) * 2u;
            S.p[0] = (const char*)Lw.wo + (size_t)in.begin * rb; S.n[0] = in.count;
            break;
        case OP_DOWN:
            rb = (uint32_t)P.F * 2u;
            S.p[0] = (const char*)Lw.w_down + (size_t)in.begin * rb; S.n[0] = in.count;
            break;
        case OP_HEAD:
            rb = (uint32_t)P.d * 2u;
            S.p[0] = (const char*)P.head + (size_t)in.begin * rb; S.n[0] = in.count;
            break;
        case OP_GATEUP:
            rb = (uint32_t)P.d * 2u;
            S.p[0] = (const char*)Lw.w_gate + (size_t)in.begin * rb;
            S.p[1] = (const char*)Lw.w_up + (size_t)in.begin * rb;
            S.n[0] = in.count;
            S.per = rb / kChunk;
            return (rb & (kChunk - 1u)) == 0;
        case OP_ATTN: {
            const int per_b = P.Hkv * P.nsplit;
            const int b = (int)in.begin / per_b, g = ((int)in.begin % per_b) / P.nsplit, s = (int)in.begin % P.nsplit;
            const SplitRange Rg = split_range<HD>(ctx[b], s, P.nsplit);
            const size_t base = ((((size_t)in.layer * P.kv_b + b) * P.Hkv + g) * P.S + Rg.s0) * HD;
            S.p[0] = (const char*)(P.kcache + base);
            S.p[1] = (const char*)(P.vcache + base);
            S.n[0] = (uint32_t)Rg.ngroups;
            S.per = 1;
            S.ncached = Rg.ncached;
            S.attn = true;
            return true;
        }
        default: return false;
    }
    if (rb & (kChunk - 1u)) return false;  // fast path needs whole chunks per row
    const uint32_t cpr = rb / kChunk;
    S.n[0] *= cpr; S.n[1] *= cpr; S.n[2] *= cpr;
    return true;
}

template <int HD>
__device__ void loader_wave(const Params& P, Ctl* ctl, char* ring, uint32_t q0, uint32_t q1, const int32_t* ctx) {
    const uint32_t ring_base = (uint32_t)(size_t)(lds_ptr_t)ring;
    const uint32_t lane16 = (uint32_t)lane_id() * 16u;
    uint32_t issued = 0, landed = 0, limit = kRingChunks;
    bool stop = false;
    // Wait until chunk `issued` may be written into the ring; refreshes `limit`.
    uint32_t stall = 0;
    auto make_room = [&]() -> bool {
        for (;;) {
            limit = min_consumed(ctl) + kRingChunks;
            if (issued < limit) return true;
            const uint32_t ts = P.trace ? (uint32_t)now_ticks() : 0u;
            wait_vmcnt<0>();
            landed = issued;
            lds_st(&ctl->landed, landed);
            if (lds_ld(&ctl->abort)) return false;
            __builtin_amdgcn_s_sleep(1);
            if (P.trace) stall += (uint32_t)now_ticks() - ts;
        }
    };
    auto issue_s = [&](const char* base, uint32_t voff) {
        dma_chunk_s(base, voff, ring_base + (issued % kRingChunks) * kChunk);
        ++issued;
        if (issued - landed > (uint32_t)kLoaderLag) {
            wait_vmcnt<kLoaderLag>();
            landed = issued - kLoaderLag;
            lds_st(&ctl->landed, landed);
        }
    };
    auto issue = [&](const char* src) {
        dma_chunk(src, ring_base + (issued % kRingChunks) * kChunk);
        ++issued;
        if (issued - landed > (uint32_t)kLoaderLag) {
            wait_vmcnt<kLoaderLag>();
            landed = issued - kLoaderLag;
            lds_st(&ctl->landed, landed);
        }
    };
    for (uint32_t i = q0; i < q1 && !stop; ++i) {
        const Instr in = ld_const(P.instrs + i);
        const uint32_t nch = instr_bytes<HD>(P, in, ctx) / kChunk;
        if (P.trace && lane_id() == 0) {
            uint32_t* rec = P.trace + ((size_t)blockIdx.x * P.trace_stride + (i - q0)) * kTraceWords;
            if (i > q0) rec[5 - kTraceWords] = (uint32_t)now_ticks();
            if (i > q0) rec[7 - kTraceWords] = stall;
        }
        stall = 0;
        if (nch == 0) continue;
        const DevLayer Lw = ld_const(P.layers + (in.layer < P.L ? in.layer : 0));
        Stream S;
        if (setup_stream<HD>(P, in, Lw, ctx, S)) {
            if (S.per == 0) {
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const char* base = uniform_ptr(S.p[r]);
                    for (uint32_t c = 0; c < S.n[r] && !stop; ++c) {
                        if (issued >= limit && !make_room()) { stop = true; break; }
                        issue_s(base, c * kChunk + lane16);
                    }
                }
            } else {
                const char* ba = uniform_ptr(S.p[0]);
                const char* bb = uniform_ptr(S.p[1]);
                // ATTN: lanes whose position lies past the cached ones re-read the block start
                const int lane_pos = lane_id() / AttnGeom<HD>::LPP;
                const uint32_t rbytes = S.per * kChunk;
                for (uint32_t r = 0; r < S.n[0] && !stop; ++r) {
                    const bool valid = !S.attn || (int)(r * AttnGeom<HD>::PPW) + lane_pos < S.ncached;
                    const uint32_t lane_off = valid ? lane16 : 0u;
                    for (uint32_t k = 0; k < S.per && !stop; ++k) {
                        if (issued >= limit && !make_room()) { stop = true; break; }
                        issue_s(ba, r * rbytes + k * kChunk + lane_off);
                    }
                    for (uint32_t k = 0; k < S.per && !stop; ++k) {
                        if (issued >= limit && !make_room()) { stop = true; break; }
                        issue_s(bb, r * rbytes + k * kChunk + lane_off);
                    }
                }
            }
        } else {
            for (uint32_t c = 0; c < nch; ++c) {
                if (issued >= limit && !make_room()) { stop = true; break; }
                issue(chunk_src<HD>(P, in, Lw, c, ctx));
            }
        }
    }
    wait_vmcnt<0>();
    lds_st(&ctl->landed, issued);
    if (P.trace && q1 > q0 && lane_id() == 0) {
        P.trace[((size_t)blockIdx.x * P.trace_stride + (q1 - 1 - q0)) * kTraceWords + 5] = (uint32_t)now_ticks();
        P.trace[((size_t)blockIdx.x * P.trace_stride + (q1 - 1 - q0)) * kTraceWords + 7] = stall;
    }
}

// ------------------------------------------------------------------------------------------------
// compute waves
// ------------------------------------------------------------------------------------------------
__device__ __noinline__ void raise_error_impl(DevState* state, HostErr* herr, uint32_t* abort_flag, uint32_t code,
                                             uint32_t a, uint32_t b) {
    __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
__device__ __forceinline__ void raise_error(const Params& P, Ctl* ctl, uint32_t code, uint32_t a, uint32_t b) {
    raise_error_impl(P.state, P.host_err, &ctl->abort, code, a, b);
}

// Spin until the first n completion flags of a phase all hold `epoch` (wrapping
// compare), then acquire at agent scope.  Lane l polls flags l, l + 64, ...
__device__ __forceinline__ bool wait_flags(const Params& P, Ctl* ctl, const uint32_t* flags, uint32_t n,
                                           uint32_t epoch) {
    const uint32_t lane = (uint32_t)lane_id();
    auto ready = [&]() {
        bool ok = true;
        for (uint32_t s = lane; s < n; s += 64u) {
            const uint32_t f = __hip_atomic_load(flags + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok &= (int32_t)(f - epoch) >= 0;
        }
        return __all(ok);
    };
    if (!ready()) {
        const uint64_t t0 = now_ticks();
        uint32_t polls = 0;
        for (;;) {
            __builtin_amdgcn_s_sleep(1);
            if (ready()) break;
            if (lds_ld(&ctl->abort)) return false;
            if ((++polls & 63u) == 0) {
                if (__hip_atomic_load(&P.state->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                    lds_st(&ctl->abort, 1u);
                    return false;
                }
                if (now_ticks() - t0 > P.spin_ticks) {
                    raise_error(P, ctl, DERR_TIMEOUT, epoch, n);
                    return false;
                }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

// Wait until the loader has `need` chunks resident; adds the ticks spent waiting
// to `waited` (read only by the trace).
__device__ __forceinline__ bool wait_landed(const Params& P, Ctl* ctl, uint32_t need, uint32_t& waited) {
    if (lds_ld(&ctl->landed) >= need) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        return true;
    }
    const uint64_t t0 = now_ticks();
    uint32_t polls = 0;
    bool ok = true;
    while (lds_ld(&ctl->landed) < need) {
        if (lds_ld(&ctl->abort)) { ok = false; break; }
        if ((++polls & 255u) == 0 && now_ticks() - t0 > P.spin_ticks) {
            raise_error(P, ctl, DERR_TIMEOUT, 0xFFFFFFFFu, need);
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
struct CwBarrier {
    Ctl* ctl;
    const Params* P;
    uint32_t* gen;
    __device__ void operator()() const {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane_id() == 0) __hip_atomic_fetch_add(&ctl->bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t target = (++*gen) * (uint32_t)kComputeWaves;
        const uint64_t t0 = now_ticks();
        uint32_t polls = 0;
        while (lds_ld(&ctl->bar) < target) {
            if (lds_ld(&ctl->abort)) break;
            if ((++polls & 255u) == 0 && now_ticks() - t0 > P->spin_ticks) {
                raise_error(*P, ctl, DERR_TIMEOUT, 0xFFFFFFFEu, target);
                break;
            }
            __builtin_amdgcn_s_sleep(0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
};

// Stream rows [0, nrows) of the current instruction from the ring in batches of
// R consecutive rows; batch t goes to compute wave t mod kComputeWaves, so the
// four waves work on neighbouring rows and the ring span stays small.
template <int B, int R, class X, class Epi>
__device__ __forceinline__ bool gemv_stream(const Params& P, Ctl* ctl, const char* ring, uint32_t S, uint32_t rb,
                                            uint32_t nrows, const X& x, int wave, uint32_t& lw, Epi& epi) {
    const int np = (int)(rb >> 4);
    const RingRows rows{ring, S, rb};
    for (uint32_t r0 = (uint32_t)wave * R; r0 < nrows; r0 += (uint32_t)R * kComputeWaves) {
        const uint32_t nr = min((uint32_t)R, nrows - r0);
        const uint32_t off = S + r0 * rb;
        set_consumed(ctl, wave, off / kChunk);
        if (!wait_landed(P, ctl, (off + nr * rb + kChunk - 1u) / kChunk, lw)) return false;
        float res[R][B];
        rows_dot<B, R>(rows, r0, (int)nr, np, x, res);
        epi(r0, nr, res);
    }
    return true;
}

template <int B, int HD>
__device__ void compute_wave(const Params& P, const StepArgs& A, Ctl* ctl, const char* ring, float* xlds,
                             float* attn_lds, int wave, uint32_t q0, uint32_t q1, const int32_t* ctx) {
    const int lane = lane_id();
    uint32_t S = 0, k = 0, bar_gen = 0;
    float best_v[B];
    int32_t best_i[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        best_v[b] = -INFINITY;
        best_i[b] = 0x7FFFFFFF;
    }
    bool nan_seen = false;
    for (uint32_t qi = q0; qi < q1; ++qi, ++k) {
        const Instr in = ld_const(P.instrs + qi);
        const uint32_t bytes = instr_bytes<HD>(P, in, ctx);
        uint32_t* tr = (P.trace && wave == 0) ? P.trace + ((size_t)blockIdx.x * P.trace_stride + k) * kTraceWords : nullptr;
        if (tr && lane == 0) {
            tr[0] = (uint32_t)in.op | ((uint32_t)in.layer << 16);
            tr[1] = (uint32_t)now_ticks();
        }
        if (in.wait_ctr != kNoCounter) {
            if (!wait_flags(P, ctl, P.flags + (size_t)in.wait_ctr * P.flag_stride, in.wait_n, A.epoch)) return;
        }
        if (tr && lane == 0) tr[2] = (uint32_t)now_ticks();
        uint32_t land_wait = 0;
        const int layer = in.layer;
        const DevLayer Lw = ld_const(P.layers + (layer < P.L ? layer : 0));
        bool ok = true;
        switch (in.op) {
            case OP_QKV:
            case OP_GATEUP:
            case OP_HEAD: {
                const uint16_t* gain = in.op == OP_QKV ? Lw.attn_norm : in.op == OP_GATEUP ? Lw.mlp_norm : P.final_norm;
                const bool from_embed = (in.op == OP_QKV && layer == 0);
                rmsnorm_rows<B>(P.h, from_embed ? P.embed : nullptr, A.tok_in, A.tok_stride, P.V, gain, P.d, P.eps, xlds);
                const uint32_t rb = (uint32_t)P.d * 2u;
                const XLds x{xlds, (uint32_t)P.d};
                const uint32_t nrows = in.op == OP_GATEUP ? 2u * in.count : in.count;
                auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                    if (in.op == OP_GATEUP) {
                        for (uint32_t i = 0; i + 1 < nr; i += 2) {
                            const uint32_t f = in.begin + (r0 + i) / 2u;
                            if (lane < B) P.act[(size_t)lane * P.F + f] = silu_mul(pick<B>(res[i], lane), pick<B>(res[i + 1], lane));
                        }
                    } else if (in.op == OP_QKV) {
                        for (uint32_t i = 0; i < nr; ++i)
                            if (lane < B) P.qkv[(size_t)lane * P.qkv_rows + in.begin + r0 + i] = pick<B>(res[i], lane);
                    } else {
                        for (uint32_t i = 0; i < nr; ++i) {
                            const int32_t row = (int32_t)(in.begin + r0 + i);
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const float v = res[i][b];
                                if (v != v) nan_seen = true;
                                if (head_better(v, row, best_v[b], best_i[b])) {
                                    best_v[b] = v;
                                    best_i[b] = row;
                                }
                            }
                            if (lane < B) A.logits[(size_t)lane * P.V + row] = pick<B>(res[i], lane);
                        }
                    }
                };
                if (rows_per_batch(rb) == 4) ok = gemv_stream<B, 4>(P, ctl, ring, S, rb, nrows, x, wave, land_wait, epi);
                else ok = gemv_stream<B, 2>(P, ctl, ring, S, rb, nrows, x, wave, land_wait, epi);
                break;
            }
            case OP_O:
            case OP_DOWN: {
                const uint32_t K = in.op == OP_O ? (uint32_t)(P.Hq * HD) : (uint32_t)P.F;
                const uint32_t rb = K * 2u;
                const XGlobal x{in.op == OP_O ? P.attn : P.act, K};
                auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
                    for (uint32_t i = 0; i < nr; ++i) {
                        const uint32_t row = in.begin + r0 + i;
                        if (lane < B) {
                            float* hp = P.h + (size_t)lane * P.d + row;
                            const float resid = (in.op == OP_O && layer == 0)
                                                    ? bf_to_f(P.embed[token_row(A.tok_in, lane, A.tok_stride, P.V) * P.d + row])
                                                    : *hp;
                            *hp = resid + pick<B>(res[i], lane);
                        }
                    }
                };
                const int R = rows_per_batch(rb);
                if (R == 4) ok = gemv_stream<B, 4>(P, ctl, ring, S, rb, in.count, x, wave, land_wait, epi);
                else if (R == 2) ok = gemv_stream<B, 2>(P, ctl, ring, S, rb, in.count, x, wave, land_wait, epi);
                else ok = gemv_stream<B, 1>(P, ctl, ring, S, rb, in.count, x, wave, land_wait, epi);
                break;
            }
            case OP_ATTN: {
                const int per_b = P.Hkv * P.nsplit;
                const int b = (int)in.begin / per_b, g = ((int)in.begin % per_b) / P.nsplit,
                          s = (int)in.begin % P.nsplit;
                const int p = ctx[b];
                const RingKV kv{ring, S};
                auto need = [&](int t) {
                    const uint32_t off = S + (uint32_t)t * 2048u;
                    set_consumed(ctl, wave, off / kChunk);
                    if (!wait_landed(P, ctl, (off + 2048u) / kChunk, land_wait)) ok = false;
                };
                const CwBarrier barrier{ctl, &P, &bar_gen};
                bool merged = false;
                attn_item<HD>(P, layer, b, g, s, p, kv, need, barrier, attn_lds, wave, kComputeWaves, P.attn_ticket,
                              merged);
                break;
            }
            default: break;
        }
        if (!ok || lds_ld(&ctl->abort)) return;
        if (tr && lane == 0) {
            tr[3] = (uint32_t)now_ticks();
            tr[6] = land_wait;
        }
        S += bytes;
        set_consumed(ctl, wave, S / kChunk);
        if (in.op == OP_HEAD && lane < B) {
            HeadPart hp;
            hp.v = pick<B>(best_v, lane);
            int32_t bi = best_i[0];
#pragma unroll
            for (int b = 1; b < B; ++b)
                if (lane == b) bi = best_i[b];
            hp.i = bi;
            P.head_part[((size_t)blockIdx.x * kComputeWaves + wave) * B + lane] = hp;
        }
        // the last wave of this CU to finish the instruction publishes it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&ctl->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __shfl(old, 0, 64);
        if (old == (k + 1u) * (uint32_t)kComputeWaves - 1u && in.sig_ctr != kNoCounter) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            if (lane == 0)
                __hip_atomic_store(P.flags + (size_t)in.sig_ctr * P.flag_stride + in.slot, A.epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            uint32_t prev = 0;
            if (in.op == OP_HEAD && lane == 0)
                prev = __hip_atomic_fetch_add(P.counters + (size_t)P.head_ctr * kCtrStride, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            prev = __shfl(prev, 0, 64);
            if (in.op == OP_HEAD && prev + 1u == A.epoch * P.n_head_instr) {
                // last CU: greedy choice over every partial, then advance the contexts
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                uint32_t nanf = 0;
                reduce_head_parts(P.head_part, P.n_cu * kComputeWaves, B, A.tok_out, &nanf);
                nanf = __shfl(nanf, 0, 64) | (uint32_t)__any(nanf != 0);
                if (lane < B) P.state->ctx_len[lane] = ctx[lane] + 1;
                if (nanf) raise_error(P, ctl, DERR_NAN, 0, 0);
            }
        }
        if (in.op == OP_HEAD && nan_seen) raise_error(P, ctl, DERR_NAN, 1, blockIdx.x);
        if (tr && lane == 0) tr[4] = (uint32_t)now_ticks();
    }
}

template <int B, int HD>
__global__ void __launch_bounds__(kThreads, 1) mk_megakernel(Params P, StepArgs A) {
    __shared__ __attribute__((aligned(1024))) char ring[kRingBytes];
    constexpr uint32_t kAttnBytes = kComputeWaves * kMaxGroup * (HD + 2) * 4;
    __shared__ __attribute__((aligned(16))) char scratch[kXBytes > kAttnBytes ? kXBytes : kAttnBytes];
    __shared__ Ctl ctl;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (threadIdx.x == 0) {
        ctl.landed = 0;
        for (int w = 0; w < kComputeWaves; ++w) ctl.consumed[w] = 0;
        ctl.done = 0;
        ctl.bar = 0;
        ctl.abort = 0;
    }
    if (threadIdx.x < kMaxBatch) ctl.ctx[threadIdx.x] = (int)threadIdx.x < B ? P.state->ctx_len[threadIdx.x] : 0;
    __syncthreads();
    const uint32_t q0 = ld_const(P.queue_off + blockIdx.x), q1 = ld_const(P.queue_off + blockIdx.x + 1);
    const int32_t* ctx = ctl.ctx;
    if (wave == kComputeWaves) {
        loader_wave<HD>(P, &ctl, ring, q0, q1, ctx);
    } else {
        compute_wave<B, HD>(P, A, &ctl, ring, (float*)scratch, (float*)scratch, wave, q0, q1, ctx);
        if (lds_ld(&ctl.abort)) lds_st(&ctl.abort, 1u);
    }
}

// ------------------------------------------------------------------------------------------------
// host-side launch
// ------------------------------------------------------------------------------------------------
template <int B, int HD>
static hipError_t launch_t(const Params& P, const StepArgs& A, hipStream_t stream) {
    void* args[] = {(void*)&P, (void*)&A};
    return hipLaunchCooperativeKernel((const void*)mk_megakernel<B, HD>, dim3(P.n_cu), dim3(kThreads), args, 0,
                                      stream);
}

hipError_t launch_megakernel(const Params& P, const StepArgs& A, hipStream_t stream) {
    if (P.hd == 64) {
        if (P.B == 1) return launch_t<1, 64>(P, A, stream);
        if (P.B == 2) return launch_t<2, 64>(P, A, stream);
    } else if (P.hd == 128) {
        if (P.B == 1) return launch_t<1, 128>(P, A, stream);
        if (P.B == 2) return launch_t<2, 128>(P, A, stream);
    }
    return hipErrorInvalidValue;
}

bool megakernel_supports(int B, int hd) { return (B == 1 || B == 2) && (hd == 64 || hd == 128); }

}  // namespace mk
