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

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Token ids come from device memory; clamp so a bad id cannot index outside the
// embedding table.
__device__ __forceinline__ size_t token_row(const int32_t* tok, int b, int stride, int V) {
    const int t = tok[b * stride];
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
// Staging: wave w of nw moves elements e = 64 (w + nw i) + lane of a vector into
// LDS, kStageWords words per lane in flight, polling until every tag matches.
// ---------------------------------------------------------------------------------------------
// dst[e] = value of src[e] (optionally times the bf16 gain g[e]); ss gets the
// lane's sum of squares of the raw values in ascending i (RMSNorm statistics).
template <bool GAIN>
__device__ __forceinline__ bool stage_tagged(const uint64_t* __restrict__ src, uint32_t n, uint32_t tag,
                                             float* __restrict__ dst, const uint16_t* __restrict__ g, int w, int nw,
                                             Spin& spin, float& ss) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t step = 64u * (uint32_t)nw;
    // `base` is wave-uniform so every lane takes part in the polls
    for (uint32_t base = 64u * (uint32_t)w; base < n; base += step * kStageWords) {
        uint64_t v[kStageWords];
#pragma unroll
        for (int i = 0; i < kStageWords; ++i) {
            const uint32_t e = base + lane + step * i;
            v[i] = e < n ? ld_tagged(src + e) : ((uint64_t)tag << 32);
        }
        spin.start();
        for (;;) {
            bool ok = true;
#pragma unroll
            for (int i = 0; i < kStageWords; ++i) ok &= tv_tag(v[i]) == tag;
            if (__all(ok)) break;
            if (!spin.again(tag, base)) return false;
#pragma unroll
            for (int i = 0; i < kStageWords; ++i) {
                const uint32_t e = base + lane + step * i;
                if (tv_tag(v[i]) != tag) v[i] = ld_tagged(src + e);
            }
        }
#pragma unroll
        for (int i = 0; i < kStageWords; ++i) {
            const uint32_t e = base + lane + step * i;
            if (e < n) {
                const float x = tv_val(v[i]);
                ss = fmaf(x, x, ss);
                dst[e] = GAIN ? x * bf_to_f(g[e]) : x;
            }
        }
    }
    return true;
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
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) out[i][b] = wave_total(acc[i][b]);
}

// Rows of one compute wave's batch for a row of `rb` bytes: about 8 KB per wave.
__host__ __device__ constexpr int rows_per_batch(uint32_t rb) { return rb <= 2048u ? 4 : rb <= 4096u ? 2 : 1; }

template <int B>
__device__ __forceinline__ float pick(const float (&a)[B], int i) {
    float v = a[0];
#pragma unroll
    for (int b = 1; b < B; ++b)
        if (i == b) v = a[b];
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
// Online softmax per lane, then merges across position groups (butterfly), across
// waves (through LDS, fixed order) and, when split, across splits (fixed order, by
// the last split to finish).
//
// KV sources give the 16-byte piece (8 dims) of K or V at group t for this lane.
// Group t holds PPW consecutive positions; lane -> (position ps = lane / LPP,
// dims dl = 8 * (lane % LPP)).
// ---------------------------------------------------------------------------------------------
template <int HD>
struct AttnGeom {
    static constexpr int LPP = HD / 8;    // lanes per position
    static constexpr int PPW = 64 / LPP;  // positions per 1 KB group
};

// K/V groups of an attention item in the LDS ring: block(t0) gives the groups
// from t0 on (at most kAttnBlockGroups of them, so one wrap at most).
struct RingKV {
    const char* ring;
    uint32_t S, nchunks;  // stream byte of the item's first group (group t = [K 1 KB][V 1 KB]), ring size
    struct Block {
        const char* ring;
        uint32_t base, ring_bytes;  // ring byte of group t0
        __device__ __forceinline__ uint4 at(uint32_t off) const {
            uint32_t a = base + off + lane_id() * 16u;
            a = a >= ring_bytes ? a - ring_bytes : a;
            return *(const uint4*)(ring + a);
        }
        __device__ __forceinline__ uint4 k(int t) const { return at((uint32_t)t * 2048u); }
        __device__ __forceinline__ uint4 v(int t) const { return at((uint32_t)t * 2048u + 1024u); }
    };
    __device__ __forceinline__ Block block(int t0) const {
        const uint32_t x = S + (uint32_t)t0 * 2048u;
        return Block{ring, ((x >> 10) % nchunks) * 1024u + (x & 1023u), nchunks * 1024u};
    }
    // (cos, sin) entries i0 .. i0 + 7 of the position's RoPE row, the chunk before group 0
    __device__ __forceinline__ void rope(int i0, float2 (&cs)[8]) const {
        const uint32_t x = S - 1024u;
        const float4* q = (const float4*)(ring + ((x >> 10) % nchunks) * 1024u + (uint32_t)i0 * 8u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 v = q[e];
            cs[2 * e] = make_float2(v.x, v.y);
            cs[2 * e + 1] = make_float2(v.z, v.w);
        }
    }
};

template <int HD>
struct GlobalKV {
    const uint16_t *kb, *vb;  // cache rows of (layer, b, g): [S][HD]
    int s0, last;             // first position of the split, last valid cached position
    __device__ __forceinline__ size_t off(int t) const {
        int j = s0 + t * AttnGeom<HD>::PPW + lane_id() / AttnGeom<HD>::LPP;
        if (j > last) j = last;
        if (j < 0) j = 0;
        return (size_t)j * HD + 8 * (lane_id() % AttnGeom<HD>::LPP);
    }
    const float2* rope_row;   // (cos, sin) row of the position
    __device__ __forceinline__ void rope(int i0, float2 (&cs)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = rope_row[i0 + e];
    }
    struct Block {
        const GlobalKV* kv;
        int t0;
        __device__ __forceinline__ uint4 k(int t) const { return *(const uint4*)(kv->kb + kv->off(t0 + t)); }
        __device__ __forceinline__ uint4 v(int t) const { return *(const uint4*)(kv->vb + kv->off(t0 + t)); }
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

__device__ __forceinline__ void lse_merge(float& m, float& l, float* acc, float m2, float l2, const float* acc2) {
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;  // both empty
    const float c1 = (m == -INFINITY) ? 0.f : expf(m - mm);
    const float c2 = (m2 == -INFINITY) ? 0.f : expf(m2 - mm);
    l = l * c1 + l2 * c2;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    m = mm;
}

// RoPE of the 8 dims [dl, dl+8) of one head whose raw fp32 values start at `raw`
// (LDS): rotate-half pairs (i, i + HD/2) turn by the angles whose (cos, sin) the
// lane holds in cs (entries dl mod HD/2 .. + 7 of the position's table row).
template <int HD>
__device__ __forceinline__ void rope8(const float* raw, const float2 (&cs)[8], int dl, float* out) {
    constexpr int half = HD / 2;
    const bool lo = dl < half;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = dl + e, ii = lo ? i : i - half;
        const float a = raw[ii], b = raw[ii + half];
        out[e] = lo ? fmaf(a, cs[e].x, -(b * cs[e].y)) : fmaf(a, cs[e].y, b * cs[e].x);
    }
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

// LDS floats one attention item needs: staged q/k/v, per-head scores of one
// block of position groups (plus the group of the new position), and the
// partials of every split when this item merges them.
template <int HD>
__host__ __device__ constexpr uint32_t attn_lds_floats(int G, int nsplit) {
    return (uint32_t)((G + 2) * HD + kComputeWaves * (kAttnBlockGroups + 1) * (64 / (HD / 8)) +
                      nsplit * G * (HD + 2) + 4);
}

// Runs one attention item (sequence b, KV head g, split s) with `nw` waves of the
// workgroup, which all call it.  Wave j handles q head j of the group end to end:
// it scores every position of the split block by block (block = kAttnBlockGroups
// groups of PPW positions; lanes = (position slot, 8 dims), the per-position dot
// summed over the slot's lanes with DPP), exponentiates against the running
// maximum (two-pass softmax inside a block, rescaled across blocks), and
// accumulates the probability-weighted V per (slot, dims), summed over the slots
// at the end.  `need(t)` waits for ring group t; `release(t)` frees ring groups
// before t; `barrier()` synchronises the waves.  The new position (its K rotated
// and rounded to bf16, appended to the cache) joins as one extra group.  Writes
// the attention output (tagged) or, when split, the item's (max, sum, output)
// partial; the last split to arrive merges all partials in split order.
template <int HD, class KV, class Need, class Release, class Barrier, class Mark>
__device__ __forceinline__ bool attn_item(const Params& P, uint32_t tag0, int layer, int b, int g, int s, int p,
                                          const KV& kv, Need& need, Release& release, Barrier& barrier, float* xs,
                                          int wave, int nw, Spin& spin, Mark& mark) {
    using Geo = AttnGeom<HD>;
    constexpr int LPP = Geo::LPP, PPW = Geo::PPW;
    const int lane = lane_id();
    const int ps = lane / LPP;
    const int dl = 8 * (lane % LPP);
    const int G = P.G;
    const SplitRange R = split_range<HD>(p, s, P.nsplit);
    const float scale = P.attn_scale;
    const uint32_t tag_in = phase_tag(tag0, layer, 0) ^ ((P.inject && layer == 0) ? 0x80000000u : 0u);
    const uint32_t tag_out = phase_tag(tag0, layer, 1);
    const uint32_t stride = HD + 2;
    constexpr int kSlots = (kAttnBlockGroups + 1) * PPW;

    // the (cos, sin) row of position p (for the ring: the item's first chunk)
    if (!need(-1)) return false;
    float2 cs[8];
    kv.rope(dl < HD / 2 ? dl : dl - HD / 2, cs);
    float* q_raw = xs;
    float* k_raw = xs + G * HD;
    float* v_raw = k_raw + HD;
    float* sc = v_raw + HD + wave * kSlots;                // this wave's scores / weights
    float* spart = v_raw + HD + kComputeWaves * kSlots;    // [nsplit][G][HD + 2]
    uint32_t* flag = (uint32_t*)(spart + P.nsplit * G * stride);
    {
        const uint64_t* row = P.qkv + (size_t)b * P.qkv_rows;
        float ss = 0.f;
        bool ok = stage_tagged<false>(row + (size_t)g * G * HD, (uint32_t)(G * HD), tag_in, q_raw, nullptr, wave, nw,
                                      spin, ss);
        ok = ok && stage_tagged<false>(row + (size_t)(P.Hq + g) * HD, HD, tag_in, k_raw, nullptr, wave, nw, spin, ss);
        ok = ok && stage_tagged<false>(row + (size_t)(P.Hq + P.Hkv + g) * HD, HD, tag_in, v_raw, nullptr, wave, nw,
                                       spin, ss);
        if (!ok) return false;
    }
    if (!barrier()) return false;
    mark(0);

    // Rotations on every path (waves without a q head rotate a neighbour's values,
    // unused): the (cos, sin) loads are consumed here, before any store, so no
    // load stays pending past this instruction.
    const int j = wave;  // q head of this wave
    float q[8];
    rope8<HD>(q_raw + j * HD, cs, dl, q);
    // the new position: K rotated, K and V rounded to bf16 as the cache holds them
    float kr[8];
    rope8<HD>(k_raw, cs, dl, kr);
    const uint4 kn = make_uint4(pack_bf2(kr[0], kr[1]), pack_bf2(kr[2], kr[3]), pack_bf2(kr[4], kr[5]),
                                pack_bf2(kr[6], kr[7]));
    const uint4 vn = make_uint4(pack_bf2(v_raw[dl], v_raw[dl + 1]), pack_bf2(v_raw[dl + 2], v_raw[dl + 3]),
                                pack_bf2(v_raw[dl + 4], v_raw[dl + 5]), pack_bf2(v_raw[dl + 6], v_raw[dl + 7]));
    if (R.has_new && wave == 0 && ps == 0) {  // KV append at position p (read by later steps)
        const size_t row = ((((size_t)layer * P.kv_b + b) * P.Hkv + g) * P.S + p) * HD + dl;
        *(uint4*)(P.kcache + row) = kn;
        *(uint4*)(P.vcache + row) = vn;
    }
    const int ngr = R.ngroups + (R.has_new ? 1 : 0);  // ring groups, then the new position's group
    float m_run = -INFINITY, l_run = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (j < G) {
        for (int t0 = 0; t0 < ngr; t0 += kAttnBlockGroups) {
            const int t1 = min(ngr, t0 + kAttnBlockGroups);
            const auto blk = kv.block(t0);
            // every ring group of the block resident (one wait per block)
            if (t0 < R.ngroups && !need(min(t1, R.ngroups) - 1)) return false;
            // scores of the block, four groups per step so their LDS reads overlap
            float mx = -INFINITY;
            for (int t = t0; t < t1; t += 4) {
                uint4 kp[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tt = t + u;
                    kp[u] = (tt < R.ngroups && tt < t1) ? blk.k(tt - t0) : kn;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tt = t + u;
                    if (tt < t1) {
                        float v = group_sum_dpp<LPP>(qk8(q, kp[u])) * scale;
                        const bool valid = tt == R.ngroups ? ps == 0 : tt * PPW + ps < R.ncached;
                        v = valid ? v : -INFINITY;
                        if (dl == 0) sc[(tt - t0) * PPW + ps] = v;
                        mx = fmaxf(mx, v);
                    }
                }
            }
            mx = wave_maxf(mx);
            const float m_new = fmaxf(m_run, mx);
            // weights against the running maximum, and their sum
            float l_blk = 0.f;
            for (int i = lane; i < (t1 - t0) * PPW; i += 64) {
                const float v = sc[i];
                const float e = v == -INFINITY ? 0.f : expf(v - m_new);
                sc[i] = e;
                l_blk += e;
            }
            l_blk = wave_total(l_blk);
            // rescale what earlier blocks accumulated, then add this block's weighted V
            const float c = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= c;
            l_run = l_run * c + l_blk;
            m_run = m_new;
            for (int t = t0; t < t1; t += 4) {
                uint4 vp[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int tt = t + u;
                    vp[u] = (tt < R.ngroups && tt < t1) ? blk.v(tt - t0) : vn;
                    w[u] = tt < t1 ? sc[(tt - t0) * PPW + ps] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    acc[0] = fmaf(w[u], bf_lo(vp[u].x), acc[0]);
                    acc[1] = fmaf(w[u], bf_hi(vp[u].x), acc[1]);
                    acc[2] = fmaf(w[u], bf_lo(vp[u].y), acc[2]);
                    acc[3] = fmaf(w[u], bf_hi(vp[u].y), acc[3]);
                    acc[4] = fmaf(w[u], bf_lo(vp[u].z), acc[4]);
                    acc[5] = fmaf(w[u], bf_hi(vp[u].z), acc[5]);
                    acc[6] = fmaf(w[u], bf_lo(vp[u].w), acc[6]);
                    acc[7] = fmaf(w[u], bf_hi(vp[u].w), acc[7]);
                }
            }
            release(min(t1, R.ngroups));
        }
        // sum the position slots (lanes with equal dims)
#pragma unroll
        for (int msk = LPP; msk < 64; msk <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], msk, 64);
    } else {
        release(R.ngroups);
    }
    mark(1);
    uint64_t* out_b = P.attn + (size_t)b * P.Hq * HD;
    if (P.nsplit == 1) {
        if (j < G && ps == 0) {
            const float inv = 1.0f / l_run;
            uint64_t* o = out_b + (size_t)(g * G + j) * HD + dl;
#pragma unroll
            for (int e = 0; e < 8; ++e) st_tagged(o + e, acc[e] * inv, tag_out);
        }
        mark(2);
        return true;
    }
    // split: publish the partial; the last split to arrive merges all of them
    const size_t pstride = (size_t)G * stride;
    uint64_t* part = P.attn_part + (((size_t)b * P.Hkv + g) * P.nsplit) * pstride;
    uint32_t* tk = P.attn_ticket + (((size_t)layer * P.B + b) * P.Hkv + g) * kCtrStride;
    if (j < G && ps == 0) {
        uint64_t* dst = part + (size_t)s * pstride + (size_t)j * stride;
        if (dl == 0) {
            st_tagged(dst, m_run, tag_out);
            st_tagged(dst + 1, l_run, tag_out);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) st_tagged(dst + 2 + dl + e, acc[e], tag_out);
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
        float ss = 0.f;
        if (!stage_tagged<false>(part, (uint32_t)(P.nsplit * pstride), tag_out, spart, nullptr, wave, nw, spin, ss))
            return false;
    }
    if (!barrier()) return false;
    if (j < G && ps == 0) {
        const float* s0p = spart + (size_t)j * stride;
        float mm = s0p[0], ll = s0p[1], aa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) aa[e] = s0p[2 + dl + e];
        for (int sp = 1; sp < P.nsplit; ++sp) {
            const float* src = spart + (size_t)sp * pstride + (size_t)j * stride;
            float a2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) a2[e] = src[2 + dl + e];
            lse_merge(mm, ll, aa, src[0], src[1], a2);
        }
        const float inv = 1.0f / ll;
        uint64_t* o = out_b + (size_t)(g * G + j) * HD + dl;
#pragma unroll
        for (int e = 0; e < 8; ++e) st_tagged(o + e, aa[e] * inv, tag_out);
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
        for (int b = 1; b < B; ++b)
            if (lane == b) i = bi[b];
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
    if (lane < B) P.state->ctx_len[lane] = P.state->ctx_len[lane] + 1;
    if (lane == 0) __hip_atomic_store(P.head_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__any(nan_seen)) raise_error_impl(P.state, P.host_err, spin.abort_flag, DERR_NAN, 0, 0);
    return true;
}

}  // namespace mk
