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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f_to_bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float round_bf(float f) { return __uint_as_float(f_to_bf(f) << 16); }
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

// Butterfly sum over the 64 lanes.  Partner lanes add the same two partial sums
// (addition commutes), so every lane ends with the bitwise-identical total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
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
// RMSNorm of B residual rows into fp32 activations (x_i = h_i * g_i / rms(h)).
// Lane l handles 8-element pieces p = l + 64 j: it writes exactly the pieces it
// later reads in row_dot, so no other lane or wave depends on its stores.
// `src_bf16` != nullptr selects embedding rows (layer 0) instead of `h`.
// ---------------------------------------------------------------------------------------------
template <int B>
__device__ void rmsnorm_rows(const float* __restrict__ h, const uint16_t* __restrict__ emb,
                             const int32_t* __restrict__ tok, int32_t tok_stride, int V, const uint16_t* __restrict__ g,
                             int d, float eps, float* __restrict__ xout) {
    const int lane = lane_id();
    const int np = d >> 3;
    constexpr int kMaxPieces = 8;  // d <= 4096: at most 8 pieces per lane
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float* hb = h + (size_t)b * d;
        const uint16_t* eb = emb ? emb + token_row(tok, b, tok_stride, V) * d : nullptr;
        float v[kMaxPieces][8];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxPieces; ++j) {
            const int p = lane + 64 * j;
            if (p < np) {
                if (eb) {
                    uint4 u = *(const uint4*)(eb + 8 * p);
                    v[j][0] = bf_lo(u.x); v[j][1] = bf_hi(u.x); v[j][2] = bf_lo(u.y); v[j][3] = bf_hi(u.y);
                    v[j][4] = bf_lo(u.z); v[j][5] = bf_hi(u.z); v[j][6] = bf_lo(u.w); v[j][7] = bf_hi(u.w);
                } else {
                    float4 a = *(const float4*)(hb + 8 * p), c = *(const float4*)(hb + 8 * p + 4);
                    v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
                    v[j][4] = c.x; v[j][5] = c.y; v[j][6] = c.z; v[j][7] = c.w;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxPieces; ++j)
            if (lane + 64 * j < np)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(v[j][e], v[j][e], ss);
        ss = wave_total(ss);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
        for (int j = 0; j < kMaxPieces; ++j) {
            const int p = lane + 64 * j;
            if (p < np) {
                uint4 gv = *(const uint4*)(g + 8 * p);
                float gg[8] = {bf_lo(gv.x), bf_hi(gv.x), bf_lo(gv.y), bf_hi(gv.y),
                               bf_lo(gv.z), bf_hi(gv.z), bf_lo(gv.w), bf_hi(gv.w)};
                float4 o0 = make_float4(v[j][0] * r * gg[0], v[j][1] * r * gg[1], v[j][2] * r * gg[2],
                                        v[j][3] * r * gg[3]);
                float4 o1 = make_float4(v[j][4] * r * gg[4], v[j][5] * r * gg[5], v[j][6] * r * gg[6],
                                        v[j][7] * r * gg[7]);
                *(float4*)(xout + (size_t)b * d + 8 * p) = o0;
                *(float4*)(xout + (size_t)b * d + 8 * p + 4) = o1;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Row sources: piece p (16 bytes = 8 bf16) of row r of the current instruction.
// ---------------------------------------------------------------------------------------------
struct RingRows {  // rows laid back to back in the LDS ring from stream offset `base`
    const char* ring;
    uint32_t base, rb;
    __device__ __forceinline__ uint4 piece(uint32_t r, uint32_t p) const {
        return *(const uint4*)(ring + ((base + r * rb + p * 16u) & (kRingBytes - 1u)));
    }
};

// Activation sources (fp32): the 8 values of piece p of batch row b.
struct XLds {
    const float* x;
    uint32_t k;
    __device__ __forceinline__ void piece(int b, uint32_t p, float4& a, float4& c) const {
        const float* q = x + (size_t)b * k + 8 * p;
        a = *(const float4*)q;
        c = *(const float4*)(q + 4);
    }
};
struct XGlobal {
    const float* x;
    uint32_t stride;
    __device__ __forceinline__ void piece(int b, uint32_t p, float4& a, float4& c) const {
        const float* q = x + (size_t)b * stride + 8 * p;
        a = *(const float4*)q;
        c = *(const float4*)(q + 4);
    }
};

// out[i][b] = dot(row r0 + i, x_b) for i < nr (nr <= R rows processed together:
// the activation pieces are read once for all of them).  Per row, lane l
// accumulates pieces p = l, l + 64, ... in ascending order, then wave_total
// reduces in its fixed tree; the value of a row never depends on R, nr or on
// which other rows share the batch.
template <int B, int R, class Rows, class X>
__device__ __forceinline__ void rows_dot(const Rows& rows, uint32_t r0, int nr, int np, const X& x,
                                         float (&out)[R][B]) {
    const int lane = lane_id();
    float acc[R][B];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = 0.f;
#pragma unroll 2
    for (int p = lane; p < np; p += 64) {
        float4 xa[B], xb[B];
#pragma unroll
        for (int b = 0; b < B; ++b) x.piece(b, (uint32_t)p, xa[b], xb[b]);
        uint4 w[R];
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (i < nr) w[i] = rows.piece(r0 + i, (uint32_t)p);
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (i < nr)
#pragma unroll
                for (int b = 0; b < B; ++b) acc[i][b] = dot8(w[i], xa[b], xb[b], acc[i][b]);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < B; ++b) out[i][b] = (i < nr) ? wave_total(acc[i][b]) : 0.f;
}

// Rows processed together for a row of `rb` bytes: the batch of the four
// compute waves stays within 64 KB of the ring.
__host__ __device__ constexpr int rows_per_batch(uint32_t rb) { return rb <= 4096u ? 4 : rb <= 8192u ? 2 : 1; }

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

// Running greedy choice: larger value wins, ties to the lower index.
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
// Group t holds kPPW consecutive positions; lane -> (position ps = lane / LPP,
// dims dl = 8 * (lane % LPP)).
// ---------------------------------------------------------------------------------------------
template <int HD>
struct AttnGeom {
    static constexpr int LPP = HD / 8;     // lanes per position
    static constexpr int PPW = 64 / LPP;   // positions per 1 KB group
};

struct RingKV {
    const char* ring;
    uint32_t base;  // stream offset of the item: group t = [K 1 KB][V 1 KB]
    __device__ __forceinline__ uint4 k(int t) const {
        return *(const uint4*)(ring + ((base + (uint32_t)t * 2048u + lane_id() * 16u) & (kRingBytes - 1u)));
    }
    __device__ __forceinline__ uint4 v(int t) const {
        return *(const uint4*)(ring + ((base + (uint32_t)t * 2048u + 1024u + lane_id() * 16u) & (kRingBytes - 1u)));
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
    __device__ __forceinline__ uint4 k(int t) const { return *(const uint4*)(kb + off(t)); }
    __device__ __forceinline__ uint4 v(int t) const { return *(const uint4*)(vb + off(t)); }
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

// RoPE of the 8 dims [dl, dl+8) of one head whose raw fp32 values start at `raw`;
// rotate-half pairs (i, i + HD/2) turn by the angle of table row `rope_row`.
template <int HD>
__device__ __forceinline__ void rope8(const float* __restrict__ raw, const float2* __restrict__ rope_row, int dl,
                                      float* out) {
    constexpr int half = HD / 2;
    const bool lo = dl < half;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = dl + e, ii = lo ? i : i - half;
        const float a = raw[ii], b = raw[ii + half];
        const float2 cs = rope_row[ii];
        out[e] = lo ? fmaf(a, cs.x, -(b * cs.y)) : fmaf(a, cs.y, b * cs.x);
    }
}

struct AttnScratch {  // LDS scratch of one item: per wave and head (m, l, acc[HD])
    float* part;      // [kComputeWaves][kMaxGroup][HD + 2]
};

// Runs one attention item with the calling wave (`wave` of `nwaves` waves of the
// workgroup).  `need(t)` is called before group t is read (ring: wait for the
// loader), `barrier()` synchronises the waves of the item.  Returns true when
// this workgroup merged the final output (or no merge was needed).
template <int HD, class KV, class Need, class Barrier>
__device__ void attn_item(const Params& P, int layer, int b, int g, int s, int p, const KV& kv, Need need,
                          Barrier barrier, float* lds_part, int wave, int nwaves, uint32_t* tickets,
                          bool& merged_here) {
    using Geo = AttnGeom<HD>;
    const int lane = lane_id();
    const int ps = lane / Geo::LPP;
    const int dl = 8 * (lane % Geo::LPP);
    const int G = P.G;
    const SplitRange R = split_range<HD>(p, s, P.nsplit);
    const float scale = P.attn_scale;
    const float2* rope_row = P.rope + (size_t)p * (HD / 2);
    const float* qkv_b = P.qkv + (size_t)b * P.qkv_rows;

    // q heads of the group after RoPE (fp32)
    float q[kMaxGroup][8];
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) {
        if (j < G) rope8<HD>(qkv_b + (size_t)(g * G + j) * HD, rope_row, dl, q[j]);
    }
    float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][8];
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
    }
    auto consume = [&](uint4 kp, uint4 vp, bool valid) {
        const float vv[8] = {bf_lo(vp.x), bf_hi(vp.x), bf_lo(vp.y), bf_hi(vp.y),
                             bf_lo(vp.z), bf_hi(vp.z), bf_lo(vp.w), bf_hi(vp.w)};
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
            if (j < G) {
                float sc = qk8(q[j], kp);
                sc = group_sum(sc, Geo::LPP) * scale;
                if (valid) {
                    const float mn = fmaxf(m[j], sc);
                    const float c = (m[j] == -INFINITY) ? 0.f : expf(m[j] - mn);
                    const float e = expf(sc - mn);
                    l[j] = l[j] * c + e;
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[j][k] = fmaf(e, vv[k], acc[j][k] * c);
                    m[j] = mn;
                }
            }
        }
    };
    for (int t = wave; t < R.ngroups; t += nwaves) {
        need(t);
        const uint4 kp = kv.k(t), vp = kv.v(t);
        consume(kp, vp, R.s0 + t * Geo::PPW + ps < R.s0 + R.ncached);
    }
    // the new position: rotated k and bf16 k/v from this step's projections
    if (R.has_new && wave == 0) {
        const float* kraw = qkv_b + (size_t)P.Hq * HD + (size_t)g * HD;
        const float* vraw = qkv_b + (size_t)(P.Hq + P.Hkv) * HD + (size_t)g * HD;
        float kr[8];
        rope8<HD>(kraw, rope_row, dl, kr);
        const uint4 kp = make_uint4(pack_bf2(kr[0], kr[1]), pack_bf2(kr[2], kr[3]), pack_bf2(kr[4], kr[5]),
                                    pack_bf2(kr[6], kr[7]));
        const uint4 vp = make_uint4(pack_bf2(vraw[dl], vraw[dl + 1]), pack_bf2(vraw[dl + 2], vraw[dl + 3]),
                                    pack_bf2(vraw[dl + 4], vraw[dl + 5]), pack_bf2(vraw[dl + 6], vraw[dl + 7]));
        if (ps == 0) {  // KV append at position p
            const size_t row = ((((size_t)layer * P.kv_b + b) * P.Hkv + g) * P.S + p) * HD + dl;
            *(uint4*)(P.kcache + row) = kp;
            *(uint4*)(P.vcache + row) = vp;
        }
        consume(kp, vp, ps == 0);
    }
    // merge the position groups of the wave (lanes with equal dims)
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) {
        if (j < G) {
            for (int msk = Geo::LPP; msk < 64; msk <<= 1) {
                float acc2[8];
                const float m2 = __shfl_xor(m[j], msk, 64), l2 = __shfl_xor(l[j], msk, 64);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[j][e], msk, 64);
                lse_merge(m[j], l[j], acc[j], m2, l2, acc2);
            }
        }
    }
    // merge the waves in order through LDS
    const int stride = HD + 2;
    if (ps == 0) {
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
            if (j < G) {
                float* dst = lds_part + ((size_t)wave * kMaxGroup + j) * stride;
                if (dl == 0) {
                    dst[0] = m[j];
                    dst[1] = l[j];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[2 + dl + e] = acc[j][e];
            }
        }
    }
    barrier();
    merged_here = false;
    if (wave != 0) return;
    if (ps == 0) {
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
            if (j < G) {
                const float* src = lds_part + (size_t)j * stride;
                float mm = src[0], ll = src[1], aa[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) aa[e] = src[2 + dl + e];
                for (int w = 1; w < nwaves; ++w) {
                    const float* sw = lds_part + ((size_t)w * kMaxGroup + j) * stride;
                    float a2[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) a2[e] = sw[2 + dl + e];
                    lse_merge(mm, ll, aa, sw[0], sw[1], a2);
                }
                m[j] = mm;
                l[j] = ll;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = aa[e];
            }
        }
    }
    float* out_b = P.attn + (size_t)b * P.Hq * HD;
    if (P.nsplit == 1) {
        if (ps == 0) {
#pragma unroll
            for (int j = 0; j < kMaxGroup; ++j) {
                if (j < G) {
                    const float inv = 1.0f / l[j];
                    float* o = out_b + (size_t)(g * G + j) * HD + dl;
                    *(float4*)o = make_float4(acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv);
                    *(float4*)(o + 4) = make_float4(acc[j][4] * inv, acc[j][5] * inv, acc[j][6] * inv, acc[j][7] * inv);
                }
            }
        }
        merged_here = true;
        return;
    }
    // split: publish the partial, the last split to arrive merges all of them in order
    const size_t pstride = (size_t)G * stride;
    float* part = P.attn_part + (((size_t)b * P.Hkv + g) * P.nsplit) * pstride;
    if (ps == 0) {
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
            if (j < G) {
                float* dst = part + (size_t)s * pstride + (size_t)j * stride;
                if (dl == 0) {
                    dst[0] = m[j];
                    dst[1] = l[j];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[2 + dl + e] = acc[j][e];
            }
        }
    }
    uint32_t* tk = tickets + (((size_t)layer * P.B + b) * P.Hkv + g) * kCtrStride;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)P.nsplit - 1u) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (ps == 0) {
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
            if (j < G) {
                const float* s0p = part + (size_t)j * stride;
                float mm = s0p[0], ll = s0p[1], aa[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) aa[e] = s0p[2 + dl + e];
                for (int sp = 1; sp < P.nsplit; ++sp) {
                    const float* src = part + (size_t)sp * pstride + (size_t)j * stride;
                    float a2[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) a2[e] = src[2 + dl + e];
                    lse_merge(mm, ll, aa, src[0], src[1], a2);
                }
                const float inv = 1.0f / ll;
                float* o = out_b + (size_t)(g * G + j) * HD + dl;
                *(float4*)o = make_float4(aa[0] * inv, aa[1] * inv, aa[2] * inv, aa[3] * inv);
                *(float4*)(o + 4) = make_float4(aa[4] * inv, aa[5] * inv, aa[6] * inv, aa[7] * inv);
            }
        }
    }
    if (lane == 0) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merged_here = true;
}

// ---------------------------------------------------------------------------------------------
// Greedy argmax over the per-wave partials (value, index) of every sequence.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void reduce_head_parts(const HeadPart* parts, int nparts, int B, int32_t* tok_out,
                                                  uint32_t* nan_flag) {
    const int lane = lane_id();
    for (int b = 0; b < B; ++b) {
        float bv = -INFINITY;
        int32_t bi = 0x7FFFFFFF;
        for (int k = lane; k < nparts; k += 64) {
            HeadPart hp = parts[(size_t)k * B + b];
            if (hp.v != hp.v) *nan_flag = 1;
            if (head_better(hp.v, hp.i, bv, bi)) {
                bv = hp.v;
                bi = hp.i;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int32_t oi = __shfl_xor(bi, m, 64);
            if (head_better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == 0) tok_out[b] = bi;
    }
}

}  // namespace mk
