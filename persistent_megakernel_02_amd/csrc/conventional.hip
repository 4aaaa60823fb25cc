// The conventional decode step: one kernel per op, five per layer plus the LM
// head, replayed from a hipGraph.  This is the design the megakernel replaces
// (page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "传统推理方式效率低下的根源剖析": many small kernels in sequence, each launch leaving
// a gap in which no weight is loaded).  Every kernel calls the same tile
// functions as the megakernel with the same four-wave lane mapping, so the two
// paths give bitwise-identical logits and tokens.
#include <hip/hip_runtime.h>

#include "mk_device.h"

namespace mk {

constexpr int kConvWaves = kComputeWaves;  // same wave count per item as the megakernel
constexpr int kConvThreads = 64 * kConvWaves;
constexpr int kRowsPerBlock = 16;

struct QkvRows {
    const uint16_t *wq, *wk, *wv;
    uint32_t d, nq, nk, begin;
    __device__ __forceinline__ uint4 piece(uint32_t r, uint32_t p) const {
        const uint32_t row = begin + r;
        const uint16_t* base = row < nq ? wq + (size_t)row * d
                             : row < nq + nk ? wk + (size_t)(row - nq) * d
                                             : wv + (size_t)(row - nq - nk) * d;
        return *(const uint4*)(base + 8 * p);
    }
};
struct PlainRows {
    const uint16_t* w;
    uint32_t k, begin;
    __device__ __forceinline__ uint4 piece(uint32_t r, uint32_t p) const {
        return *(const uint4*)(w + (size_t)(begin + r) * k + 8 * p);
    }
};
struct PairRows {  // stream row 2i = gate row, 2i + 1 = up row of f = begin + i
    const uint16_t *wg, *wu;
    uint32_t d, begin;
    __device__ __forceinline__ uint4 piece(uint32_t r, uint32_t p) const {
        const uint16_t* w = (r & 1u) ? wu : wg;
        return *(const uint4*)(w + (size_t)(begin + (r >> 1)) * d + 8 * p);
    }
};

// Rows [0, count) of a block in batches of R rows per wave (the same tile
// function as the megakernel, so every row's value is bitwise identical).
template <int B, int R, class Rows, class X, class Epi>
__device__ __forceinline__ void conv_rows(const Rows& rows, uint32_t count, int np, const X& x, Epi&& epi) {
    const int wave = threadIdx.x >> 6;
    for (uint32_t r0 = (uint32_t)wave * R; r0 < count; r0 += (uint32_t)R * kConvWaves) {
        const uint32_t nr = min((uint32_t)R, count - r0);
        float res[R][B];
        rows_dot<B, R>(rows, r0, (int)nr, np, x, res);
        epi(r0, nr, res);
    }
}

template <int B>
__global__ void __launch_bounds__(kConvThreads) k_qkv(Params P, StepArgs A, int layer) {
    __shared__ __attribute__((aligned(16))) float xs[kXBytes / 4];
    const int lane = lane_id();
    const DevLayer Lw = P.layers[layer];
    rmsnorm_rows<B>(P.h, layer == 0 ? P.embed : nullptr, A.tok_in, A.tok_stride, P.V, Lw.attn_norm, P.d, P.eps, xs);
    const uint32_t begin = blockIdx.x * kRowsPerBlock;
    const uint32_t count = min((uint32_t)kRowsPerBlock, (uint32_t)P.qkv_rows - begin);
    const QkvRows rows{Lw.wq, Lw.wk, Lw.wv, (uint32_t)P.d, (uint32_t)(P.Hq * P.hd), (uint32_t)(P.Hkv * P.hd), begin};
    const XLds x{xs, (uint32_t)P.d};
    conv_rows<B, 4>(rows, count, P.d >> 3, x, [&](uint32_t r0, uint32_t nr, auto& res) {
        for (uint32_t i = 0; i < nr; ++i)
            if (lane < B) P.qkv[(size_t)lane * P.qkv_rows + begin + r0 + i] = pick<B>(res[i], lane);
    });
}

template <int B>
__global__ void __launch_bounds__(kConvThreads) k_gateup(Params P, StepArgs A, int layer) {
    __shared__ __attribute__((aligned(16))) float xs[kXBytes / 4];
    const int lane = lane_id();
    const DevLayer Lw = P.layers[layer];
    rmsnorm_rows<B>(P.h, nullptr, A.tok_in, A.tok_stride, P.V, Lw.mlp_norm, P.d, P.eps, xs);
    const uint32_t begin = blockIdx.x * kRowsPerBlock;
    const uint32_t count = min((uint32_t)kRowsPerBlock, (uint32_t)P.F - begin);
    const PairRows rows{Lw.w_gate, Lw.w_up, (uint32_t)P.d, begin};
    const XLds x{xs, (uint32_t)P.d};
    conv_rows<B, 4>(rows, 2u * count, P.d >> 3, x, [&](uint32_t r0, uint32_t nr, auto& res) {
        for (uint32_t i = 0; i + 1 < nr; i += 2)
            if (lane < B)
                P.act[(size_t)lane * P.F + begin + (r0 + i) / 2u] = silu_mul(pick<B>(res[i], lane), pick<B>(res[i + 1], lane));
    });
}

// O projection (is_down = 0) or down projection (is_down = 1) with residual add.
template <int B>
__global__ void __launch_bounds__(kConvThreads) k_proj_resid(Params P, StepArgs A, int layer, int is_down) {
    const int lane = lane_id();
    const DevLayer Lw = P.layers[layer];
    const uint32_t K = is_down ? (uint32_t)P.F : (uint32_t)(P.Hq * P.hd);
    const uint32_t begin = blockIdx.x * kRowsPerBlock;
    const uint32_t count = min((uint32_t)kRowsPerBlock, (uint32_t)P.d - begin);
    const PlainRows rows{is_down ? Lw.w_down : Lw.wo, K, begin};
    const XGlobal x{is_down ? P.act : P.attn, K};
    auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
        for (uint32_t i = 0; i < nr; ++i) {
            const uint32_t row = begin + r0 + i;
            if (lane < B) {
                float* hp = P.h + (size_t)lane * P.d + row;
                const float resid = (!is_down && layer == 0)
                                        ? bf_to_f(P.embed[token_row(A.tok_in, lane, A.tok_stride, P.V) * P.d + row])
                                        : *hp;
                *hp = resid + pick<B>(res[i], lane);
            }
        }
    };
    conv_rows<B, 4>(rows, count, (int)(K >> 3), x, epi);
}

template <int HD>
__global__ void __launch_bounds__(kConvThreads) k_attn(Params P, StepArgs A, int layer) {
    __shared__ __attribute__((aligned(16))) float part[kConvWaves * kMaxGroup * (HD + 2)];
    const int wave = threadIdx.x >> 6;
    const int item = blockIdx.x;
    const int per_b = P.Hkv * P.nsplit;
    const int b = item / per_b, g = (item % per_b) / P.nsplit, s = item % P.nsplit;
    const int p = P.state->ctx_len[b];
    const SplitRange R = split_range<HD>(p, s, P.nsplit);
    const size_t base = (((size_t)layer * P.kv_b + b) * P.Hkv + g) * (size_t)P.S * HD;
    const GlobalKV<HD> kv{P.kcache + base, P.vcache + base, R.s0, max(0, R.s0 + R.ncached - 1)};
    auto need = [](int) {};
    auto barrier = []() { __syncthreads(); };
    bool merged = false;
    attn_item<HD>(P, layer, b, g, s, p, kv, need, barrier, part, wave, kConvWaves, P.attn_ticket, merged);
}

// LM head rows with per-wave argmax partials; the last block chooses the tokens
// and advances the context lengths.
template <int B>
__global__ void __launch_bounds__(kConvThreads) k_head(Params P, StepArgs A, uint32_t* ticket) {
    __shared__ __attribute__((aligned(16))) float xs[kXBytes / 4];
    const int wave = threadIdx.x >> 6, lane = lane_id();
    rmsnorm_rows<B>(P.h, nullptr, A.tok_in, A.tok_stride, P.V, P.final_norm, P.d, P.eps, xs);
    const uint32_t begin = blockIdx.x * kRowsPerBlock;
    const uint32_t count = min((uint32_t)kRowsPerBlock, (uint32_t)P.V - begin);
    const PlainRows rows{P.head, (uint32_t)P.d, begin};
    const XLds x{xs, (uint32_t)P.d};
    float best_v[B];
    int32_t best_i[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        best_v[b] = -INFINITY;
        best_i[b] = 0x7FFFFFFF;
    }
    conv_rows<B, 4>(rows, count, P.d >> 3, x, [&](uint32_t r0, uint32_t nr, auto& res) {
        for (uint32_t i = 0; i < nr; ++i) {
            const int32_t row = (int32_t)(begin + r0 + i);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (head_better(res[i][b], row, best_v[b], best_i[b])) {
                    best_v[b] = res[i][b];
                    best_i[b] = row;
                }
            }
            if (lane < B) A.logits[(size_t)lane * P.V + row] = pick<B>(res[i], lane);
        }
    });
    if (lane < B) {
        HeadPart hp;
        hp.v = pick<B>(best_v, lane);
        int32_t bi = best_i[0];
#pragma unroll
        for (int b = 1; b < B; ++b)
            if (lane == b) bi = best_i[b];
        hp.i = bi;
        P.head_part[((size_t)blockIdx.x * kConvWaves + wave) * B + lane] = hp;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (wave != 0) return;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != gridDim.x - 1u) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t nanf = 0;
    reduce_head_parts(P.head_part, (int)gridDim.x * kConvWaves, B, A.tok_out, &nanf);
    if (lane < B) P.state->ctx_len[lane] = P.state->ctx_len[lane] + 1;
    if (lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__any(nanf != 0) && lane == 0) {
        uint32_t expected = 0;
        if (__hip_atomic_compare_exchange_strong(&P.state->error, &expected, (uint32_t)DERR_NAN, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &&
            P.host_err)
            __hip_atomic_store(&P.host_err->code, (uint32_t)DERR_NAN, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// ------------------------------------------------------------------------------------------------
// host-side launch of one step (the host captures this sequence into a graph)
// ------------------------------------------------------------------------------------------------
int conventional_kernels_per_step(const Params& P) { return P.L * kPhasesPerLayer + 1; }

int conventional_head_blocks(const Params& P) { return (P.V + kRowsPerBlock - 1) / kRowsPerBlock; }

template <int B, int HD>
static hipError_t launch_step_t(const Params& P, const StepArgs& A, uint32_t* head_ticket, hipStream_t st) {
    const dim3 blk(kConvThreads);
    const int qkv_blocks = (P.qkv_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int d_blocks = (P.d + kRowsPerBlock - 1) / kRowsPerBlock;
    const int f_blocks = (P.F + kRowsPerBlock - 1) / kRowsPerBlock;
    const int items = P.B * P.Hkv * P.nsplit;
    for (int l = 0; l < P.L; ++l) {
        hipLaunchKernelGGL(k_qkv<B>, dim3(qkv_blocks), blk, 0, st, P, A, l);
        hipLaunchKernelGGL(k_attn<HD>, dim3(items), blk, 0, st, P, A, l);
        hipLaunchKernelGGL(k_proj_resid<B>, dim3(d_blocks), blk, 0, st, P, A, l, 0);
        hipLaunchKernelGGL(k_gateup<B>, dim3(f_blocks), blk, 0, st, P, A, l);
        hipLaunchKernelGGL(k_proj_resid<B>, dim3(d_blocks), blk, 0, st, P, A, l, 1);
    }
    hipLaunchKernelGGL(k_head<B>, dim3(conventional_head_blocks(P)), blk, 0, st, P, A, head_ticket);
    return hipGetLastError();
}

hipError_t launch_conventional(const Params& P, const StepArgs& A, uint32_t* head_ticket, hipStream_t stream) {
    if (P.hd == 64) {
        if (P.B == 1) return launch_step_t<1, 64>(P, A, head_ticket, stream);
        if (P.B == 2) return launch_step_t<2, 64>(P, A, head_ticket, stream);
    } else if (P.hd == 128) {
        if (P.B == 1) return launch_step_t<1, 128>(P, A, head_ticket, stream);
        if (P.B == 2) return launch_step_t<2, 128>(P, A, head_ticket, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mk
