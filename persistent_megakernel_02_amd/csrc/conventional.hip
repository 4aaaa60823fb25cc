// The conventional decode step: one kernel per op, five per layer plus the LM
// head, replayed from a hipGraph.  This is the design the megakernel replaces
// (page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "传统推理方式效率低下的根源剖析": many small kernels in sequence, each launch leaving
// a gap in which no weight is loaded).  Every kernel stages its inputs and calls
// the same tile functions as the megakernel with the same four-wave lane mapping,
// so the two paths give bitwise-identical logits and tokens.  Kernel order makes
// every tag match on the first poll.
#include <hip/hip_runtime.h>

#include "mk_device.h"

namespace mk {

constexpr int kConvWaves = kComputeWaves;  // same wave count per item as the megakernel
constexpr int kConvThreads = 64 * kConvWaves;
constexpr uint32_t kRowsPerBlock = 16;       // most rows of a projection per workgroup
constexpr uint32_t kHeadRowsPerBlock = 128;  // LM-head rows per workgroup (the input staging amortised)

// Rows per workgroup of a projection with `total` rows: at most kRowsPerBlock, and
// few enough that the grid covers every CU.
__host__ __device__ inline uint32_t rows_per_block(uint32_t total, int n_cu) {
    const uint32_t per_cu = (total + (uint32_t)n_cu - 1u) / (uint32_t)n_cu;
    return per_cu < 1u ? 1u : per_cu > kRowsPerBlock ? kRowsPerBlock : per_cu;
}

struct BlockBarrier {
    __device__ __forceinline__ bool operator()() {
        __syncthreads();
        return true;
    }
};

// R rows of a batch read straight from global memory.
template <int R>
struct GlobalBatch {
    const uint16_t* row[R];
    __device__ __forceinline__ uint4 piece(uint32_t i, uint32_t p) const {
        return *(const uint4*)(row[i] + 8 * p);
    }
};

// Row j of an instruction's row sequence (QKV: [Wq; Wk; Wv] rows from `begin`;
// GATEUP: gate row, up row of f = begin + j / 2; others: rows from `begin`).
template <int OP>
__device__ __forceinline__ const uint16_t* seq_row(const Params& P, const DevLayer& Lw, uint32_t begin, uint32_t j) {
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

// Rows [0, nrows) of the block in batches of R rows per wave (rows of a short
// last batch repeat its first row; their results are not used).
// `col0`: first column of the rows (a column slice of DOWN), rb: bytes per row used.
template <int B, int R, int OP, class X, class Epi>
__device__ __forceinline__ void conv_rows(const Params& P, const DevLayer& Lw, uint32_t begin, uint32_t nrows,
                                          uint32_t rb, const X& x, Epi& epi, uint32_t col0 = 0) {
    const int wave = threadIdx.x >> 6;
    for (uint32_t r0 = (uint32_t)wave * R; r0 < nrows; r0 += (uint32_t)R * kConvWaves) {
        const uint32_t nr = min((uint32_t)R, nrows - r0);
        GlobalBatch<R> rows;
#pragma unroll
        for (int i = 0; i < R; ++i)
            rows.row[i] = seq_row<OP>(P, Lw, begin, r0 + ((uint32_t)i < nr ? (uint32_t)i : 0u)) + col0;
        float res[R][B];
        rows_dot<B, R>(rows, (int)(rb >> 4), x, res);
        epi(r0, nr, res);
    }
}

template <int B, int OP, class X, class Epi>
__device__ __forceinline__ void conv_rows_auto(const Params& P, const DevLayer& Lw, uint32_t begin, uint32_t nrows,
                                               uint32_t rb, const X& x, Epi& epi, uint32_t col0 = 0) {
    const int R = rows_per_batch(rb, B);
    if (R >= 4) conv_rows<B, 4, OP>(P, Lw, begin, nrows, rb, x, epi, col0);
    else if (R == 2 || OP == OP_GATEUP) conv_rows<B, 2, OP>(P, Lw, begin, nrows, rb, x, epi, col0);
    else conv_rows<B, 1, OP>(P, Lw, begin, nrows, rb, x, epi, col0);
}

// RMSNorm + rows: QKV, GATEUP (row pairs) and the LM head.
template <int B, int OP>
__global__ void __launch_bounds__(kConvThreads) k_norm_gemv(Params P, StepArgs A, int layer, uint32_t rpb) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ float ssp[kMaxBatch][kConvWaves];
    float* xs = (float*)lds;
    const int wave = threadIdx.x >> 6, lane = lane_id();
    Spin spin(&P, nullptr);
    const DevLayer Lw = P.layers[layer < P.L ? layer : 0];
    const uint16_t* gain = OP == OP_QKV ? Lw.attn_norm : OP == OP_GATEUP ? Lw.mlp_norm : P.final_norm;
    const uint32_t tag_in = OP == OP_QKV      ? phase_tag(A.tag0, layer - 1, 4)
                            : OP == OP_GATEUP ? phase_tag(A.tag0, layer, 2)
                                              : phase_tag(A.tag0, P.L - 1, 4);
    const uint32_t d = (uint32_t)P.d;
    float ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = 0.f;
    if (OP == OP_QKV && layer == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b)
            stage_bf16(P.embed + token_row(A, b, P.V) * d, d, xs + b * d, gain, wave, kConvWaves,
                       ss[b]);
    } else {
        const StageSeg sg[1] = {{P.h, xs, gain, d, (uint32_t)B, d, d, tag_in}};
        if (!stage_segs<kStagePassWords, B, 1>(sg, wave, kConvWaves, spin, ss)) return;
    }
    wave_total_n<B>(ss);
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) ssp[b][wave] = ss[b];
    }
    __syncthreads();
    float r[B];
#pragma unroll
    for (int b = 0; b < B; ++b) r[b] = rms_scale(ssp[b], kConvWaves, P.d, P.eps);
    const uint32_t total = OP == OP_QKV ? (uint32_t)P.qkv_rows : OP == OP_GATEUP ? (uint32_t)P.F : (uint32_t)P.V;
    const uint32_t begin = blockIdx.x * rpb;
    const uint32_t count = min(rpb, total - begin);
    const uint32_t nrows = OP == OP_GATEUP ? 2u * count : count;
    const XLds x{xs, d};
    if (OP == OP_QKV) {
        const uint32_t tag_out = phase_tag(A.tag0, layer, 0);
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i)
                if (i < nr && lane < B)
                    st_tagged(P.qkv + (size_t)lane * P.qkv_rows + begin + r0 + i,
                              pick<B>(res[i], lane) * pick<B>(r, lane), tag_out);
        };
        conv_rows_auto<B, OP>(P, Lw, begin, nrows, d * 2u, x, epi);
    } else if (OP == OP_GATEUP) {
        const uint32_t tag_out = phase_tag(A.tag0, layer, 3);
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i + 1 < (uint32_t)(sizeof(res) / sizeof(res[0])); i += 2) {
                if (i + 1 >= nr) break;
                const uint32_t f = begin + (r0 + i) / 2u;
                if (lane < B) {
                    const float rr = pick<B>(r, lane);
                    st_tagged(P.act + (size_t)lane * P.F + f,
                              silu_mul(pick<B>(res[i], lane) * rr, pick<B>(res[i + 1], lane) * rr), tag_out);
                }
            }
        };
        conv_rows_auto<B, OP>(P, Lw, begin, nrows, d * 2u, x, epi);
    } else {
        float best_v[B];
        int32_t best_i[B];
        bool nan_seen = false;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            best_v[b] = -INFINITY;
            best_i[b] = 0x7FFFFFFF;
        }
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i) {
                if (i >= nr) break;
                const int32_t row = (int32_t)(begin + r0 + i);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float v = res[i][b] * r[b];
                    if (v != v) nan_seen = true;
                    if (head_better(v, row, best_v[b], best_i[b])) {
                        best_v[b] = v;
                        best_i[b] = row;
                    }
                }
                if (lane < B) A.logits[(size_t)lane * P.V + row] = pick<B>(res[i], lane) * pick<B>(r, lane);
            }
        };
        conv_rows_auto<B, OP>(P, Lw, begin, nrows, d * 2u, x, epi);
        if (nan_seen) {
#pragma unroll
            for (int b = 0; b < B; ++b) best_v[b] = __int_as_float(0x7FC00000);
        }
        head_publish<B>(P, A, blockIdx.x * kConvWaves + (uint32_t)wave, best_v, best_i, spin);
    }
}

// O projection (is_down = 0) or down projection (is_down = 1) with residual add.
template <int B>
__global__ void __launch_bounds__(kConvThreads) k_proj(Params P, StepArgs A, int layer, int is_down, uint32_t rpb) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float* xs = (float*)lds;
    const int wave = threadIdx.x >> 6, lane = lane_id();
    Spin spin(&P, nullptr);
    const DevLayer Lw = P.layers[layer];
    const uint32_t K = is_down ? (uint32_t)P.F : (uint32_t)(P.Hq * P.hd);
    const uint32_t tag_x = is_down ? phase_tag(A.tag0, layer, 3) : phase_tag(A.tag0, layer, 1);
    const uint32_t tag_res = is_down ? phase_tag(A.tag0, layer, 2) : phase_tag(A.tag0, layer - 1, 4);
    const uint32_t tag_out = is_down ? phase_tag(A.tag0, layer, 4) : phase_tag(A.tag0, layer, 2);
    const uint32_t begin = blockIdx.x * rpb;
    const uint32_t count = min(rpb, (uint32_t)P.d - begin);
    if (B == 1 && is_down && P.down_q) {
        // by column quarters, as the persistent kernel's down_q_instr (weights from HBM)
        float* hres1 = xs + K;
        float* part4 = hres1 + kMaxResidRows;
        float ss[1] = {0.f};
        const StageSeg sg[2] = {{P.act, xs, nullptr, K, 1u, K, K, tag_x},
                                {P.h + begin, hres1, nullptr, count, 1u, (uint32_t)P.d, count, tag_res}};
        if (!stage_segs<kStagePassWordsWide, 1, 2>(sg, wave, kConvWaves, spin, ss)) return;
        __syncthreads();
        const XLds x{xs, K};
        float4 xa[4], xb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x.piece(0, (uint32_t)wave * kDownQPieces + (uint32_t)lane + 64u * (uint32_t)k, xa[k], xb[k]);
        for (uint32_t j = 0; j < count; ++j) {
            const uint4* rp = (const uint4*)(Lw.w_down + (size_t)(begin + j) * K) + (uint32_t)wave * kDownQPieces + lane;
            uint4 w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = rp[64 * k];
            const float v = down_q_partial(w, xa, xb);
            if (lane == 0) part4[j * 4u + (uint32_t)wave] = v;
        }
        __syncthreads();
        if (wave == 0)
            for (uint32_t j = (uint32_t)lane; j < count; j += 64u)
                st_tagged(P.h + begin + j, hres1[j] + down_q_row(part4 + j * 4u), tag_out);
        return;
    }
    // DOWN runs over P.down_slices column slices of its input; partial sums wait in LDS
    const uint32_t ns = is_down ? (uint32_t)P.down_slices : 1u, Ks = K / ns;
    float* hres = xs + B * Ks;
    float* part = hres + B * count;
    for (uint32_t ks = 0; ks < ns; ++ks) {
        if (ks > 0) __syncthreads();  // every wave is done with the previous slice
        float ss[1] = {0.f};
        const StageSeg sx = {(is_down ? P.act : P.attn) + ks * Ks, xs, nullptr, Ks, (uint32_t)B, K, Ks, tag_x};
        if (ks > 0) {
            const StageSeg sg[1] = {sx};
            if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kConvWaves, spin, ss)) return;
        } else if (!is_down && layer == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b)
                stage_bf16(P.embed + token_row(A, b, P.V) * P.d + begin, count, hres + b * count,
                           nullptr, wave, kConvWaves, ss[0]);
            const StageSeg sg[1] = {sx};
            if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kConvWaves, spin, ss)) return;
        } else {
            const StageSeg sg[2] = {sx, {P.h + begin, hres, nullptr, count, (uint32_t)B, (uint32_t)P.d, count, tag_res}};
            if (!stage_segs<kStagePassWordsWide, 1, 2>(sg, wave, kConvWaves, spin, ss)) return;
        }
        __syncthreads();
        const XLds x{xs, Ks};
        const bool last = ks + 1 == ns;
        auto epi = [&](uint32_t r0, uint32_t nr, auto& res) {
            #pragma unroll
            for (uint32_t i = 0; i < (uint32_t)(sizeof(res) / sizeof(res[0])); ++i) {
                if (i >= nr) break;
                const uint32_t j = r0 + i;
                if (lane < B) {
                    float v = pick<B>(res[i], lane);
                    if (ks > 0) v = part[lane * count + j] + v;
                    if (!last) {
                        part[lane * count + j] = v;
                    } else {
                        st_tagged(P.h + (size_t)lane * P.d + begin + j, hres[lane * count + j] + v, tag_out);
                    }
                }
            }
        };
        if (is_down) conv_rows_auto<B, OP_DOWN>(P, Lw, begin, count, Ks * 2u, x, epi, ks * Ks);
        else conv_rows_auto<B, OP_O>(P, Lw, begin, count, Ks * 2u, x, epi);
    }
}

// Split down projection, one part per workgroup (the persistent kernel's OP_DPART
// with the transposed Wdown rows read from HBM instead of the ring).
struct DpartGlobalRows {
    const uint16_t* w;  // the part's first transposed row
    uint32_t d, o;      // row length, this lane's first output
    bool on;
    __device__ __forceinline__ bool get(uint32_t f, uint4 (&q)[kDpartRowsPerGet]) {
#pragma unroll
        for (int u = 0; u < kDpartRowsPerGet; ++u)
            q[u] = on ? *(const uint4*)(w + (size_t)(f + (uint32_t)u) * d + o) : make_uint4(0u, 0u, 0u, 0u);
        return true;
    }
};

template <int B>
__global__ void __launch_bounds__(kConvThreads) k_dpart(Params P, StepArgs A, int layer) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float* xs = (float*)lds;
    const int wave = threadIdx.x >> 6, lane = lane_id();
    Spin spin(&P, nullptr);
    const DevLayer Lw = P.layers[layer];
    const uint32_t j = blockIdx.x, d = (uint32_t)P.d, f0 = j * kDownPart;
    const uint32_t tag_a = phase_tag(A.tag0, layer, 3);
    float ss[1] = {0.f};
    const StageSeg sg[1] = {{P.act + f0, xs, nullptr, kDownPart, (uint32_t)B, (uint32_t)P.F, kDownPart, tag_a, 0u}};
    if (!stage_segs<kStagePassWordsWide, 1, 1>(sg, wave, kConvWaves, spin, ss)) return;
    __syncthreads();
    const uint32_t o = 8u * (uint32_t)(wave * 64 + lane);
    DpartGlobalRows rows{Lw.w_down_t + (size_t)f0 * d, d, o, o < d};
    float acc[B][8];
    dpart_acc<B>(rows, xs, kDownPart, acc);
    float* out = xs + B * kDownPart;  // [B][d], stored with consecutive lanes on consecutive words
    if (rows.on) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float* q = out + (size_t)b * d + o;
            *(float4*)q = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
            *(float4*)(q + 4) = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
        }
    }
    __syncthreads();
    dpart_store<B>(P, out, j, tag_a, wave, kConvWaves);
}

// Split down projection, the row sums: rows [blockIdx.x rpb, + rpb).
template <int B>
__global__ void __launch_bounds__(kConvThreads) k_dred(Params P, StepArgs A, int layer, uint32_t rpb) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float* xs = (float*)lds;
    const int wave = threadIdx.x >> 6;
    Spin spin(&P, nullptr);
    const uint32_t d = (uint32_t)P.d, begin = blockIdx.x * rpb, cnt = min(rpb, d - begin);
    const uint32_t np = (uint32_t)P.F / kDownPart;
    float* hres = xs;
    float* part = hres + B * cnt;
    if (!stage_grid<kStagePassWordsWide>(P.h + begin, (uint32_t)B, phase_tag(A.tag0, layer, 2), P.dpart + begin,
                                         np * (uint32_t)B, phase_tag(A.tag0, layer, 3), d, cnt, xs, wave, kConvWaves,
                                         spin))
        return;
    __syncthreads();
    dred_out<B>(P, part, hres, begin, cnt, np, phase_tag(A.tag0, layer, 4), wave, kConvWaves);
}

// bf16 transpose through LDS: dst [cols][rows] = src [rows][cols]^T (the split
// down projection's copy of Wdown, made once at create).
__global__ void __launch_bounds__(256) k_transpose_bf16(uint16_t* dst, const uint16_t* src, int rows, int cols) {
    __shared__ uint16_t t[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    for (int i = threadIdx.y; i < 64; i += blockDim.y) {
        const int r = r0 + i, c = c0 + (int)threadIdx.x;
        if (r < rows && c < cols) t[i][threadIdx.x] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int i = threadIdx.y; i < 64; i += blockDim.y) {
        const int c = c0 + i, r = r0 + (int)threadIdx.x;
        if (c < cols && r < rows) dst[(size_t)c * rows + r] = t[threadIdx.x][i];
    }
}

hipError_t transpose_bf16(uint16_t* dst, const uint16_t* src, int rows, int cols, hipStream_t stream) {
    const dim3 blk(64, 4), grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(k_transpose_bf16, grid, blk, 0, stream, dst, src, rows, cols);
    return hipGetLastError();
}

template <int HD>
__global__ void __launch_bounds__(kConvThreads) k_attn(Params P, StepArgs A, int layer) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float* xs = (float*)lds;
    const int wave = threadIdx.x >> 6;
    const int item = blockIdx.x;
    const int per_b = P.Hkv * P.nsplit;
    const int b = item / per_b, g = (item % per_b) / P.nsplit, s = item % P.nsplit;
    const int p = P.ctx_len[b];
    const SplitRange R = split_range<HD>(p, s, P.nsplit);
    const size_t base = (((size_t)layer * P.kv_b + b) * P.Hkv + g) * (size_t)P.S * HD;
    const GlobalKV<HD> kv{P.kcache + base, P.vcache + base, R.s0, max(0, R.s0 + R.ncached - 1),
                          P.rope + (size_t)p * (HD / 2)};
    auto need = [](int) { return true; };
    auto release = [](int) {};
    BlockBarrier barrier;
    Spin spin(&P, nullptr);
    auto mark = [](int) {};
    attn_item<HD, false>(P, A.tag0, layer, b, g, s, 0, P.G, p, p, 1, b, true, kv, need, release, barrier, xs, wave, kConvWaves,
                  spin, mark);
}

// ------------------------------------------------------------------------------------------------
// host-side launch of one step (the host captures this sequence into a graph)
// ------------------------------------------------------------------------------------------------
int conventional_kernels_per_step(const Params& P) { return P.L * (kPhasesPerLayer + (P.down_split ? 1 : 0)) + 1; }

int conventional_head_blocks(const Params& P) { return (int)((P.V + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock); }

template <int B, int HD>
static hipError_t prepare_t(size_t lds) {
    const void* fns[] = {(const void*)k_norm_gemv<B, OP_QKV>, (const void*)k_norm_gemv<B, OP_GATEUP>,
                         (const void*)k_norm_gemv<B, OP_HEAD>, (const void*)k_proj<B>, (const void*)k_attn<HD>,
                         (const void*)k_dpart<B>, (const void*)k_dred<B>};
    for (const void* f : fns) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int B, int HD>
static hipError_t launch_step_t(const Params& P, const StepArgs& A, hipStream_t st) {
    const dim3 blk(kConvThreads);
    const size_t lds = P.x_bytes;
    const uint32_t qkv_rpb = rows_per_block((uint32_t)P.qkv_rows, P.n_cu);
    const uint32_t d_rpb = rows_per_block((uint32_t)P.d, P.n_cu), f_rpb = rows_per_block((uint32_t)P.F, P.n_cu);
    const int qkv_blocks = (int)((P.qkv_rows + qkv_rpb - 1) / qkv_rpb);
    const int d_blocks = (int)((P.d + d_rpb - 1) / d_rpb);
    const int f_blocks = (int)((P.F + f_rpb - 1) / f_rpb);
    const int items = P.B * P.Hkv * P.nsplit;
    for (int l = 0; l < P.L; ++l) {
        hipLaunchKernelGGL((k_norm_gemv<B, OP_QKV>), dim3(qkv_blocks), blk, lds, st, P, A, l, qkv_rpb);
        hipLaunchKernelGGL(k_attn<HD>, dim3(items), blk, lds, st, P, A, l);
        hipLaunchKernelGGL(k_proj<B>, dim3(d_blocks), blk, lds, st, P, A, l, 0, d_rpb);
        hipLaunchKernelGGL((k_norm_gemv<B, OP_GATEUP>), dim3(f_blocks), blk, lds, st, P, A, l, f_rpb);
        if (P.down_split) {
            const uint32_t rr = dred_rows((uint32_t)P.d, (uint32_t)P.F);
            hipLaunchKernelGGL(k_dpart<B>, dim3((unsigned)(P.F / (int)kDownPart)), blk, lds, st, P, A, l);
            hipLaunchKernelGGL(k_dred<B>, dim3((unsigned)((P.d + rr - 1) / rr)), blk, lds, st, P, A, l, rr);
        } else {
            hipLaunchKernelGGL(k_proj<B>, dim3(d_blocks), blk, lds, st, P, A, l, 1, d_rpb);
        }
    }
    hipLaunchKernelGGL((k_norm_gemv<B, OP_HEAD>), dim3(conventional_head_blocks(P)), blk, lds, st, P, A, P.L,
                       kHeadRowsPerBlock);
    return hipGetLastError();
}

hipError_t prepare_conventional(const Params& P) {
    if (P.hd == 64) {
        if (P.B == 1) return prepare_t<1, 64>(P.x_bytes);
        if (P.B == 2) return prepare_t<2, 64>(P.x_bytes);
        if (P.B == 4) return prepare_t<4, 64>(P.x_bytes);
        if (P.B == 8) return prepare_t<8, 64>(P.x_bytes);
    } else if (P.hd == 128) {
        if (P.B == 1) return prepare_t<1, 128>(P.x_bytes);
        if (P.B == 2) return prepare_t<2, 128>(P.x_bytes);
        if (P.B == 4) return prepare_t<4, 128>(P.x_bytes);
        if (P.B == 8) return prepare_t<8, 128>(P.x_bytes);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_conventional(const Params& P, const StepArgs& A, hipStream_t stream) {
    if (P.hd == 64) {
        if (P.B == 1) return launch_step_t<1, 64>(P, A, stream);
        if (P.B == 2) return launch_step_t<2, 64>(P, A, stream);
        if (P.B == 4) return launch_step_t<4, 64>(P, A, stream);
        if (P.B == 8) return launch_step_t<8, 64>(P, A, stream);
    } else if (P.hd == 128) {
        if (P.B == 1) return launch_step_t<1, 128>(P, A, stream);
        if (P.B == 2) return launch_step_t<2, 128>(P, A, stream);
        if (P.B == 4) return launch_step_t<4, 128>(P, A, stream);
        if (P.B == 8) return launch_step_t<8, 128>(P, A, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mk
