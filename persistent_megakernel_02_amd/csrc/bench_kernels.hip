// Measurement helpers: a streaming-read kernel (the practical HBM read ceiling
// the decode step is compared with) and a plain copy kernel of known size (its
// counter readings calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk_bench.h"

namespace {

// Each workgroup reads one contiguous slice of the buffer; every thread keeps 16
// non-temporal 16-byte loads in flight (a workgroup row of 4 KB per load), the
// fastest of the read patterns measured on the device for a multi-GB buffer.
constexpr int kReadUnroll = 16;

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ src, size_t n16, uint32_t* sink) {
    uint32_t acc = 0;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = min(n16, (size_t)blockIdx.x * per), b1 = min(n16, b0 + per);
    size_t i = b0 + threadIdx.x;
    for (; i + (kReadUnroll - 1) * 256 < b1; i += kReadUnroll * 256) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = ld_nt(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += 256) {
        const uint4 a = ld_nt(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads alive, practically never stores
}

__global__ void __launch_bounds__(256) k_copy(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int device_cus() {
    int dev = 0, cus = 256;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
        cus = prop.multiProcessorCount;
    return cus;
}

// workgroups of 256 threads for n16 16-byte elements, at most `per_cu` per CU
int blocks_for(size_t n16, int per_cu) {
    size_t want = (n16 + 255) / 256;
    size_t cap = (size_t)device_cus() * (size_t)per_cu;
    return (int)(want < cap ? (want ? want : 1) : cap);
}

}  // namespace

extern "C" {

int mk_bench_stream_read(const void* d_src, size_t bytes, void* d_sink, void* stream) {
    if (!d_src || !d_sink || (bytes & 15) || ((uintptr_t)d_src & 15)) return 1;
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_stream_read, dim3(blocks_for(n16, 16)), dim3(256), 0, (hipStream_t)stream, (const uint4*)d_src,
                       n16, (uint32_t*)d_sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int mk_bench_copy(void* d_dst, const void* d_src, size_t bytes, void* stream) {
    if (!d_src || !d_dst || (bytes & 15) || ((uintptr_t)d_src & 15) || ((uintptr_t)d_dst & 15)) return 1;
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_copy, dim3(blocks_for(n16, 8)), dim3(256), 0, (hipStream_t)stream, (uint4*)d_dst,
                       (const uint4*)d_src, n16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Cost of one all-to-all dependency (every workgroup publishes a slot, signals,
// waits for all, reads every slot back), the synchronisation pattern of the
// decode step.  Slots are double-buffered by round parity, so a fast workgroup
// writing round r + 1 never overwrites what a slow one still reads of round r.
//   mode 0: one counter (atomic add), release / acquire fences, plain data
//   mode 1: one counter, data and ordering through agent-scope relaxed atomics
//   mode 2: one completion flag per workgroup (plain store of the round), fences
//   mode 3: per-workgroup flags, agent-scope relaxed atomics for the data
//   mode 4: no counter or flag: every slot is an 8-byte {value, round} word
//           stored with one agent-scope atomic, and readers re-poll the words
//           whose round does not match yet (the decode step's protocol)
// out[0] = ticks (100 MHz) of `rounds` rounds on workgroup 0, out[1] = data
// mismatches seen by any workgroup.
// ------------------------------------------------------------------------------------------------
namespace {
// mode 4: slots are 8-byte words, data holds 2 * n * 64 of them
__device__ void sync_tagged(uint64_t* data, int rounds, uint64_t* out) {
    const int n = gridDim.x, wg = blockIdx.x, lane = threadIdx.x;
    uint32_t errors = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool lost = false;
    for (int r = 1; r <= rounds && !lost; ++r) {
        uint64_t* buf = data + (size_t)(r & 1) * n * 64;
        const uint64_t v = ((uint64_t)(uint32_t)r << 32) | ((uint32_t)r * 4096u + (uint32_t)wg);
        __hip_atomic_store(&buf[wg * 64 + lane], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every lane reads slot word (k & 63) of workgroups k = lane, lane + 64, ...
        for (int k0 = 0; k0 < n && !lost; k0 += 64) {
            const int k = k0 + lane;
            uint32_t guard = 0;
            bool ok = k >= n;
            while (!__all(ok)) {
                if (!ok) {
                    const uint64_t w = __hip_atomic_load(&buf[k * 64 + (k & 63)], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                    if ((uint32_t)(w >> 32) == (uint32_t)r) {
                        ok = true;
                        errors += ((uint32_t)w != (uint32_t)r * 4096u + (uint32_t)k);
                    }
                }
                if (++guard > 4000000u) {  // bounded: a missing workgroup ends the run
                    lost = true;
                    errors += 1u << 20;
                    break;
                }
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    for (int m = 32; m >= 1; m >>= 1) errors += __shfl_xor(errors, m, 64);
    if (lane == 0) {
        if (wg == 0) out[0] = t1 - t0;
        if (errors) atomicAdd((unsigned long long*)&out[1], (unsigned long long)errors);
    }
}

template <int MODE>
__global__ void __launch_bounds__(64) k_sync(uint32_t* ctr, uint32_t* data, int rounds, uint64_t* out) {
    if constexpr (MODE == 4) {
        sync_tagged((uint64_t*)data, rounds, out);
        return;
    }
    constexpr bool kFence = (MODE == 0 || MODE == 2);
    constexpr bool kFlags = (MODE >= 2);
    const int n = gridDim.x, wg = blockIdx.x, lane = threadIdx.x;
    uint32_t* flags = ctr + 64;  // per-workgroup flags follow the counter line
    uint32_t errors = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int r = 1; r <= rounds; ++r) {
        uint32_t* buf = data + (size_t)(r & 1) * n * 64;
        const uint32_t v = (uint32_t)r * 4096u + (uint32_t)wg;
        if (kFence) {
            buf[wg * 64 + lane] = v;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        } else {
            __hip_atomic_store(&buf[wg * 64 + lane], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
        }
        if (lane == 0) {
            if (kFlags)
                __hip_atomic_store(&flags[wg], (uint32_t)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        uint64_t guard = 0;
        for (;;) {
            bool ok;
            if (kFlags) {
                ok = true;
                for (int k = lane; k < n; k += 64)
                    ok &= (int32_t)(__hip_atomic_load(&flags[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                                    (uint32_t)r) >= 0;
                ok = __all(ok);
            } else {
                ok = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)r * (uint32_t)n;
            }
            if (ok) break;
            __builtin_amdgcn_s_sleep(1);
            if (++guard > 20000000ull) break;  // bounded: never spins forever
        }
        if (kFence) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int k = lane; k < n; k += 64) {
            const uint32_t want = (uint32_t)r * 4096u + (uint32_t)k;
            const uint32_t got = kFence ? buf[k * 64 + (k & 63)]
                                        : __hip_atomic_load(&buf[k * 64 + (k & 63)], __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
            errors += (got != want);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    for (int m = 32; m >= 1; m >>= 1) errors += __shfl_xor(errors, m, 64);
    if (lane == 0) {
        if (wg == 0) out[0] = t1 - t0;
        if (errors) atomicAdd((unsigned long long*)&out[1], (unsigned long long)errors);
    }
}
}  // namespace

extern "C" int mk_bench_sync(int mode, int n_wg, int rounds, void* d_ctr, void* d_data, void* d_out, void* stream) {
    if (n_wg < 1 || n_wg > 1024 || rounds < 1 || rounds > 100000 || !d_ctr || !d_data || !d_out || mode < 0 ||
        mode > 4)
        return 1;
    const void* fns[5] = {(const void*)k_sync<0>, (const void*)k_sync<1>, (const void*)k_sync<2>,
                          (const void*)k_sync<3>, (const void*)k_sync<4>};
    void* args[] = {&d_ctr, &d_data, &rounds, &d_out};
    hipError_t e = hipLaunchCooperativeKernel(fns[mode], dim3(n_wg), dim3(64), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : 4;
}

// ------------------------------------------------------------------------------------------------
// One-way latency of a value passed between two workgroups: workgroup 0 and
// workgroup `peer` bounce an 8-byte {round, round} word back and forth `rounds`
// times; the other workgroups of the grid leave at once.  Workgroups are placed
// round-robin over the XCDs, so the peer index picks same-XCD or cross-XCD pairs
// (out[2], out[3] report the XCC of each side).
//   flavor 0: agent-scope relaxed atomic load and store
//   flavor 1: system-scope relaxed atomic load and store
// out[0] = ticks of workgroup 0 for all rounds, out[1] = waits that hit the bound.
// ------------------------------------------------------------------------------------------------
namespace {
__device__ __forceinline__ uint32_t xcc_id() {
    // HW_REG_XCC_ID (hardware register 20), bits [3:0]
    return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 15u;
}

template <int FLAVOR>
__global__ void __launch_bounds__(64) k_pingpong(uint64_t* words, int peer, int rounds, uint64_t* out) {
    const int wg = blockIdx.x;
    if ((wg != 0 && wg != peer) || threadIdx.x != 0) return;
    constexpr int scope = FLAVOR == 0 ? __HIP_MEMORY_SCOPE_AGENT : __HIP_MEMORY_SCOPE_SYSTEM;
    uint64_t* mine = words + (wg == 0 ? 0 : 32);   // 256 bytes apart
    uint64_t* theirs = words + (wg == 0 ? 32 : 0);
    uint64_t misses = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int r = 1; r <= rounds; ++r) {
        const uint64_t want = ((uint64_t)(uint32_t)r << 32) | (uint32_t)r;
        if (wg == 0) __hip_atomic_store(mine, want, __ATOMIC_RELAXED, scope);
        uint32_t guard = 0;
        while ((int32_t)((uint32_t)(__hip_atomic_load(theirs, __ATOMIC_RELAXED, scope) >> 32) - (uint32_t)r) < 0) {
            if (++guard > 4000000u) {
                ++misses;
                break;
            }
        }
        if (misses) break;  // the other side is missing: stop
        if (wg != 0) __hip_atomic_store(mine, want, __ATOMIC_RELAXED, scope);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (wg == 0) {
        out[0] = t1 - t0;
        out[1] += misses;
        out[2] = xcc_id();
    } else {
        out[3] = xcc_id();
        if (misses) atomicAdd((unsigned long long*)&out[1], (unsigned long long)misses);
    }
}
}  // namespace

extern "C" int mk_bench_pingpong(int flavor, int peer, int rounds, void* d_words, void* d_out, void* stream) {
    if (peer < 1 || peer > 255 || rounds < 1 || rounds > 100000 || !d_words || !d_out || flavor < 0 || flavor > 1)
        return 1;
    const void* f = flavor == 0 ? (const void*)k_pingpong<0> : (const void*)k_pingpong<1>;
    void* args[] = {&d_words, &peer, &rounds, &d_out};
    hipError_t e = hipLaunchCooperativeKernel(f, dim3(peer + 1), dim3(64), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : 4;
}

// ------------------------------------------------------------------------------------------------
// One dependency edge of the decode step at its real size, with or without the
// weight stream running beside it.  Each workgroup has four compute waves and
// four streaming waves.  Per round every workgroup publishes `w` 8-byte
// {value, round} words (agent-scope atomic stores), then its compute waves
// gather all n * w words into LDS, re-polling the words whose round does not
// match yet, and meet at a barrier of the four compute waves.  With `stream`
// set, the streaming waves meanwhile read `src` into LDS with direct-to-LDS
// loads (eight 1 KB loads in flight per wave) until the compute waves finish;
// stream == 2 marks those loads non-temporal.
// Words are double-buffered by round parity.  out[0] = ticks of workgroup 0's
// rounds, out[1] = mismatches or lost waits, out[2] = KB streamed by workgroup 0.
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kEdgeMaxWords = 64;

__global__ void __launch_bounds__(512) k_edge(uint64_t* data, int w, int rounds, int stream, const char* src,
                                              size_t src_kb, uint64_t* out) {
    __shared__ float stage[4096];
    __shared__ __attribute__((aligned(1024))) char ring[4 * 8 * 1024];
    __shared__ uint32_t ctl[4];  // barrier arrivals, done flag
    const int n = gridDim.x, wg = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < 4) ctl[tid] = 0;
    __syncthreads();
    if (wave >= 4) {
        // streaming wave: stream its share of src round and round until done
        const int sw = wave - 4;
        const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)ring + sw * 8192u;
        const size_t streams = (size_t)n * 4, sid = (size_t)wg * 4 + sw;
        const size_t per = src_kb / streams;
        uint64_t kb = 0;
        if (stream && per > 0) {
            for (uint32_t guard = 0; guard < (1u << 24); ++guard) {
                if (__hip_atomic_load(&ctl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
                const size_t c = sid * per + (guard % per);
                if (stream == 2)
                    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                                 :
                                 : "{m0}"(__builtin_amdgcn_readfirstlane(base + (guard & 7u) * 1024u)),
                                   "v"(src + c * 1024 + lane * 16)
                                 : "memory");
                else
                    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                                 :
                                 : "{m0}"(__builtin_amdgcn_readfirstlane(base + (guard & 7u) * 1024u)),
                                   "v"(src + c * 1024 + lane * 16)
                                 : "memory");
                __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
                ++kb;
            }
        }
        __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
        if (wg == 0 && sw == 0 && lane == 0) out[2] = kb;
        return;
    }
    const int total = n * w;
    uint32_t errors = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool lost = false;
    for (int r = 1; r <= rounds && !lost; ++r) {
        uint64_t* buf = data + (size_t)(r & 1) * total;
        if (wave == 0 && lane < w) {
            const uint32_t val = (uint32_t)r * 131071u + (uint32_t)(wg * w + lane);
            __hip_atomic_store(&buf[wg * w + lane], ((uint64_t)(uint32_t)r << 32) | val, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        // gather: lane of wave `wave` takes words e = 64 * wave + lane + 256 * i
        for (int e0 = 64 * wave; e0 < total && !lost; e0 += 256 * 16) {
            uint64_t v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = e0 + lane + 256 * i;
                v[i] = e < total ? __hip_atomic_load(&buf[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : ((uint64_t)(uint32_t)r << 32);
            }
            for (uint32_t guard = 0;; ++guard) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < 16; ++i) ok &= (uint32_t)(v[i] >> 32) == (uint32_t)r;
                if (__all(ok)) break;
                if (guard > 4000000u) {
                    lost = true;
                    errors += 1u << 20;
                    break;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = e0 + lane + 256 * i;
                    if ((uint32_t)(v[i] >> 32) != (uint32_t)r)
                        v[i] = __hip_atomic_load(&buf[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = e0 + lane + 256 * i;
                if (e < total) {
                    errors += (uint32_t)v[i] != (uint32_t)r * 131071u + (uint32_t)e;
                    if (e < 4096) stage[e] = __uint_as_float((uint32_t)v[i]);
                }
            }
        }
        // barrier of the four compute waves
        if (lane == 0) __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (uint32_t guard = 0; __hip_atomic_load(&ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <
                                 (uint32_t)(4 * r);
             ++guard) {
            if (guard > 4000000u) {
                lost = true;
                break;
            }
            __builtin_amdgcn_s_sleep(0);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) __hip_atomic_store(&ctl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int m = 32; m >= 1; m >>= 1) errors += __shfl_xor(errors, m, 64);
    if (lane == 0) {
        if (wg == 0 && wave == 0) out[0] = t1 - t0;
        if (errors) atomicAdd((unsigned long long*)&out[1], (unsigned long long)errors);
    }
}
}  // namespace

extern "C" int mk_bench_edge(int n_wg, int words, int rounds, int stream, const void* d_src, size_t src_bytes,
                             void* d_data, void* d_out, void* hstream) {
    if (n_wg < 1 || n_wg > 256 || words < 1 || words > kEdgeMaxWords || rounds < 1 || rounds > 100000 || !d_data ||
        !d_out || (stream && (!d_src || src_bytes < (size_t)n_wg * 4 * 1024)))
        return 1;
    size_t kb = stream ? src_bytes / 1024 : 0;
    void* args[] = {&d_data, &words, &rounds, &stream, (void*)&d_src, &kb, &d_out};
    hipError_t e = hipLaunchCooperativeKernel((const void*)k_edge, dim3(n_wg), dim3(512), args, 0,
                                              (hipStream_t)hstream);
    return e == hipSuccess ? 0 : 4;
}

// ------------------------------------------------------------------------------------------------
// Gap per kernel of a captured graph: a graph of n empty kernels replayed `reps`
// times; the time per kernel is what one op of the one-kernel-per-op path pays
// in launch and boundary cost before it does any work.
// ------------------------------------------------------------------------------------------------
namespace {
__global__ void __launch_bounds__(64) k_empty(int* sink, int v) {
    if (v == 0x7FFFFFFF && threadIdx.x == 0) *sink = v;  // never true; keeps a body
}
}  // namespace

extern "C" int mk_bench_graph_gap(int n_kernels, int reps, int blocks, void* d_sink, float* h_us_per_kernel,
                                  void* stream) {
    if (n_kernels < 1 || n_kernels > 4096 || reps < 1 || blocks < 1 || blocks > 65536 || !d_sink || !h_us_per_kernel)
        return 1;
    hipStream_t st = (hipStream_t)stream;
    hipStream_t cap = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = 4;
    if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) return 4;
    if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) == hipSuccess) {
        for (int i = 0; i < n_kernels; ++i) hipLaunchKernelGGL(k_empty, dim3(blocks), dim3(64), 0, cap, (int*)d_sink, i);
        if (hipStreamEndCapture(cap, &g) == hipSuccess && hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) == hipSuccess &&
            hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
            bool ok = hipGraphLaunch(ge, st) == hipSuccess && hipStreamSynchronize(st) == hipSuccess;  // warm-up
            ok = ok && hipEventRecord(e0, st) == hipSuccess;
            for (int r = 0; r < reps && ok; ++r) ok = hipGraphLaunch(ge, st) == hipSuccess;
            ok = ok && hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
            float ms = 0.f;
            if (ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess) {
                *h_us_per_kernel = ms * 1000.0f / (float)((double)reps * n_kernels);
                rc = 0;
            }
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    (void)hipStreamDestroy(cap);
    return rc;
}

// ------------------------------------------------------------------------------------------------
// The device math the decode step uses, evaluated elementwise so its error can be
// measured against double precision: fn 0 expf (softmax weights), 1 sqrtf, 2 the
// fp32 divide 1 / x, 3 the RMSNorm scale 1 / sqrtf(x), 4 silu(z) = z / (1 + expf(-z)).
// The expressions are the ones the kernel's code uses (same compiler flags).
// ------------------------------------------------------------------------------------------------
namespace {
__global__ void __launch_bounds__(256) k_device_math(int fn, const float* __restrict__ x, float* __restrict__ y,
                                                     size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float v = x[i];
    float r;
    switch (fn) {
        case 0: r = expf(v); break;
        case 1: r = sqrtf(v); break;
        case 2: r = 1.0f / v; break;
        case 3: r = 1.0f / sqrtf(v); break;
        default: r = v / (1.0f + expf(-v)); break;
    }
    y[i] = r;
}
}  // namespace

extern "C" int mk_bench_device_math(int fn, const void* d_x, void* d_y, size_t n, void* stream) {
    if (fn < 0 || fn > 4 || !d_x || !d_y || n == 0) return 1;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_device_math, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, fn,
                       (const float*)d_x, (float*)d_y, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
