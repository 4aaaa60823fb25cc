/*
 * mk_bench.h - measurement helpers shipped with the decode library.
 *
 * The decode step is bounded by HBM bandwidth, so its report needs the device's
 * practical streaming-read ceiling next to the nominal peak, and the HBM byte
 * counters of the profiler need a calibration against a transfer of known size.
 * (The page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
 * "Megakernel：从零设计的深度融合方案", reports the megakernel as a fraction of
 * memory bandwidth; these kernels give the MI355X denominators.)
 */
#ifndef MK_BENCH_H
#define MK_BENCH_H
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (multiple of 16, 16-byte aligned) from device memory d_src with
 * non-temporal 16-byte vector loads over the whole device (16 workgroups per CU,
 * each reading one contiguous slice with 16 loads in flight per thread); d_sink
 * is a device word the kernel may write.  Enqueued on `stream` (hipStream_t).  Returns 0, 1 on bad arguments,
 * 4 on a launch error. */
int mk_bench_stream_read(const void* d_src, size_t bytes, void* d_sink, void* stream);

/* Copy `bytes` (multiple of 16, both pointers 16-byte aligned) device to device
 * with 16-byte loads and stores.  Same return codes. */
int mk_bench_copy(void* d_dst, const void* d_src, size_t bytes, void* stream);

/* Cost of the all-to-all dependency pattern: n_wg workgroups (one wave each,
 * co-resident, cooperative launch) run `rounds` rounds of publish -> signal ->
 * wait for all -> read every slot (slots double-buffered by round parity).
 * mode 0: one atomic counter + agent-scope release/acquire fences; mode 1: one
 * counter + agent-scope relaxed atomics for data, vmcnt waits; mode 2: one
 * completion flag per workgroup + fences; mode 3: flags + relaxed atomics;
 * mode 4: no counter or flag, every slot an 8-byte {value, round} word that
 * readers re-poll until the round matches (the decode step's protocol).
 * d_ctr: 64 + n_wg zeroed uint32 (counter line, then flags); d_data: 2 * n_wg
 * * 64 uint32 (modes 0-3) or 2 * n_wg * 64 zeroed uint64 (mode 4); d_out: two zeroed uint64 = {ticks of 100 MHz for all rounds on
 * workgroup 0, data mismatches}.  Each wait is bounded, so the kernel ends even
 * if a workgroup is missing.  Returns 0, 1 on bad arguments, 4 on launch error. */
int mk_bench_sync(int mode, int n_wg, int rounds, void* d_ctr, void* d_data, void* d_out, void* stream);

/* One-way latency of a value passed between two workgroups: workgroups 0 and
 * `peer` (1..255) bounce an 8-byte word `rounds` times (flavor 0: agent-scope
 * relaxed atomics; flavor 1: system scope).  Workgroups are dealt round-robin
 * over the XCDs, so `peer` selects a same-XCD or a cross-XCD pair.  d_words: 64
 * zeroed uint64; d_out: four zeroed uint64 = {ticks (100 MHz) of all rounds,
 * waits that hit their bound, XCC id of workgroup 0, XCC id of the peer}.  Each
 * wait is bounded.  Returns 0, 1 on bad arguments, 4 on launch error. */
int mk_bench_pingpong(int flavor, int peer, int rounds, void* d_words, void* d_out, void* stream);

/* One dependency edge of the decode step at its real size: n_wg (1..256)
 * workgroups of four compute and four streaming waves, co-resident (cooperative
 * launch).  Per round each workgroup publishes `words` (1..64) 8-byte {value,
 * round} words; its compute waves gather all n_wg * words into LDS, re-polling
 * stale words, then meet at a barrier.  stream != 0: the streaming waves read
 * d_src (src_bytes >= n_wg * 4 KB) into LDS with direct-to-LDS loads, eight
 * 1 KB loads in flight per wave, for as long as the rounds run (stream == 2:
 * the loads carry the non-temporal hint).  d_data: 2 *
 * n_wg * words zeroed uint64; d_out: three zeroed uint64 = {ticks (100 MHz) of
 * workgroup 0's rounds, mismatches (lost waits count 2^20), KB streamed by
 * workgroup 0's first streaming wave}.  Waits are bounded.  Returns 0, 1 on bad
 * arguments, 4 on launch error. */
int mk_bench_edge(int n_wg, int words, int rounds, int stream, const void* d_src, size_t src_bytes, void* d_data,
                  void* d_out, void* hstream);

/* Launch gap of a captured graph [page "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞",
 * section "传统推理方式效率低下的根源剖析": every kernel boundary costs a launch gap
 * even with graphs]: captures n_kernels (1..4096) empty kernels of `blocks`
 * workgroups, replays the graph once untimed and `reps` times timed on `stream`
 * (synchronised), and writes the mean microseconds per kernel to the host float
 * *h_us_per_kernel.  d_sink: a device int the kernels could write (they never
 * do).  Returns 0, 1 on bad arguments, 4 on a runtime error. */
int mk_bench_graph_gap(int n_kernels, int reps, int blocks, void* d_sink, float* h_us_per_kernel, void* stream);

/* The device math of the decode step, elementwise, for error measurements:
 * fn 0 expf, 1 sqrtf, 2 1.0f / x, 3 1.0f / sqrtf(x), 4 x / (1 + expf(-x)) (silu),
 * the expressions the kernel uses.  d_x, d_y: device fp32 [n].  Enqueued on
 * `stream`.  Returns 0, 1 on bad arguments, 4 on a launch error. */
int mk_bench_device_math(int fn, const void* d_x, void* d_y, size_t n, void* stream);

#ifdef __cplusplus
}
#endif
#endif
