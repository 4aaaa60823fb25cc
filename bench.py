#!/usr/bin/env python3
"""Decode benchmark: µs/token of the persistent megakernel at batch 1 on the
Llama-3.2-1B shape (32 prompt tokens, then greedy decode), as a fraction of the
MI355X HBM roofline, next to the one-kernel-per-op hipGraph path, the measured
streaming-read ceiling, and the CPU oracle timed on the host.

One "step" is one decode step (one token per sequence): a single persistent
launch.  Weights are random (seeded, bf16 N(0, 0.02)), inputs already resident
in HBM when timing starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 128] [--warmup 32]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth

# Kernel sources whose hash keys the committed counter summary: the summary's
# traffic figure is reported only while these files are unchanged.
KERNEL_SOURCES = ["persistent_megakernel_02_amd/csrc/megakernel.hip",
                  "persistent_megakernel_02_amd/csrc/megakernel_impl.h",
                  "persistent_megakernel_02_amd/csrc/mk_kernels_valu.hip",
                  "persistent_megakernel_02_amd/csrc/mk_device.h",
                  "persistent_megakernel_02_amd/csrc/mk_internal.h",
                  "persistent_megakernel_02_amd/csrc/host.hip"]
COUNTER_SUMMARY = "profiles/mk_megakernel_llama1b_b1_hbm_counters.md"


def kernel_sources_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per megakernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the factor the same
    counter reads for a copy kernel of known size), or None when the summary is
    missing or was taken from different kernel sources."""
    path = os.path.join(ROOT, COUNTER_SUMMARY)
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_sources_hash():
        return None, "kernel changed since the counters were taken"
    return int(fields["traffic_bytes_per_launch"]), COUNTER_SUMMARY


def profile_run(args) -> int:
    """Workload for the counter runs: a few megakernel decode steps on the 1B
    shape at batch 1, then a 256 MiB device copy whose counter readings give the
    scale factors of FETCH_SIZE and WRITE_SIZE."""
    import torch

    import persistent_megakernel_02_amd.inputs as I
    import persistent_megakernel_02_amd.mk as mk

    cfg = I.LLAMA_1B
    dev = torch.device("cuda:0")
    w = I.make_weights(cfg, seed=args.seed)
    n_prompt, horizon = WORKLOADS["1b"]["prompt"], WORKLOADS["1b"]["horizon"]
    prompt = torch.from_numpy(I.make_prompt(cfg, 1, n_prompt, seed=args.seed)).to(dev)
    dec = mk.Decoder(cfg, w, max_batch=1, max_seq=n_prompt + horizon + 1, device="cuda:0")
    tok, logits = dec.prefill(prompt)
    for _ in range(args.steps):
        dec.decode_step(tok, tok, logits)
    torch.cuda.synchronize()
    dec.close()
    nb = 256 << 20
    a = torch.empty(nb, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        mk.bench_copy(b, a)
    torch.cuda.synchronize()
    log(f"profile run: prefill {n_prompt} + {args.steps} decode steps, 2 copies of {nb} B")
    return 0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prefill_latency(dec, prompt_dev, reps: int = 10) -> dict:
    """Time to process the prompt (first token's latency without queueing): mk_prefill
    (launches of up to 8 prompt positions in the persistent mode) against one decode
    launch per prompt position; median over `reps`, µs, events on the launch stream."""
    import numpy as np
    import torch

    B, P = prompt_dev.shape
    out = {}
    for name in ("multi_position", "one_position_per_launch"):
        times = []
        for r in range(reps + 2):
            dec.set_context_len([0] * B)  # synchronises
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(dec.stream)
            if name == "multi_position":
                dec.prefill(prompt_dev)
            else:
                for t in range(P):
                    dec.decode_step(prompt_dev[:, t].contiguous())
            e1.record(dec.stream)
            e1.synchronize()
            if r >= 2:
                times.append(e0.elapsed_time(e1) * 1000.0)
        out[f"us_{name}"] = round(float(np.median(times)), 1)
    out["prompt_tokens"] = int(P)
    return out


def cut_study(dec, start, steps: int = 64) -> dict:
    """The decode step as k persistent launches (mk_set_cuts, equal layer runs):
    measured µs/step for k = 1, 2, 4 and one launch per layer plus the LM head;
    the cut planner, given the one- and two-launch figures (their difference is
    one launch plus the prefetch lost at a cut), predicts the others and picks
    the design."""
    import numpy as np
    import torch

    import persistent_megakernel_02_amd.mk as mk

    L = dec.cfg.n_layers
    designs = {"1": [], "2": [L // 2], "4": [L // 4, L // 2, 3 * L // 4], str(L + 1): list(range(1, L + 1))}
    measured = {}
    for name, cuts in designs.items():
        dec.set_cuts(cuts)
        times = []
        for rep_ in range(2):
            tok = start()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(dec.stream)
            for _ in range(steps):
                dec.decode_step(tok, tok)
            e1.record(dec.stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1000.0 / steps)
        measured[name] = round(float(np.min(times)), 2)
    dec.set_cuts([])
    t1, t2 = measured["1"], measured["2"]
    per_cut = t2 - t1
    # every launch pays per_cut; the split of the rest between layers and head does not move the choice
    body = (t1 - per_cut) / (L + 1)
    plan = mk.plan_cuts([body] * L, launch_us=per_cut, head_us=body, refill_us=None)
    predicted = {name: round(t1 + (len(cuts)) * per_cut, 2) for name, cuts in designs.items()}
    return {"launches_per_step": list(designs), "measured_us": measured, "predicted_us": predicted,
            "cost_per_cut_us": round(per_cut, 2), "planner_cuts": plan["cuts"],
            "planner_predicted_us": round(plan["predicted_us"], 2)}


def micro_benchmarks(dev, n_cu: int) -> dict:
    """The synchronisation and launch costs the persistent kernel is built
    around: the gap one kernel boundary costs inside a replayed hipGraph, an
    all-to-all dependency round over every CU with a counter + fences and with
    tagged words, the one-way CU-to-CU latency across and within an XCD, and one
    dependency edge at the decode step's sizes idle and under a full weight
    stream.  Every figure is a mean over many rounds, in microseconds."""
    import torch

    import persistent_megakernel_02_amd.mk as mk

    out = {"graph_gap_us_per_kernel": round(mk.bench_graph_gap(1000, 10, n_cu), 3)}
    for name, mode in (("counter_fences", 0), ("tagged_words", 4)):
        r = mk.bench_sync(mode, n_cu, 2000)
        if r["mismatches"]:
            raise RuntimeError(f"sync benchmark mode {mode}: {r['mismatches']} mismatches")
        out[f"all_to_all_round_us_{name}"] = round(r["us_per_round"], 3)
    for name, peer in (("cross_xcd", 1), ("same_xcd", 8)):
        r = mk.bench_pingpong(peer, 20000)
        if r["lost"]:
            raise RuntimeError(f"pingpong benchmark peer {peer}: {r['lost']} lost waits")
        out[f"one_way_us_{name}"] = round(r["us_one_way"], 3)
        out[f"one_way_xcc_{name}"] = r["xcc"]
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)  # 1 GiB: beyond the 256 MiB last-level cache
    for words in (8, 32):
        for name, s in (("idle", None), ("streaming", src)):
            r = mk.bench_edge(n_cu, words, 1000, s)
            if r["mismatches"]:
                raise RuntimeError(f"edge benchmark {words} words: {r['mismatches']} mismatches")
            out[f"edge_us_{n_cu * words}_words_{name}"] = round(r["us_per_round"], 3)
    del src
    return out


def expert_bytes(cfg) -> int:
    """Bytes of one expert's gate, up and down matrices (bf16)."""
    return 3 * cfg.expert_ffn * cfg.hidden * 2


def step_bytes(cfg, batch: int, positions, slots_per_step: float = 0.0) -> int:
    """Algorithmic HBM bytes of one decode step: every weight byte once, each
    sequence's embedding row, the K/V of its cached positions read once per
    (sequence, KV head), its new K/V written, the fp32 logits written.
    `positions`: the position each sequence decodes at this step (one per sequence,
    or a single value shared by all).  MoE: only the streamed expert slots count,
    `slots_per_step` of them summed over the layers (the shared experts plus the
    union the router selected, as the kernel counts them)."""
    kv_pos = cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * 2
    pos = [int(p) for p in positions]
    if len(pos) == 1:
        pos = pos * batch
    w = cfg.weight_bytes()
    if cfg.is_moe:
        w -= (cfg.n_experts + cfg.n_shared) * expert_bytes(cfg) * cfg.n_layers
        w += int(round(slots_per_step * expert_bytes(cfg)))
    b = w + batch * cfg.hidden * 2
    b += sum(pos) * kv_pos     # cached positions 0..p-1 read
    b += batch * kv_pos        # position p written
    b += batch * cfg.vocab * 4
    return b


# Workloads: model, batch, prompt tokens (or a synthetic context), decode steps
# per horizon.  "1b" is the headline one.
WORKLOADS = {
    "1b": dict(model="LLAMA_1B", batch=1, prompt=32, ctx=0, horizon=128,
               text="llama-3.2-1b-shape decode, batch 1, 32 prompt tokens then greedy steps"),
    "1b-b4": dict(model="LLAMA_1B", batch=4, prompt=0, ctx=8192, horizon=128,
                  text="llama-3.2-1b-shape decode, batch 4, 8192-position synthetic bf16 KV context per sequence"),
    "1b-b8": dict(model="LLAMA_1B", batch=8, prompt=0, ctx=8192, horizon=128,
                  text="llama-3.2-1b-shape decode, batch 8, 8192-position synthetic bf16 KV context per sequence"),
    "8b": dict(model="LLAMA_8B", batch=1, prompt=128, ctx=0, horizon=256,
               text="llama-3-8b-shape decode, batch 1, 128 prompt tokens then greedy steps"),
    "moe-b4": dict(model="MOE", batch=4, prompt=0, ctx=4096, horizon=64,
                   text="synthetic MoE decode (64 experts, top 6, one shared), batch 4, 4096-position synthetic "
                        "bf16 KV context per sequence"),
    "moe-b8": dict(model="MOE", batch=8, prompt=0, ctx=4096, horizon=64,
                   text="synthetic MoE decode (64 experts, top 6, one shared), batch 8, 4096-position synthetic "
                        "bf16 KV context per sequence"),
}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="1b", choices=sorted(WORKLOADS))
    ap.add_argument("--gemv", default="auto", choices=["auto", "valu", "mfma"],
                    help="GEMV arithmetic of the persistent kernel (auto: matrix cores from batch 4)")
    ap.add_argument("--down-split", default="auto", choices=["auto", "on", "off"],
                    help="dense down projection split by columns (automatic: batch 4 and 8)")
    ap.add_argument("--no-graph", action="store_true", help="skip the one-kernel-per-op comparison")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=24)
    ap.add_argument("--no-micro", action="store_true", help="skip the synchronisation / launch micro-benchmarks")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--profile-run", action="store_true",
                    help="untimed workload for rocprofv3 counter runs (no JSON line)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this decode path runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not built)"}))
        return 2

    if args.profile_run:
        return profile_run(args)

    import numpy as np
    import torch

    import persistent_megakernel_02_amd.inputs as I
    import persistent_megakernel_02_amd.mk as mk

    W = WORKLOADS[args.config]
    cfg = getattr(I, W["model"])
    B, H, CTX = W["batch"], W["horizon"], W["ctx"]
    P = W["prompt"] if CTX == 0 else CTX  # position of the first timed step
    max_seq = P + H + 1
    dev = torch.device("cuda:0")
    t0 = time.time()
    w = I.make_weights(cfg, seed=args.seed)
    prompt = I.make_prompt(cfg, B, max(1, W["prompt"]), seed=args.seed)
    log(f"weights generated in {time.time() - t0:.1f}s")
    dw = mk.upload_weights(w, dev)
    torch.cuda.synchronize()
    prompt_dev = torch.from_numpy(prompt).to(dev)
    kv_host = None
    if CTX:
        shape = (cfg.n_layers, B, cfg.n_kv_heads, max_seq, cfg.head_dim)
        kv_host = (np.zeros(shape, np.uint16), np.zeros(shape, np.uint16))
        I.fill_kv_context(cfg, kv_host[0], kv_host[1], B, CTX, seed=args.seed)
        log(f"synthetic context of {CTX} positions filled in {time.time() - t0:.1f}s")

    gemv = {"auto": mk.MK_GEMV_AUTO, "valu": mk.MK_GEMV_VALU, "mfma": mk.MK_GEMV_MFMA}[args.gemv]

    def run_path(mode: int, label: str):
        dec = mk.Decoder(cfg, w, max_batch=B, max_seq=max_seq, mode=mode, device="cuda:0", device_weights=dw,
                         gemv_kind=gemv if mode == mk.MK_MODE_MEGAKERNEL else mk.MK_GEMV_AUTO,
                         down_split={"auto": 0, "on": 1, "off": -1}[args.down_split])
        st = dec.stream
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device=dev)
        if kv_host is not None:
            kd, vd = dec.kv_views()
            kd.copy_(torch.from_numpy(kv_host[0].view(np.int16)))
            vd.copy_(torch.from_numpy(kv_host[1].view(np.int16)))
            torch.cuda.synchronize()

        def start_horizon():
            if CTX:
                dec.set_context_len([CTX] * B)
                tok.copy_(prompt_dev[:, 0])
            else:
                dec.set_context_len([0] * B)
                dec.prefill(prompt_dev, logits, tok)

        # warmup
        start_horizon()
        done = 0
        for _ in range(args.warmup):
            if done == H:
                start_horizon()
                done = 0
            dec.decode_step(tok, tok, logits)
            done += 1
        torch.cuda.synchronize()
        # timed: horizons of <= H steps from the prompt; events on the launch stream
        total_ms, left, positions, per_h = 0.0, args.steps, [], []
        slots = 0
        while left > 0:
            n = min(left, H)
            start_horizon()
            torch.cuda.synchronize()
            slots0 = dec.moe_slots() if cfg.is_moe else 0
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for i in range(n):
                dec.decode_step(tok, tok, logits)
            e1.record(st)
            e1.synchronize()
            if cfg.is_moe:
                slots += dec.moe_slots() - slots0
            ms = e0.elapsed_time(e1)
            total_ms += ms
            per_h.append(ms * 1000.0 / n)
            positions.extend(range(P, P + n))
            left -= n
        # separate pass with an event after every step, for the percentiles and the
        # time against the context length
        per_step, per_pos = [], []
        left = args.steps
        while left > 0:
            n = min(left, H)
            start_horizon()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record(st)
            for i in range(n):
                dec.decode_step(tok, tok, logits)
                ev[i + 1].record(st)
            ev[-1].synchronize()
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(n))
            per_pos.extend((P + i, ev[i].elapsed_time(ev[i + 1]) * 1000.0) for i in range(n))
            left -= n
        kps = dec.kernels_per_step()
        dec.close()
        us = total_ms * 1000.0 / args.steps
        pct = (float(np.percentile(per_step, 50)), float(np.percentile(per_step, 95)))
        log(f"{label}: {us:.1f} us/token over {args.steps} steps ({kps} kernels/step), "
            f"p50 {pct[0]:.1f} p95 {pct[1]:.1f}")
        # mean step time over quarters of the horizon (the context grows by one per step)
        by_pos = {}
        q = max(1, H // 4)
        for a in range(P, P + H, q):
            vals = [t for p_, t in per_pos if a <= p_ < a + q]
            if vals:
                by_pos[f"{a}-{a + q - 1}"] = round(float(np.mean(vals)), 2)
        return us, positions, kps, per_h, pct, slots / args.steps, by_pos

    gemv_used = mk.mk_plan_inspect(mk.model_config(cfg), mk.runtime_config(B, max_seq, gemv_kind=gemv),
                                   torch.cuda.get_device_properties(dev).multi_processor_count)[1]["gemv_kind"]
    us_mk, positions, kps_mk, per_h, pct_mk, slots_step, by_pos = run_path(mk.MK_MODE_MEGAKERNEL, "megakernel")
    prefill = cuts = None
    if CTX == 0:
        pdec = mk.Decoder(cfg, w, max_batch=B, max_seq=max_seq, device="cuda:0", device_weights=dw)
        prefill = prefill_latency(pdec, prompt_dev)
        log(f"prefill of {prefill['prompt_tokens']} tokens: {prefill}")
        if args.config == "1b" and not args.no_micro:

            def restart():
                pdec.set_context_len([0] * B)
                nxt, _ = pdec.prefill(prompt_dev)
                return nxt

            cuts = cut_study(pdec, restart)
            log(f"cut study: {cuts}")
        pdec.close()
    # every sequence at position p; MoE: the expert slots the kernel counted, mean per step
    bytes_step = [step_bytes(cfg, B, [p], slots_step) for p in positions]
    mean_bytes = float(np.mean(bytes_step))
    gbs = mean_bytes / (us_mk * 1e-6) / 1e9

    us_graph = kps_graph = pct_graph = None
    if not args.no_graph and not cfg.is_moe:  # the one-kernel-per-op path has no MoE kernels
        us_graph, _, kps_graph, _, pct_graph, _, _ = run_path(mk.MK_MODE_GRAPH, "hipGraph one-kernel-per-op")

    # streaming-read ceiling on a buffer the size of the step
    buf = torch.empty(int(mean_bytes) // 16 * 16, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        mk.bench_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reps = 10
    for _ in range(reps):
        mk.bench_stream_read(buf, sink)
    e1.record()
    e1.synchronize()
    ceil_gbs = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    log(f"streaming-read ceiling: {ceil_gbs:.0f} GB/s")

    micro = None
    if not args.no_micro and args.config == "1b":
        micro = micro_benchmarks(dev, torch.cuda.get_device_properties(dev).multi_processor_count)
        log(f"micro-benchmarks: {micro}")

    cpu = None
    if not args.no_cpu:
        import oracle as O

        orc = O.Oracle(cfg, w, B, max_seq)
        nsteps = args.cpu_steps if B == 1 and cfg is I.LLAMA_1B else 4
        if CTX:
            orc.set_context(CTX, lambda k, v: (np.copyto(k, kv_host[0]), np.copyto(v, kv_host[1])))
            nxt = prompt[:, 0]
        else:
            nxt, _ = orc.prefill(prompt[:, :4])
            orc.pos[:] = P
        step_us = []
        for _ in range(nsteps):
            t2 = time.time()
            nxt, _ = orc.step(nxt)
            step_us.append((time.time() - t2) * 1e6)
        cpu_us = float(np.median(step_us))  # median over the sampled steps
        cpu = {"value": round(cpu_us, 1), "unit": "us/token" if B == 1 else "us/step", "cores": O.threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "tokens_per_s": round(B * 1e6 / cpu_us, 2),
               "sample": f"median of {nsteps} batch-{B} decode steps of the same {cfg.name} model at positions "
                         f"{P}..{P + nsteps - 1} (fp64-accumulated C oracle, OpenMP over rows)"}
        log(f"cpu oracle: {cpu_us / 1000:.1f} ms/step on {O.threads()} threads")

    traffic, traffic_src = counter_traffic() if args.config == "1b" else (None, "counters taken for the 1b workload only")
    headline = args.config == "1b"
    out = {
        "metric": "decode us/token at batch 1 (Llama-3.2-1B shape) + % of peak HBM BW" if headline
        else f"decode us/step ({W['text']}) + % of peak HBM BW",
        "value": round(us_mk, 2),
        "unit": "us/token" if B == 1 else "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_mk / 1000.0, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W["text"] + ", random bf16 weights N(0,0.02)", "batch": B,
                   "prompt": W["prompt"], "context": CTX, "horizon": H,
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "vocab": cfg.vocab,
                   "gemv": "mfma" if gemv_used == mk.MK_GEMV_MFMA else "valu",
                   "expert_slots_per_step": round(slots_step, 2) if cfg.is_moe else None},
        "tokens_per_s": round(B * 1e6 / us_mk, 1),
        "us_per_token_p50": round(pct_mk[0], 2),
        "us_per_token_p95": round(pct_mk[1], 2),
        "pct_peak_hbm": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "pct_stream_ceiling": round(100.0 * gbs / ceil_gbs, 2),
        "stream_read_ceiling_gbs": round(ceil_gbs, 1),
        "kernels_per_step": kps_mk,
        "us_per_token_per_horizon": [round(x, 2) for x in per_h],
        "us_per_step_by_position": by_pos,
        "graph_path": None if us_graph is None else {"us_per_token": round(us_graph, 2),
                                                     "p50": round(pct_graph[0], 2),
                                                     "p95": round(pct_graph[1], 2),
                                                     "kernels_per_step": kps_graph,
                                                     "pct_peak_hbm": round(100.0 * mean_bytes / (us_graph * 1e-6)
                                                                           / 1e9 / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic if headline else None,
                     "bytes_per_launch": int(mean_bytes), "traffic_source": traffic_src},
        "cpu_baseline": cpu,
        "micro": micro,
        "prefill": prefill,
        "cuts": cuts,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    # Return normally on success: a profiler that writes its results from exit
    # handlers has lost them when the interpreter left through SystemExit.
    rc = main()
    if rc:
        sys.exit(rc)
