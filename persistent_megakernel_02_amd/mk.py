"""Python binding of the C ABI in ``include/mk.h`` (argument marshalling only).

Every function keeps the C name.  PyTorch provides device memory and streams:
the weights, workspace, KV cache, token and logit buffers are torch tensors on
the GPU whose pointers are handed to the library; every step of the decode path
runs in the HIP kernels of ``libmk.so``.  There is no fallback: if the library
is missing the import raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")
TRACE_WORDS = 12  # uint32 per trace record (include/mk.h, mk_read_trace)

MK_OK, MK_E_INVALID, MK_E_UNSUPPORTED, MK_E_CAPACITY, MK_E_HIP, MK_E_DEVICE_TIMEOUT, MK_E_STATE, MK_E_DEVICE_NAN = range(8)
MK_MODE_MEGAKERNEL, MK_MODE_GRAPH, MK_MODE_ENV = 0, 1, 2
MK_GEMV_AUTO, MK_GEMV_VALU, MK_GEMV_MFMA = 0, 1, 2

EXPORTS = ["mk_query_sizes", "mk_create", "mk_create_static", "mk_kv_layout", "mk_prefill", "mk_set_context_len", "mk_decode_step",
           "mk_get_context_len", "mk_reset", "mk_debug_inject", "mk_status_string", "mk_last_error",
           "mk_plan_inspect", "mk_kernels_per_step", "mk_destroy", "mk_bench_stream_read", "mk_bench_copy",
           "mk_bench_sync", "mk_read_trace", "mk_bench_pingpong", "mk_bench_edge", "mk_bench_graph_gap", "mk_moe_slots", "mk_verify_step", "mk_set_cuts",
           "mk_event_sim", "mk_plan_cuts", "mk_bench_device_math"]


class mk_model_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_double), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared_experts", ctypes.c_int32), ("expert_ffn", ctypes.c_int32)]


class mk_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up",
                                               "w_down", "router", "e_gate", "e_up", "e_down", "s_gate", "s_up",
                                               "s_down")]


class mk_weights(ctypes.Structure):
    _fields_ = [("tok_embedding", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(mk_layer_weights))]


MK_EVENT_MAX_DEPS = 8


class mk_event_task(ctypes.Structure):
    _fields_ = [("duration", ctypes.c_double), ("dispatch", ctypes.c_double), ("stream", ctypes.c_int32),
                ("n_deps", ctypes.c_int32), ("deps", ctypes.c_int32 * MK_EVENT_MAX_DEPS)]


class mk_cut_costs(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("launch_us", ctypes.c_double),
                ("layer_us", ctypes.POINTER(ctypes.c_double)), ("refill_us", ctypes.POINTER(ctypes.c_double)),
                ("head_us", ctypes.c_double), ("conventional_us", ctypes.c_double)]


class mk_runtime_config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("gemv_kind", ctypes.c_int32), ("spin_timeout_ms", ctypes.c_uint32),
                ("trace", ctypes.c_int32), ("attn_splits", ctypes.c_int32), ("down_split", ctypes.c_int32)]


_lib = None

# Handles still open when the interpreter exits are destroyed from an atexit hook:
# Python runs it before it tears down modules and before the HIP runtime's own
# exit handlers, so mk_destroy still has a live runtime.  A Decoder collected
# during interpreter finalisation makes no library call at all.
_live: "weakref.WeakSet[Decoder]" = weakref.WeakSet()


def _close_live_handles() -> None:
    for d in list(_live):
        try:
            d.close()
        except Exception:
            pass


atexit.register(_close_live_handles)


def lib():
    """Load libmk.so (built in-tree by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mk_query_sizes.argtypes = [ctypes.POINTER(mk_model_config), ctypes.POINTER(mk_runtime_config),
                                     ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.mk_create.argtypes = [ctypes.POINTER(mk_model_config), ctypes.POINTER(mk_weights),
                                ctypes.POINTER(mk_runtime_config), vp, sz, vp, sz, vp, ctypes.POINTER(vp)]
        L.mk_create_static.argtypes = [ctypes.POINTER(mk_model_config), ctypes.POINTER(mk_weights),
                                       ctypes.POINTER(mk_runtime_config), vp, sz, vp, ctypes.POINTER(vp)]
        L.mk_kv_layout.argtypes = [vp, ctypes.POINTER(ctypes.c_int64)]
        L.mk_prefill.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.mk_set_context_len.argtypes = [vp, ctypes.POINTER(i32), i32]
        L.mk_get_context_len.argtypes = [vp, ctypes.POINTER(i32), i32]
        L.mk_decode_step.argtypes = [vp, vp, i32, vp, vp, vp]
        L.mk_reset.argtypes = [vp, vp]
        L.mk_debug_inject.argtypes = [vp, i32, i32]
        L.mk_status_string.argtypes = [ctypes.c_int]
        L.mk_status_string.restype = ctypes.c_char_p
        L.mk_last_error.argtypes = [vp]
        L.mk_last_error.restype = ctypes.c_char_p
        L.mk_plan_inspect.argtypes = [ctypes.POINTER(mk_model_config), ctypes.POINTER(mk_runtime_config), i32,
                                      ctypes.POINTER(ctypes.c_int64), i32]
        L.mk_kernels_per_step.argtypes = [vp]
        L.mk_kernels_per_step.restype = i32
        L.mk_destroy.argtypes = [vp]
        L.mk_bench_stream_read.argtypes = [vp, sz, vp, vp]
        L.mk_bench_copy.argtypes = [vp, vp, sz, vp]
        L.mk_bench_sync.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
        L.mk_bench_pingpong.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.mk_bench_edge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, sz, vp, vp, vp]
        L.mk_read_trace.argtypes = [vp, vp, sz, ctypes.POINTER(sz), ctypes.POINTER(i32)]
        L.mk_bench_graph_gap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.POINTER(ctypes.c_float), vp]
        L.mk_moe_slots.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64)]
        L.mk_verify_step.argtypes = [vp, i32, vp, i32, vp, vp, vp]
        L.mk_set_cuts.argtypes = [vp, vp, i32]
        L.mk_event_sim.argtypes = [vp, i32, vp]
        L.mk_bench_device_math.argtypes = [ctypes.c_int, vp, vp, sz, vp]
        L.mk_plan_cuts.argtypes = [ctypes.POINTER(mk_cut_costs), vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        for n in ("mk_query_sizes", "mk_create", "mk_create_static", "mk_kv_layout", "mk_prefill", "mk_set_context_len",
                  "mk_get_context_len", "mk_decode_step", "mk_reset", "mk_debug_inject", "mk_plan_inspect",
                  "mk_destroy", "mk_bench_stream_read", "mk_bench_copy", "mk_bench_sync", "mk_read_trace",
                  "mk_bench_pingpong", "mk_bench_edge", "mk_bench_graph_gap", "mk_moe_slots", "mk_verify_step", "mk_set_cuts",
                  "mk_event_sim", "mk_plan_cuts", "mk_bench_device_math"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


class MKError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = lib().mk_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status}){': ' + detail if detail else ''}")


def model_config(cfg) -> mk_model_config:
    """Marshal a ModelConfig-like object (see persistent_megakernel_02_amd.inputs)."""
    c = mk_model_config()
    c.n_layers, c.hidden, c.n_q_heads, c.n_kv_heads = cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads
    c.head_dim, c.ffn, c.vocab = cfg.head_dim, cfg.ffn, cfg.vocab
    c.tied_embeddings = 1 if cfg.tied else 0
    c.rms_eps = cfg.rms_eps
    c.rope_theta = cfg.rope_theta
    c.n_experts, c.top_k, c.n_shared_experts, c.expert_ffn = cfg.n_experts, cfg.top_k, cfg.n_shared, cfg.expert_ffn
    return c


def runtime_config(max_batch: int, max_seq: int, mode: int = MK_MODE_MEGAKERNEL, num_cus: int = 0,
                   spin_timeout_ms: int = 0, attn_splits: int = 0, trace: int = 0,
                   gemv_kind: int = MK_GEMV_AUTO, down_split: int = 0) -> mk_runtime_config:
    r = mk_runtime_config()
    r.max_batch, r.max_seq, r.mode, r.num_cus = max_batch, max_seq, mode, num_cus
    r.gemv_kind, r.spin_timeout_ms, r.trace, r.attn_splits = gemv_kind, spin_timeout_ms, trace, attn_splits
    r.down_split = down_split
    return r


def mk_query_sizes(cfg: mk_model_config, rt: mk_runtime_config):
    ws, kv = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib().mk_query_sizes(ctypes.byref(cfg), ctypes.byref(rt), ctypes.byref(ws), ctypes.byref(kv))
    return st, ws.value, kv.value


def mk_plan_inspect(cfg: mk_model_config, rt: mk_runtime_config, num_cus: int):
    keys = ["cus", "instructions", "ring_chunks", "max_per_cu", "weight_bytes", "verify", "attn_splits", "phases",
            "x_bytes", "head_instructions", "gemv_kind", "attn_hsplit", "max_wave_span", "down_split",
            "gateup_by_loaders", "down_quarters", "o_by_loaders"]
    out = (ctypes.c_int64 * len(keys))()
    st = lib().mk_plan_inspect(ctypes.byref(cfg), ctypes.byref(rt), num_cus, out, len(keys))
    return st, dict(zip(keys, list(out)))


def _stream_ptr(stream) -> Optional[int]:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Decoder:
    """Owns the torch device buffers for one handle: weights, workspace, KV cache.

    ``weights`` is an inputs.Weights (numpy bf16 bit patterns); they are copied to
    the GPU once.  Tokens and logits stay on the GPU between steps.
    """

    def __init__(self, cfg, weights, max_batch: int, max_seq: int, mode: int = MK_MODE_MEGAKERNEL,
                 device: str = "cuda:0", num_cus: int = 0, spin_timeout_ms: int = 0, attn_splits: int = 0,
                 device_weights: Optional[Dict[str, object]] = None, trace: int = 0,
                 gemv_kind: int = 0, static_workspace: bool = False, down_split: int = 0):
        import torch

        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.B = max_batch
        self.max_seq = max_seq
        self._c = model_config(cfg)
        self._rt = runtime_config(max_batch, max_seq, mode, num_cus, spin_timeout_ms, attn_splits, trace, gemv_kind,
                                  down_split)
        st, ws, kv = mk_query_sizes(self._c, self._rt)
        if st != MK_OK:
            raise MKError(st, "mk_query_sizes")
        self._keep: List[object] = []
        dw = device_weights if device_weights is not None else upload_weights(weights, self.device)
        self.dw = dw
        L = self.cfg.n_layers
        layers = (mk_layer_weights * L)()
        for l in range(L):
            dl = dw["layers"][l]
            for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down", "router", "s_gate",
                      "s_up", "s_down"):
                if n in dl:
                    setattr(layers[l], n, dl[n].data_ptr())
            for n in ("e_gate", "e_up", "e_down"):  # host arrays of per-expert device pointers
                if n in dl:
                    arr = (ctypes.c_void_p * len(dl[n]))(*[t.data_ptr() for t in dl[n]])
                    self._keep.append(arr)
                    setattr(layers[l], n, ctypes.cast(arr, ctypes.c_void_p))
        self._layers = layers
        w = mk_weights()
        w.tok_embedding = dw["embed"].data_ptr()
        w.lm_head = dw["lm_head"].data_ptr() if dw.get("lm_head") is not None else None
        w.final_norm = dw["final_norm"].data_ptr()
        w.layers = layers
        self._w = w
        self.kv = torch.empty(kv, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        if static_workspace:
            # the library's static per-device workspace (mk_create_static): no workspace tensor
            self.workspace = None
            st = lib().mk_create_static(ctypes.byref(self._c), ctypes.byref(w), ctypes.byref(self._rt),
                                        self.kv.data_ptr(), kv, self.stream.cuda_stream, ctypes.byref(h))
            if st != MK_OK:
                raise MKError(st, "mk_create_static")
        else:
            self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
            st = lib().mk_create(ctypes.byref(self._c), ctypes.byref(w), ctypes.byref(self._rt),
                                 self.workspace.data_ptr(), ws, self.kv.data_ptr(), kv, self.stream.cuda_stream,
                                 ctypes.byref(h))
            if st != MK_OK:
                raise MKError(st, "mk_create")
        self.h = h
        _live.add(self)
        self.tok = torch.zeros(max_batch, dtype=torch.int32, device=self.device)
        self.logits = torch.empty((max_batch, cfg.vocab), dtype=torch.float32, device=self.device)

    # -- ABI wrappers --------------------------------------------------------------------------
    def _check(self, st: int, where: str):
        if st != MK_OK:
            raise MKError(st, where, lib().mk_last_error(self.h).decode())

    def kv_layout(self):
        s = (ctypes.c_int64 * 5)()
        self._check(lib().mk_kv_layout(self.h, s), "mk_kv_layout")
        return list(s)

    def kv_views(self):
        """(K, V) uint16 views [L][B][Hkv][S][hd] of the cache."""
        t = self.torch
        c = self.cfg
        shape = (c.n_layers, self.B, c.n_kv_heads, self.max_seq, c.head_dim)
        n = int(np.prod(shape))
        flat = self.kv.view(t.int16)
        return flat[:n].view(shape), flat[n:2 * n].view(shape)

    def prefill(self, prompt_dev, logits_out=None, next_out=None):
        """prompt_dev int32 [B, P] on the device -> (next tokens [B], logits [B, V]) device tensors."""
        t = self.torch
        B, P = prompt_dev.shape
        logits_out = self.logits if logits_out is None else logits_out
        next_out = self.tok if next_out is None else next_out
        self._check(lib().mk_prefill(self.h, prompt_dev.data_ptr(), B, P, logits_out.data_ptr(), next_out.data_ptr(),
                                     self.stream.cuda_stream), "mk_prefill")
        return next_out, logits_out

    def decode_step(self, tok_in, tok_out=None, logits_out=None):
        tok_out = self.tok if tok_out is None else tok_out
        logits_out = self.logits if logits_out is None else logits_out
        self._check(lib().mk_decode_step(self.h, tok_in.data_ptr(), self.B, tok_out.data_ptr(), logits_out.data_ptr(),
                                         self.stream.cuda_stream), "mk_decode_step")
        return tok_out, logits_out

    def set_context_len(self, lens: Sequence[int]):
        arr = (ctypes.c_int32 * self.B)(*[int(x) for x in lens])
        self._check(lib().mk_set_context_len(self.h, arr, self.B), "mk_set_context_len")

    def context_len(self):
        arr = (ctypes.c_int32 * self.B)()
        self._check(lib().mk_get_context_len(self.h, arr, self.B), "mk_get_context_len")
        return list(arr)

    def reset(self):
        self._check(lib().mk_reset(self.h, self.stream.cuda_stream), "mk_reset")

    def debug_inject(self, fault: int, arg: int = 0):
        self._check(lib().mk_debug_inject(self.h, fault, arg), "mk_debug_inject")

    def read_trace(self):
        """Timeline of the last megakernel step: uint32 [n_cu, records, TRACE_WORDS] (see mk.h)."""
        n, per = ctypes.c_size_t(0), ctypes.c_int32(0)
        self._check(lib().mk_read_trace(self.h, None, 0, ctypes.byref(n), ctypes.byref(per)), "mk_read_trace")
        buf = np.zeros(n.value // 4, np.uint32)
        self._check(lib().mk_read_trace(self.h, buf.ctypes.data, n.value, ctypes.byref(n), ctypes.byref(per)),
                    "mk_read_trace")
        return buf.reshape(-1, per.value, TRACE_WORDS)

    def kernels_per_step(self) -> int:
        return int(lib().mk_kernels_per_step(self.h))

    def verify_step(self, seq: int, tokens, logits_out=None, next_out=None):
        """Tokens [n] (n <= 8) at the next positions of sequence `seq` in one launch;
        returns (greedy tokens [n], logits [n, V]) and advances that sequence by n."""
        import torch

        n = int(tokens.numel())
        logits_out = torch.empty((n, self.cfg.vocab), dtype=torch.float32, device=self.device) \
            if logits_out is None else logits_out
        next_out = torch.empty(n, dtype=torch.int32, device=self.device) if next_out is None else next_out
        self._check(lib().mk_verify_step(self.h, int(seq), tokens.data_ptr(), n, logits_out.data_ptr(),
                                         next_out.data_ptr(), self.stream.cuda_stream), "mk_verify_step")
        return next_out, logits_out

    def set_cuts(self, layers: Sequence[int]):
        """Run each decode step as len(layers) + 1 persistent launches, a new one
        starting before each listed layer (mk_set_cuts); [] restores one launch."""
        arr = (ctypes.c_int32 * max(1, len(layers)))(*[int(x) for x in layers])
        self._check(lib().mk_set_cuts(self.h, arr, len(layers)), "mk_set_cuts")

    def moe_slots(self) -> int:
        """Expert slots streamed by the MoE layers since creation (mk_moe_slots)."""
        v = ctypes.c_uint64(0)
        self._check(lib().mk_moe_slots(self.h, ctypes.byref(v)), "mk_moe_slots")
        return int(v.value)

    def close(self):
        if getattr(self, "h", None):
            lib().mk_destroy(self.h)
            self.h = None
        _live.discard(self)

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals such as `sys` may already be None here)
        if _finalizing():
            return  # the atexit hook has closed every live handle already
        try:
            self.close()
        except Exception:
            pass


def upload_weights(weights, device) -> Dict[str, object]:
    """Copy numpy bf16 bit patterns to device int16 tensors (same bytes)."""
    import torch

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device, non_blocking=False)

    out: Dict[str, object] = {"embed": dev(weights.embed), "final_norm": dev(weights.final_norm),
                              "lm_head": dev(weights.lm_head) if weights.lm_head is not None else None, "layers": []}
    for L in weights.layers:
        d = {}
        for k, v in L.items():
            if isinstance(v, np.ndarray):
                d[k] = dev(v)
            elif isinstance(v, (list, tuple)):  # per-expert matrices
                d[k] = [dev(a) for a in v]
        out["layers"].append(d)
    return out


def bench_stream_read(src, sink, stream=None) -> int:
    return lib().mk_bench_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                      _stream_ptr(stream))


def bench_copy(dst, src, stream=None) -> int:
    return lib().mk_bench_copy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(), _stream_ptr(stream))


def _bench_check(rc: int, name: str) -> None:
    if rc != 0:
        raise MKError(MK_E_INVALID if rc == 1 else MK_E_HIP, name)


def bench_sync(mode: int, n_wg: int, rounds: int, device="cuda:0") -> Dict[str, float]:
    """All-to-all dependency rounds of n_wg co-resident workgroups (mode 0: one
    counter with agent-scope release/acquire fences; 4: tagged {value, round}
    words, the decode step's protocol).  Returns microseconds per round and the
    data mismatches seen."""
    import torch

    ctr = torch.zeros(64 + n_wg, dtype=torch.int32, device=device)
    data = torch.zeros(2 * n_wg * 64, dtype=torch.int64, device=device)
    out = torch.zeros(2, dtype=torch.int64, device=device)
    _bench_check(lib().mk_bench_sync(mode, n_wg, rounds, ctr.data_ptr(), data.data_ptr(), out.data_ptr(),
                                     _stream_ptr(None)), "mk_bench_sync")
    torch.cuda.synchronize()
    ticks, bad = (int(x) for x in out.cpu())
    return {"us_per_round": ticks * 0.01 / rounds, "mismatches": bad}


def bench_pingpong(peer: int, rounds: int, flavor: int = 0, device="cuda:0") -> Dict[str, float]:
    """One-way latency of an 8-byte word bounced between workgroup 0 and `peer`
    (agent-scope relaxed atomics for flavor 0).  Returns microseconds one way,
    lost waits, and the XCC of each side."""
    import torch

    words = torch.zeros(64, dtype=torch.int64, device=device)
    out = torch.zeros(4, dtype=torch.int64, device=device)
    _bench_check(lib().mk_bench_pingpong(flavor, peer, rounds, words.data_ptr(), out.data_ptr(),
                                         _stream_ptr(None)), "mk_bench_pingpong")
    torch.cuda.synchronize()
    ticks, lost, x0, x1 = (int(x) for x in out.cpu())
    return {"us_one_way": ticks * 0.01 / rounds / 2.0, "lost": lost, "xcc": [x0, x1]}


def bench_edge(n_wg: int, words: int, rounds: int, src=None, device="cuda:0") -> Dict[str, float]:
    """One dependency edge at the decode step's size: every workgroup publishes
    `words` tagged words and gathers all n_wg * words; with `src` (a uint8 device
    tensor) four waves per workgroup stream it non-temporally into LDS meanwhile.
    Returns microseconds per round and mismatches."""
    import torch

    data = torch.zeros(2 * n_wg * words, dtype=torch.int64, device=device)
    out = torch.zeros(3, dtype=torch.int64, device=device)
    s_ptr, s_bytes, mode = (None, 0, 0) if src is None else (src.data_ptr(), src.numel(), 2)
    _bench_check(lib().mk_bench_edge(n_wg, words, rounds, mode, s_ptr, s_bytes, data.data_ptr(), out.data_ptr(),
                                     _stream_ptr(None)), "mk_bench_edge")
    torch.cuda.synchronize()
    ticks, bad, kb = (int(x) for x in out.cpu())
    return {"us_per_round": ticks * 0.01 / rounds, "mismatches": bad, "kb_streamed_wg0": kb}


def bench_graph_gap(n_kernels: int, reps: int, blocks: int, device="cuda:0") -> float:
    """Mean microseconds per kernel of a captured graph of n_kernels empty kernels."""
    import torch

    sink = torch.zeros(1, dtype=torch.int32, device=device)
    us = ctypes.c_float(0.0)
    torch.cuda.synchronize()
    _bench_check(lib().mk_bench_graph_gap(n_kernels, reps, blocks, sink.data_ptr(), ctypes.byref(us),
                                          _stream_ptr(torch.cuda.current_stream())), "mk_bench_graph_gap")
    return float(us.value)


def event_sim(tasks) -> list:
    """Finish times of event-graph tasks: each a dict(duration, dispatch=0, stream=0,
    deps=()) in dependency order (mk_event_sim)."""
    arr = (mk_event_task * len(tasks))()
    for t, d in zip(arr, tasks):
        t.duration, t.dispatch, t.stream = float(d["duration"]), float(d.get("dispatch", 0.0)), int(d.get("stream", 0))
        deps = list(d.get("deps", ()))
        t.n_deps = len(deps)
        for i, j in enumerate(deps):
            t.deps[i] = int(j)
    out = (ctypes.c_double * max(1, len(tasks)))()
    st = lib().mk_event_sim(arr, len(tasks), out)
    if st != MK_OK:
        raise MKError(st, "mk_event_sim")
    return [float(out[i]) for i in range(len(tasks))]


def plan_cuts(layer_us, launch_us: float, head_us: float, refill_us=None, conventional_us: float = 0.0) -> dict:
    """Best design of a decode step from its service table (mk_plan_cuts)."""
    L = len(layer_us)
    lay = (ctypes.c_double * L)(*layer_us)
    ref = (ctypes.c_double * (L + 1))(*refill_us) if refill_us is not None else None
    c = mk_cut_costs(L, float(launch_us), lay, ref, float(head_us), float(conventional_us))
    cuts = (ctypes.c_int32 * L)()
    n, conv = ctypes.c_int32(0), ctypes.c_int32(0)
    pred, single = ctypes.c_double(0.0), ctypes.c_double(0.0)
    st = lib().mk_plan_cuts(ctypes.byref(c), cuts, ctypes.byref(n), ctypes.byref(pred), ctypes.byref(single),
                            ctypes.byref(conv))
    if st != MK_OK:
        raise MKError(st, "mk_plan_cuts")
    return {"cuts": [int(cuts[i]) for i in range(n.value)], "predicted_us": pred.value,
            "single_launch_us": single.value, "conventional": bool(conv.value)}


def device_math(fn: int, x):
    """The decode step's device math on a CUDA fp32 tensor (mk_bench_device_math)."""
    import torch

    y = torch.empty_like(x)
    _bench_check(lib().mk_bench_device_math(fn, x.data_ptr(), y.data_ptr(), x.numel(), _stream_ptr(None)),
                 "mk_bench_device_math")
    torch.cuda.synchronize()
    return y
