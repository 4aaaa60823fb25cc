"""CPU oracle for the decode step (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain C, fp64
accumulation, OpenMP over output rows) through ctypes and shares no code with
the HIP path: inputs arrive as numpy bf16 bit patterns from the seeded input
generator, through duck-typed config and weight objects.

Every function is pinned by ``tests/test_oracle_pins.py``; see the header of
``oracle.h`` for the sources and the rounding contract.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

c_i32, c_f32, c_f64, c_u16p = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.POINTER(ctypes.c_uint16)


class OrcCfg(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                     "n_experts", "top_k", "n_shared", "expert_ffn")] + [("rms_eps", c_f64),
                                                                                         ("rope_theta", c_f64)]


class OrcLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up",
                                               "w_down", "router", "e_gate", "e_up", "e_down", "s_gate", "s_up",
                                               "s_down")]


class OrcWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(OrcLayer))]


class OrcCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("batch", c_i32), ("max_seq", c_i32)]


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_bf16_bits.argtypes = [c_f32]
        L.orc_dot.restype = c_f32
        L.orc_dot.argtypes = [ctypes.c_void_p, ctypes.c_void_p, c_i32]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, c_i32, c_f64, ctypes.c_void_p]
        L.orc_rope.restype = None
        L.orc_rope.argtypes = [ctypes.c_void_p, c_i32, c_i32, c_f64]
        L.orc_attend.restype = None
        L.orc_attend.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, c_i32, c_i32,
                                 ctypes.c_void_p]
        L.orc_swiglu.restype = c_f32
        L.orc_swiglu.argtypes = [c_f32, c_f32]
        L.orc_argmax.restype = c_i32
        L.orc_argmax.argtypes = [ctypes.c_void_p, c_i32]
        L.orc_route.restype = None
        L.orc_route.argtypes = [ctypes.c_void_p, c_i32, c_i32, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_threads.restype = c_i32
        L.orc_step.restype = ctypes.c_int
        L.orc_step.argtypes = [ctypes.POINTER(OrcCfg), ctypes.POINTER(OrcWeights), ctypes.POINTER(OrcCache), c_i32,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_prefill.restype = ctypes.c_int
        L.orc_prefill.argtypes = [ctypes.POINTER(OrcCfg), ctypes.POINTER(OrcWeights), ctypes.POINTER(OrcCache), c_i32,
                                  c_i32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_sequence.restype = ctypes.c_int
        L.orc_sequence.argtypes = [ctypes.POINTER(OrcCfg), ctypes.POINTER(OrcWeights), ctypes.c_void_p, c_i32,
                                   ctypes.c_void_p]
        L.orc_ffn.restype = ctypes.c_int
        L.orc_ffn.argtypes = [ctypes.POINTER(OrcCfg), ctypes.POINTER(OrcLayer), c_i32, ctypes.c_void_p]
        L.orc_set_moe_trace.restype = None
        L.orc_set_moe_trace.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


# ---------------------------------------------------------------------------------------------
# primitives (thin wrappers, used by the pin tests)
# ---------------------------------------------------------------------------------------------
def bf16_bits(x: float) -> int:
    return int(lib().orc_bf16_bits(float(x)))


def bf16_round(a: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda v: bf16_bits(float(v)), otypes=[np.uint16])
    return (f(np.asarray(a, np.float32)).astype(np.uint32) << 16).view(np.float32)


def dot(w_bits: np.ndarray, x: np.ndarray) -> float:
    w_bits = np.ascontiguousarray(w_bits, np.uint16)
    x = np.ascontiguousarray(x, np.float32)
    assert w_bits.size == x.size
    return float(lib().orc_dot(_ptr(w_bits), _ptr(x), x.size))


def rmsnorm(h: np.ndarray, g_bits: np.ndarray, eps: float) -> np.ndarray:
    h = np.ascontiguousarray(h, np.float32)
    g_bits = np.ascontiguousarray(g_bits, np.uint16)
    out = np.empty_like(h)
    lib().orc_rmsnorm(_ptr(h), _ptr(g_bits), h.size, eps, _ptr(out))
    return out


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    v = np.array(v, np.float32, copy=True)
    lib().orc_rope(_ptr(v), v.size, pos, theta)
    return v


def attend(q: np.ndarray, K_bits: np.ndarray, V_bits: np.ndarray) -> np.ndarray:
    """q [hd] float32, K/V [n, hd] bf16 bits -> o [hd] float32."""
    q = np.ascontiguousarray(q, np.float32)
    K_bits = np.ascontiguousarray(K_bits, np.uint16)
    V_bits = np.ascontiguousarray(V_bits, np.uint16)
    n, hd = K_bits.shape
    o = np.empty(hd, np.float32)
    lib().orc_attend(_ptr(q), _ptr(K_bits), _ptr(V_bits), hd, n, hd, _ptr(o))
    return o


def swiglu(z: float, u: float) -> float:
    return float(lib().orc_swiglu(z, u))


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, np.float32)
    return int(lib().orc_argmax(_ptr(v), v.size))


def route(zeta: np.ndarray, k: int):
    zeta = np.ascontiguousarray(zeta, np.float32)
    sel = np.empty(k, np.int32)
    prob = np.empty(zeta.size, np.float32)
    lib().orc_route(_ptr(zeta), zeta.size, k, _ptr(sel), _ptr(prob))
    return sel, prob


def threads() -> int:
    return int(lib().orc_threads())


# ---------------------------------------------------------------------------------------------
# whole model
# ---------------------------------------------------------------------------------------------
class Oracle:
    """Holds ctypes views of a weight set and a KV cache [L][B][Hkv][S][hd]."""

    def __init__(self, cfg, weights, batch: int, max_seq: int):
        self.cfg = cfg
        self.w = weights
        self.batch = batch
        self.max_seq = max_seq
        c = OrcCfg()
        for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_experts", "top_k",
                  "n_shared", "expert_ffn"):
            setattr(c, n, int(getattr(cfg, n)))
        c.rms_eps = float(cfg.rms_eps)
        c.rope_theta = float(cfg.rope_theta)
        self._cfg = c
        self._keep: List[object] = []
        layers = (OrcLayer * max(1, cfg.n_layers))()
        for l, L in enumerate(weights.layers):
            ol = layers[l]
            for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down", "router", "s_gate",
                      "s_up", "s_down"):
                a = L.get(n)
                if a is not None:
                    setattr(ol, n, _ptr(a))
            for n in ("e_gate", "e_up", "e_down"):
                lst = L.get(n)
                if lst is not None:
                    arr = (ctypes.c_void_p * len(lst))(*[_ptr(a) for a in lst])
                    self._keep.append(arr)
                    setattr(ol, n, ctypes.cast(arr, ctypes.c_void_p))
        self._layers = layers
        ow = OrcWeights()
        ow.embed = _ptr(weights.embed)
        ow.lm_head = _ptr(weights.head)
        ow.final_norm = _ptr(weights.final_norm)
        ow.layers = layers
        self._w = ow
        shape = (cfg.n_layers, batch, cfg.n_kv_heads, max_seq, cfg.head_dim)
        self.k_cache = np.zeros(shape, np.uint16)
        self.v_cache = np.zeros(shape, np.uint16)
        kc = OrcCache()
        kc.k = _ptr(self.k_cache)
        kc.v = _ptr(self.v_cache)
        kc.batch = batch
        kc.max_seq = max_seq
        self._kc = kc
        self.pos = np.zeros(batch, np.int32)

    def step(self, tokens: Sequence[int], moe_trace: bool = False):
        """Feed one token per sequence at the current positions; returns (next tokens, logits [B, V])."""
        B, V = self.batch, self.cfg.vocab
        tok = np.ascontiguousarray(tokens, np.int32).reshape(B)
        logits = np.empty((B, V), np.float32)
        nxt = np.empty(B, np.int32)
        pos = np.ascontiguousarray(self.pos, np.int32)
        sel = prob = None
        if moe_trace and self.cfg.n_experts:
            sel = np.empty((self.cfg.n_layers, B, self.cfg.top_k), np.int32)
            prob = np.empty((self.cfg.n_layers, B, self.cfg.n_experts), np.float32)
            lib().orc_set_moe_trace(_ptr(sel), _ptr(prob))
        try:
            rc = lib().orc_step(ctypes.byref(self._cfg), ctypes.byref(self._w), ctypes.byref(self._kc), B, _ptr(pos),
                                _ptr(tok), _ptr(logits), _ptr(nxt))
        finally:
            if sel is not None:
                lib().orc_set_moe_trace(None, None)
        if rc != 0:
            raise RuntimeError(f"orc_step failed with code {rc}")
        self.pos += 1
        if moe_trace:
            return nxt, logits, sel, prob
        return nxt, logits

    def prefill(self, prompt: np.ndarray, batched: bool = True):
        """prompt [B, P] at the current positions; returns (next tokens, logits of the
        last position).  batched: one layer-major pass over all P positions
        (orc_prefill, equal bit for bit to P steps and much faster for large
        models); else P single-position steps."""
        prompt = np.ascontiguousarray(prompt, np.int32)
        B, P = prompt.shape
        if not batched:
            nxt = logits = None
            for t in range(P):
                nxt, logits = self.step(prompt[:, t])
            return nxt, logits
        assert B == self.batch
        logits = np.empty((B, self.cfg.vocab), np.float32)
        nxt = np.empty(B, np.int32)
        pos = np.ascontiguousarray(self.pos, np.int32)
        rc = lib().orc_prefill(ctypes.byref(self._cfg), ctypes.byref(self._w), ctypes.byref(self._kc), B, P,
                               _ptr(pos), _ptr(prompt), _ptr(logits), _ptr(nxt))
        if rc != 0:
            raise RuntimeError(f"orc_prefill failed with code {rc}")
        self.pos += P
        return nxt, logits

    def set_context(self, ctx: int, fill) -> None:
        """Fill positions < ctx of every sequence via fill(k_cache, v_cache) and set positions to ctx."""
        fill(self.k_cache, self.v_cache)
        self.pos[:] = ctx

    def ffn(self, layer: int, h: np.ndarray) -> np.ndarray:
        """h [B, d] float32 -> h + FFN_layer(RMSNorm(h)) (copy)."""
        h = np.array(h, np.float32, copy=True, order="C")
        B = h.shape[0]
        rc = lib().orc_ffn(ctypes.byref(self._cfg), ctypes.byref(self._layers[layer]), B, _ptr(h))
        if rc != 0:
            raise RuntimeError(f"orc_ffn failed with code {rc}")
        return h

    def sequence(self, tokens: Sequence[int]) -> np.ndarray:
        tok = np.ascontiguousarray(tokens, np.int32)
        logits = np.empty((tok.size, self.cfg.vocab), np.float32)
        rc = lib().orc_sequence(ctypes.byref(self._cfg), ctypes.byref(self._w), _ptr(tok), tok.size, _ptr(logits))
        if rc != 0:
            raise RuntimeError(f"orc_sequence failed with code {rc}")
        return logits
