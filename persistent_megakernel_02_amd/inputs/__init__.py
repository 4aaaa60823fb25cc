"""Seeded synthetic inputs shared by the HIP path and the CPU oracle's tests.

Nothing here computes any part of the decode step.  The module defines the
model shapes used for testing and benchmarking, and produces bf16 weights,
prompt tokens and pre-filled KV contexts from a counter-based SplitMix64
stream (see ``gen.c``), so that both sides of every parity check read the very
same bytes.

Input recipe (all seeded, default seed 0):
  * every weight matrix: N(0, 0.02) rounded to bf16;
  * every RMSNorm gain: 1 + 0.02 * N(0, 1) rounded to bf16 (unit scale, so a
    missing gain is visible in the logits);
  * prompt tokens: uniform over [0, vocab);
  * synthetic KV context: N(0, 1) bf16 for every position below the context
    length, in every layer, sequence and KV head (K taken as already rotated).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmkgen.so")

# stream tags (one independent stream per tensor, layer and expert)
TAG_EMBED, TAG_LM_HEAD, TAG_FINAL_NORM = 1, 2, 3
TAG_ATTN_NORM, TAG_WQ, TAG_WK, TAG_WV, TAG_WO, TAG_MLP_NORM = 10, 11, 12, 13, 14, 15
TAG_W_GATE, TAG_W_UP, TAG_W_DOWN, TAG_ROUTER = 16, 17, 18, 19
TAG_E_GATE, TAG_E_UP, TAG_E_DOWN = 20, 21, 22
TAG_S_GATE, TAG_S_UP, TAG_S_DOWN = 23, 24, 25
TAG_PROMPT, TAG_KV_K, TAG_KV_V, TAG_START = 40, 41, 42, 43


def build(verbose: bool = False) -> str:
    """Compile gen.c into libmkgen.so next to this file (gcc, -O2)."""
    import subprocess

    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gen_key.restype = ctypes.c_uint64
        lib.gen_key.argtypes = [ctypes.c_uint64] * 4
        lib.gen_u64.restype = ctypes.c_uint64
        lib.gen_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.gen_normal_at.restype = ctypes.c_double
        lib.gen_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.gen_normal_bf16.restype = None
        lib.gen_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        lib.gen_uniform_int.restype = None
        lib.gen_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(int(os.environ.get("OMP_NUM_THREADS", n)), n, 64))


def key(seed: int, tag: int, a: int = 0, b: int = 0) -> int:
    return int(_load().gen_key(seed & (2**64 - 1), tag, a & (2**64 - 1), b & (2**64 - 1)))


def normal_bf16(k: int, shape, mean: float = 0.0, std: float = 1.0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of mean + std * N(0,1) from stream ``k``."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        _load().gen_normal_bf16(k, n, mean, std, out.ctypes.data, _threads())
    return out


def uniform_int(k: int, n: int, m: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _load().gen_uniform_int(k, n, m, out.ctypes.data)
    return out


def u64(k: int, i: int) -> int:
    return int(_load().gen_u64(k, i))


def normal_at(k: int, i: int) -> float:
    return float(_load().gen_normal_at(k, i))


# ----------------------------------------------------------------------------------------------
# model shapes
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    tied: bool = True
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    n_experts: int = 0
    top_k: int = 0
    n_shared: int = 0
    expert_ffn: int = 0

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def weight_bytes(self) -> int:
        """bf16 bytes of every matrix and gain the decode step reads once (dense models)."""
        d, hd = self.hidden, self.head_dim
        per_layer = (self.n_q_heads + 2 * self.n_kv_heads) * hd * d + d * self.n_q_heads * hd + 2 * d
        if self.is_moe:
            per_layer += self.n_experts * d + (self.n_shared + self.n_experts) * 3 * self.expert_ffn * d
        else:
            per_layer += 3 * self.ffn * d
        return 2 * (self.n_layers * per_layer + self.vocab * d + d)


TINY = ModelConfig("tiny", 2, 256, 4, 2, 64, 768, 4096, tied=True, rope_theta=10000.0)
LLAMA_1B = ModelConfig("llama-3.2-1b-shape", 16, 2048, 32, 8, 64, 8192, 128256, tied=True, rope_theta=500000.0)
LLAMA_8B = ModelConfig("llama-3-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, tied=False, rope_theta=500000.0)
MOE = ModelConfig("synthetic-moe", 8, 4096, 32, 8, 128, 0, 65536, tied=False, rope_theta=500000.0,
                  n_experts=64, top_k=6, n_shared=1, expert_ffn=1536)

CONFIGS = {c.name: c for c in (TINY, LLAMA_1B, LLAMA_8B, MOE)}


@dataclass
class Weights:
    """bf16 bit patterns (uint16 numpy arrays), row-major [out, in] matrices."""
    cfg: ModelConfig
    embed: np.ndarray
    lm_head: Optional[np.ndarray]  # None when tied to the embedding
    final_norm: np.ndarray
    layers: List[Dict[str, object]] = field(default_factory=list)

    @property
    def head(self) -> np.ndarray:
        return self.embed if self.lm_head is None else self.lm_head


def make_weights(cfg: ModelConfig, seed: int = 0, weight_std: float = 0.02, gain_std: float = 0.02) -> Weights:
    d, hd, V = cfg.hidden, cfg.head_dim, cfg.vocab
    embed = normal_bf16(key(seed, TAG_EMBED), (V, d), 0.0, weight_std)
    lm_head = None if cfg.tied else normal_bf16(key(seed, TAG_LM_HEAD), (V, d), 0.0, weight_std)
    final_norm = normal_bf16(key(seed, TAG_FINAL_NORM), (d,), 1.0, gain_std)
    layers = []
    for l in range(cfg.n_layers):
        L: Dict[str, object] = {
            "attn_norm": normal_bf16(key(seed, TAG_ATTN_NORM, l), (d,), 1.0, gain_std),
            "wq": normal_bf16(key(seed, TAG_WQ, l), (cfg.n_q_heads * hd, d), 0.0, weight_std),
            "wk": normal_bf16(key(seed, TAG_WK, l), (cfg.n_kv_heads * hd, d), 0.0, weight_std),
            "wv": normal_bf16(key(seed, TAG_WV, l), (cfg.n_kv_heads * hd, d), 0.0, weight_std),
            "wo": normal_bf16(key(seed, TAG_WO, l), (d, cfg.n_q_heads * hd), 0.0, weight_std),
            "mlp_norm": normal_bf16(key(seed, TAG_MLP_NORM, l), (d,), 1.0, gain_std),
        }
        if cfg.is_moe:
            E, Fe = cfg.n_experts, cfg.expert_ffn
            L["router"] = normal_bf16(key(seed, TAG_ROUTER, l), (E, d), 0.0, weight_std)
            L["e_gate"] = [normal_bf16(key(seed, TAG_E_GATE, l, e), (Fe, d), 0.0, weight_std) for e in range(E)]
            L["e_up"] = [normal_bf16(key(seed, TAG_E_UP, l, e), (Fe, d), 0.0, weight_std) for e in range(E)]
            L["e_down"] = [normal_bf16(key(seed, TAG_E_DOWN, l, e), (d, Fe), 0.0, weight_std) for e in range(E)]
            L["s_gate"] = normal_bf16(key(seed, TAG_S_GATE, l), (Fe, d), 0.0, weight_std)
            L["s_up"] = normal_bf16(key(seed, TAG_S_UP, l), (Fe, d), 0.0, weight_std)
            L["s_down"] = normal_bf16(key(seed, TAG_S_DOWN, l), (d, Fe), 0.0, weight_std)
        else:
            L["w_gate"] = normal_bf16(key(seed, TAG_W_GATE, l), (cfg.ffn, d), 0.0, weight_std)
            L["w_up"] = normal_bf16(key(seed, TAG_W_UP, l), (cfg.ffn, d), 0.0, weight_std)
            L["w_down"] = normal_bf16(key(seed, TAG_W_DOWN, l), (d, cfg.ffn), 0.0, weight_std)
        layers.append(L)
    return Weights(cfg, embed, lm_head, final_norm, layers)


def make_prompt(cfg: ModelConfig, batch: int, length: int, seed: int = 0) -> np.ndarray:
    """int32 [batch, length], independent uniform tokens per sequence."""
    out = np.empty((batch, length), dtype=np.int32)
    for b in range(batch):
        out[b] = uniform_int(key(seed, TAG_PROMPT, b), length, cfg.vocab)
    return out


def make_start_tokens(cfg: ModelConfig, batch: int, seed: int = 0) -> np.ndarray:
    """int32 [batch]: the first input token after a synthetic context."""
    return uniform_int(key(seed, TAG_START), batch, cfg.vocab)


def kv_context_block(cfg: ModelConfig, which: str, layer: int, b: int, g: int, ctx: int, seed: int = 0) -> np.ndarray:
    """bf16 [ctx, head_dim] values of K (which='k') or V for positions 0..ctx-1 of (layer, b, g)."""
    tag = TAG_KV_K if which == "k" else TAG_KV_V
    return normal_bf16(key(seed, tag, layer, b * cfg.n_kv_heads + g), (ctx, cfg.head_dim), 0.0, 1.0)


def fill_kv_context(cfg: ModelConfig, k_cache: np.ndarray, v_cache: np.ndarray, batch: int, ctx: int,
                    seed: int = 0) -> None:
    """Fill caches laid out [L][B][Hkv][S][hd] (uint16) at positions < ctx."""
    for l in range(cfg.n_layers):
        for b in range(batch):
            for g in range(cfg.n_kv_heads):
                k_cache[l, b, g, :ctx] = kv_context_block(cfg, "k", l, b, g, ctx, seed)
                v_cache[l, b, g, :ctx] = kv_context_block(cfg, "v", l, b, g, ctx, seed)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for reporting only)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


__all__ = [
    "ModelConfig", "Weights", "TINY", "LLAMA_1B", "LLAMA_8B", "MOE", "CONFIGS", "make_weights", "make_prompt",
    "make_start_tokens", "kv_context_block", "fill_kv_context", "normal_bf16", "uniform_int", "key", "u64",
    "normal_at", "build", "bf16_bits_to_f32", "replace",
]
