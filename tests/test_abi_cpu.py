"""Host-only checks of the C ABI: the library loads, exports every function the
headers declare, validates shapes, and builds schedules that verify."""
import ctypes
import os
import re

import pytest

import persistent_megakernel_02_amd.inputs as I
import persistent_megakernel_02_amd.mk as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("mk.h", "mk_bench.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[\w\s\*]+?\b(mk_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    lib = mk.lib()
    decl = declared_functions()
    assert len(decl) >= 15
    missing = [n for n in sorted(decl) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(mk.EXPORTS) == decl


def test_status_strings():
    for s in range(8):
        assert mk.lib().mk_status_string(s)
    assert b"unknown" in mk.lib().mk_status_string(99)


def rt(b=1, s=161, mode=mk.MK_MODE_MEGAKERNEL, cus=256, splits=0):
    return mk.runtime_config(b, s, mode, cus, 0, splits)


def test_query_sizes_kv_bytes_match_layout():
    c = mk.model_config(I.LLAMA_1B)
    st, ws, kv = mk.mk_query_sizes(c, rt(1, 160))
    assert st == mk.MK_OK
    assert kv == 2 * 16 * 1 * 8 * 160 * 64 * 2
    assert 0 < ws < 64 << 20


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, mk.MK_E_UNSUPPORTED),
    ("n_kv_heads", 5, mk.MK_E_UNSUPPORTED),
    ("hidden", 300, mk.MK_E_UNSUPPORTED),
    ("n_layers", 0, mk.MK_E_INVALID),
    ("n_experts", 64, mk.MK_E_INVALID),  # an MoE model needs top_k and expert_ffn
])
def test_query_sizes_rejects_bad_shapes(field, value, status):
    c = mk.model_config(I.LLAMA_1B)
    setattr(c, field, value)
    st, _, _ = mk.mk_query_sizes(c, rt())
    assert st == status


def test_runtime_validation():
    c = mk.model_config(I.TINY)
    assert mk.mk_query_sizes(c, rt(b=0))[0] == mk.MK_E_UNSUPPORTED
    assert mk.mk_query_sizes(c, rt(b=9))[0] == mk.MK_E_UNSUPPORTED
    assert mk.mk_query_sizes(c, rt(s=0))[0] == mk.MK_E_INVALID
    bad = rt()
    bad.mode = 7
    assert mk.mk_query_sizes(c, bad)[0] == mk.MK_E_INVALID
    bad = rt()
    bad.trace = 2
    assert mk.mk_query_sizes(c, bad)[0] == mk.MK_E_INVALID
    ok = rt()
    ok.trace = 1
    st, ws_tr, _ = mk.mk_query_sizes(c, ok)
    assert st == mk.MK_OK and ws_tr > mk.mk_query_sizes(c, rt())[1]


LDS_BYTES, LDS_STATIC, CHUNK, MIN_RING = 160 * 1024, 1024, 1024, 72


def staged_bytes(cfg, batch):
    """fp32 activations one GEMV instruction stages in LDS: x rows of the widest
    input (d, Hq*hd or ffn) plus up to 64 residual rows for O / DOWN."""
    return 4 * batch * max(cfg.hidden, cfg.n_q_heads * cfg.head_dim + 64, cfg.ffn + 64)


@pytest.mark.parametrize("cfg", [I.TINY, I.LLAMA_1B, I.LLAMA_8B], ids=lambda c: c.name)
@pytest.mark.parametrize("cus", [256, 304, 80, 7, 1])
@pytest.mark.parametrize("batch", [1, 2])
def test_schedule_verifies(cfg, cus, batch):
    st, info = mk.mk_plan_inspect(mk.model_config(cfg), rt(batch, 200), cus)
    if LDS_BYTES - LDS_STATIC - staged_bytes(cfg, batch) < MIN_RING * CHUNK:  # no room left for the weight ring
        assert st == mk.MK_E_UNSUPPORTED
        return
    assert st == mk.MK_OK
    assert info["verify"] == 0
    assert info["phases"] == 5 * cfg.n_layers + 1
    assert info["weight_bytes"] == cfg.weight_bytes()
    assert info["x_bytes"] >= staged_bytes(cfg, batch)
    assert info["ring_chunks"] == (LDS_BYTES - LDS_STATIC - info["x_bytes"]) // CHUNK >= MIN_RING
    items = batch * cfg.n_kv_heads * info["attn_splits"] * info["attn_hsplit"]
    G = cfg.n_q_heads // cfg.n_kv_heads
    # one item per q head when a single position split leaves CUs idle
    assert info["attn_hsplit"] == (G if info["attn_splits"] == 1 and batch * cfg.n_kv_heads * G <= cus else 1)
    od = -(-(-(-cfg.hidden // cus)) // 64)  # O / DOWN instructions per CU (<= 64 rows each)
    assert info["instructions"] <= cfg.n_layers * (2 * cus + items + 2 * od * cus) + cus
    assert info["head_instructions"] == min(cus, cfg.vocab)


def test_schedule_one_tile_per_cu_per_matrix():
    st, info = mk.mk_plan_inspect(mk.model_config(I.LLAMA_1B), rt(1, 161), 256)
    assert st == mk.MK_OK
    # 16 layers x (QKV, O, gate/up, down) one tile on each CU, attention items (one
    # per q head: 32), LM head
    assert info["attn_splits"] == 1 and info["attn_hsplit"] == 4
    items = 8 * info["attn_splits"] * info["attn_hsplit"]
    assert info["instructions"] == 16 * (4 * 256 + items) + 256
    assert info["max_per_cu"] == 16 * 5 + 1


def test_schedule_balances_bytes():
    """Rows per CU differ by at most one in every matrix: no tail wave of
    stragglers (512 blocks on 148 SMs leave 80 SMs idle in the last wave)."""
    import math
    blocks, sms = 512, 148
    waves = math.ceil(blocks / sms)
    assert waves == 4 and blocks - (waves - 1) * sms == 68 and sms - 68 == 80
    for R in (3072, 2048, 8192, 128256):
        per = [(R * (c + 1)) // 256 - (R * c) // 256 for c in range(256)]
        assert max(per) - min(per) <= 1 and sum(per) == R


def test_gemv_kind_validation():
    c = mk.model_config(I.TINY)
    assert mk.mk_query_sizes(c, mk.runtime_config(1, 64, gemv_kind=3))[0] == mk.MK_E_UNSUPPORTED
    assert mk.mk_query_sizes(c, mk.runtime_config(1, 64, gemv_kind=-1))[0] == mk.MK_E_UNSUPPORTED
    # the matrix-core GEMV runs in the persistent mode only
    graph_mfma = mk.runtime_config(1, 64, mk.MK_MODE_GRAPH, gemv_kind=mk.MK_GEMV_MFMA)
    assert mk.mk_query_sizes(c, graph_mfma)[0] == mk.MK_E_UNSUPPORTED
    for b in (1, 2, 4, 8):
        for kind in (mk.MK_GEMV_AUTO, mk.MK_GEMV_VALU, mk.MK_GEMV_MFMA):
            assert mk.mk_query_sizes(c, mk.runtime_config(b, 64, gemv_kind=kind))[0] == mk.MK_OK


def parts_bytes(batch, k):
    """bf16 parts of `batch` fp32 rows of k values: 3 parts while 3 * batch
    columns fit one 16-column matrix-core tile, else 2; at least parts * batch
    bf16 per element (the area pads its rows to an odd number of 16-byte slots)."""
    return 2 * (3 if 3 * batch <= 16 else 2) * batch * k


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_mfma_activation_area(batch):
    """The matrix-core GEMV stages bf16 parts of the activations (plus cross-wave
    partial tiles); the area still leaves at least the minimum weight ring."""
    cfg = I.LLAMA_1B
    st, info = mk.mk_plan_inspect(mk.model_config(cfg), mk.runtime_config(batch, 200, gemv_kind=mk.MK_GEMV_MFMA),
                                  256)
    assert st == mk.MK_OK and info["verify"] == 0
    assert info["x_bytes"] >= max(parts_bytes(batch, cfg.hidden), parts_bytes(batch, cfg.n_q_heads * cfg.head_dim))
    assert info["ring_chunks"] == (LDS_BYTES - LDS_STATIC - info["x_bytes"]) // CHUNK >= MIN_RING


def test_gemv_kind_in_effect():
    """Automatic selection takes VALU at every batch (the faster kind on the 1B
    shape at batch 1, 4 and 8 by measurement); MFMA runs where it is asked for and
    its parts area fits; it is refused where three bf16 parts of the hidden state
    would leave too small a ring (hidden 4096 at batch 4: 96 KB of parts against
    64 KB of fp32 for VALU)."""
    c = mk.model_config(I.LLAMA_1B)
    for b in (1, 2, 4, 8):
        assert mk.mk_plan_inspect(c, mk.runtime_config(b, 200), 256)[1]["gemv_kind"] == mk.MK_GEMV_VALU
        mf = mk.mk_plan_inspect(c, mk.runtime_config(b, 200, gemv_kind=mk.MK_GEMV_MFMA), 256)[1]
        assert mf["gemv_kind"] == mk.MK_GEMV_MFMA
    graph = mk.runtime_config(8, 200, mk.MK_MODE_GRAPH)
    assert mk.mk_plan_inspect(c, graph, 256)[1]["gemv_kind"] == mk.MK_GEMV_VALU
    wide = mk.model_config(I.replace(I.LLAMA_1B, hidden=4096))
    assert mk.mk_query_sizes(wide, mk.runtime_config(4, 200, gemv_kind=mk.MK_GEMV_VALU))[0] == mk.MK_OK
    assert mk.mk_query_sizes(wide, mk.runtime_config(4, 200, gemv_kind=mk.MK_GEMV_MFMA))[0] == mk.MK_E_UNSUPPORTED


SMALL_MOE = I.replace(I.TINY, name="small-moe", hidden=512, n_q_heads=8, n_kv_heads=4, ffn=0, n_experts=8,
                      top_k=2, n_shared=1, expert_ffn=512, tied=False)


def test_moe_validation():
    c = mk.model_config(I.MOE)
    assert mk.mk_query_sizes(c, rt(4, 4200))[0] == mk.MK_OK
    # the persistent mode and the VALU GEMV only
    assert mk.mk_query_sizes(c, rt(4, 4200, mode=mk.MK_MODE_GRAPH))[0] == mk.MK_E_UNSUPPORTED
    assert mk.mk_query_sizes(c, mk.runtime_config(4, 4200, gemv_kind=mk.MK_GEMV_MFMA))[0] == mk.MK_E_UNSUPPORTED
    # batch 8: the 8 x 4096 fp32 inputs (128 KB) go in two column slices
    assert mk.mk_query_sizes(c, rt(8, 4200))[0] == mk.MK_OK
    assert mk.mk_query_sizes(c, rt(8, 4200, mode=mk.MK_MODE_GRAPH))[0] == mk.MK_E_UNSUPPORTED
    for field, value, status in (("n_experts", 65, mk.MK_E_INVALID), ("top_k", 9, mk.MK_E_UNSUPPORTED),
                                 ("top_k", 0, mk.MK_E_INVALID), ("n_shared_experts", 2, mk.MK_E_UNSUPPORTED),
                                 ("expert_ffn", 1000, mk.MK_E_UNSUPPORTED)):
        bad = mk.model_config(I.MOE)
        setattr(bad, field, value)
        if field == "n_experts":  # 65 experts with top_k 6 passes the first check, not the 64-expert mask
            assert mk.mk_query_sizes(bad, rt(4, 4200))[0] == mk.MK_E_UNSUPPORTED
        else:
            assert mk.mk_query_sizes(bad, rt(4, 4200))[0] == status, field


@pytest.mark.parametrize("cfg,batch", [(I.MOE, 4), (I.MOE, 1), (SMALL_MOE, 4), (I.MOE, 8)],
                         ids=["moe-b4", "moe-b1", "small-b4", "moe-b8"])
@pytest.mark.parametrize("cus", [256, 7])
def test_moe_schedule_verifies(cfg, batch, cus):
    st, info = mk.mk_plan_inspect(mk.model_config(cfg), rt(batch, 300), cus)
    assert st == mk.MK_OK
    assert info["verify"] == 0
    # per layer: QKV, ATTN, O, ROUTE, EGU, EPART (one expert-down share per CU),
    # EDOWN (the weighted combine); then the LM head
    assert info["phases"] == 7 * cfg.n_layers + 1
    assert info["weight_bytes"] == cfg.weight_bytes()
    assert info["ring_chunks"] >= MIN_RING
    assert info["gemv_kind"] == mk.MK_GEMV_VALU


def test_plan_inspect_rejects_bad_cu_count():
    assert mk.mk_plan_inspect(mk.model_config(I.TINY), rt(), 0)[0] == mk.MK_E_INVALID
    assert mk.mk_plan_inspect(mk.model_config(I.TINY), rt(), 5000)[0] == mk.MK_E_INVALID


def _expected_span(cfg, batch, mfma):
    """Ring chunks one compute wave holds at most, written out from the kernel's
    batch rules: rows of <= 2 KB go four to a batch, <= 4 KB two, longer one (two
    rows from batch 4 on); a (gate, up) pair shares a batch; rows of >= 8 KB at
    batch 1-2 stream in 8 KB segments; +1 chunk for a batch starting inside a
    chunk; a matrix-core unit is 8 chunks; an attention block is its RoPE chunk
    and 32 groups of a K and a V chunk."""
    def batch_span(rb, pairs):
        if batch <= 2 and rb >= 8192:
            return 8 + 1
        r = 2 if batch >= 4 else (4 if rb <= 2048 else 2 if rb <= 4096 else 1)
        if pairs:
            r = max(r, 2)
        return -(-(r * rb) // 1024) + 1
    span = 1 + 2 * 32
    if mfma:
        return max(span, 8)
    d2 = 2 * cfg.hidden
    xs = 1  # MoE inputs of hidden width beyond 64 KB at this batch go in column slices
    while cfg.n_experts and batch * (cfg.hidden // xs) * 4 > 64 * 1024:
        xs *= 2
    spans = [batch_span(d2 // xs, False), batch_span(d2, False),
             batch_span(2 * cfg.n_q_heads * cfg.head_dim // xs, False), batch_span(d2 // xs, True)]
    if cfg.n_experts:
        spans.append(batch_span(2 * cfg.expert_ffn, False))
    else:
        ns = 1
        while batch * (cfg.ffn // ns) * 4 > 64 * 1024 and ns < 64:
            ns *= 2
        spans.append(batch_span(2 * (cfg.ffn // ns), False))
    return max([span] + spans)


@pytest.mark.parametrize("cfg", [I.TINY, I.LLAMA_1B, I.LLAMA_8B, I.MOE,
                                 I.replace(I.TINY, name="wide-ffn", ffn=4096)], ids=lambda c: c.name)
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
@pytest.mark.parametrize("cus", [1, 7, 37, 80, 256, 304])
@pytest.mark.parametrize("kind", [mk.MK_GEMV_VALU, mk.MK_GEMV_MFMA], ids=["valu", "mfma"])
def test_ring_span_fits_every_supported_plan(cfg, batch, cus, kind):
    """Deadlock freedom of the weight ring: the loader may write a chunk only
    within ring_chunks of the smallest compute-wave mark, and a wave waits for
    its whole row batch (or segment, matrix-core unit, attention block) with its
    mark at the batch start, so that stretch must fit the ring.  Every plan that
    the library accepts satisfies it, and the library reports the stretch."""
    st, info = mk.mk_plan_inspect(mk.model_config(cfg), mk.runtime_config(batch, 200, gemv_kind=kind), cus)
    if st != mk.MK_OK:
        assert st == mk.MK_E_UNSUPPORTED
        return
    assert info["max_wave_span"] == _expected_span(cfg, batch, info["gemv_kind"] == mk.MK_GEMV_MFMA)
    assert info["max_wave_span"] <= info["ring_chunks"]


def test_dense_persistent_kernels_use_no_scratch():
    """The dense VALU persistent kernel (the headline path) keeps its values in
    registers: a spill to scratch memory puts global-memory traffic (and vmcnt
    waits) inside the inner loops, and one (56 dwords at batch 1) cost 14 % of the
    1B batch-1 step.  The budget is 256 VGPRs per wave (two waves per SIMD); the
    build records what the compiler allocated.  Batch 1 and 2 must not spill at
    all; batch 4 and 8 may spill at most eight dwords (at batch 4 set-up values
    are reloaded in a loop preheader and in the attention split merge).
    The matrix-core and MoE kinds are listed with their scratch bytes (known
    spills at batch >= 2)."""
    import json

    from persistent_megakernel_02_amd import _build

    if not os.path.exists(_build.RESOURCES):
        pytest.skip("library built without the resource report")
    res = json.load(open(_build.RESOURCES))
    mega = {k: v for k, v in res.items() if "mk_megakernel" in k}
    # 3 kinds x 4 batches x 2 head sizes, and the multi-position kernels (dense and MoE x 2 head sizes)
    assert len(mega) == 28, sorted(mega)
    assert all(v["vgpr"] <= 256 and v["occupancy"] >= 2 for v in mega.values())
    dense = {k: v for k, v in mega.items() if k.endswith("Lb0ELb0ELb0EEEvNS_6ParamsENS_8StepArgsE")}
    assert len(dense) == 8
    small = {k: v for k, v in dense.items() if k.startswith(("_ZN2mk13mk_megakernelILi1E", "_ZN2mk13mk_megakernelILi2E"))}
    assert len(small) == 4 and all(v["scratch"] == 0 for v in small.values()), small
    assert all(v["scratch"] <= 32 for v in dense.values()), dense
    print({k: v["scratch"] for k, v in mega.items() if v["scratch"]})


def test_static_create_refuses_on_the_host():
    """mk_create_static decides what it cannot do before it touches the device:
    the one-kernel-per-op mode, and a workspace larger than the static array (a
    long RoPE table), are refused with no HIP call."""
    L = mk.lib()
    cfg = mk.model_config(I.LLAMA_1B)
    w = mk.mk_weights()
    h = ctypes.c_void_p()
    graph = mk.runtime_config(1, 161, mode=mk.MK_MODE_GRAPH)
    assert L.mk_create_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(graph), None, 0, None,
                              ctypes.byref(h)) == mk.MK_E_UNSUPPORTED
    big = mk.runtime_config(1, 1 << 20)  # RoPE table alone: 2^20 positions x 32 x 8 bytes = 256 MB
    assert L.mk_create_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(big), None, 0, None,
                              ctypes.byref(h)) == mk.MK_E_CAPACITY
    assert h.value is None


def test_batch1_loader_paths_selection():
    """The three batch-1 persistent-kernel paths: the (gate, up) rows by the loader
    waves on both dense shapes (hidden 2048 / head_dim 64 and 4096 / 128), the down
    projection by column quarters where F = 8192 (the 1B shape), the O rows by the
    loader waves on the hidden-4096 shape only; none at batch 4, with MFMA, for the
    mixture of experts or off those shapes, and only the quarters in the graph
    mode."""
    keys = ("gateup_by_loaders", "down_quarters", "o_by_loaders")

    def sel(cfg, r):
        st, info = mk.mk_plan_inspect(mk.model_config(cfg), r, 256)
        assert st == mk.MK_OK
        return tuple(info[k] for k in keys)

    assert sel(I.LLAMA_1B, rt(1, 200)) == (1, 1, 0)
    assert sel(I.LLAMA_8B, rt(1, 200)) == (1, 0, 1)
    assert sel(I.LLAMA_1B, rt(4, 200)) == (0, 0, 0)
    assert sel(I.LLAMA_8B, rt(1, 200, mode=mk.MK_MODE_GRAPH)) == (0, 0, 0)
    assert sel(I.LLAMA_1B, mk.runtime_config(1, 200, gemv_kind=mk.MK_GEMV_MFMA)) == (0, 0, 0)
    # the graph mode takes the same quarter order for its DOWN kernel, not the loader rows
    assert sel(I.LLAMA_1B, rt(1, 200, mode=mk.MK_MODE_GRAPH)) == (0, 1, 0)
    assert sel(I.MOE, rt(4, 4200)) == (0, 0, 0)
    assert sel(I.TINY, rt(1, 200)) == (0, 0, 0)
