"""Runtime behaviour on the GPU through the C ABI: the KV capacity check, the
device watchdog (forced from the host: mk_debug_inject makes one step's layer-0
attention wait for a tag that no instruction writes, under a 1 ms watchdog, so
every workgroup gives up and exits), NaN logits, and recovery with mk_reset.
No test here makes a kernel fault or wait without bound."""
import numpy as np
import pytest

import oracle as O
import persistent_megakernel_02_amd.inputs as I

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dec(cfg, w, B, S, **kw):
    _torch()
    import persistent_megakernel_02_amd.mk as mk

    return mk.Decoder(cfg, w, max_batch=B, max_seq=S, **kw)


def test_capacity_exceeded_is_reported():
    import persistent_megakernel_02_amd.mk as mk

    torch = _torch()
    cfg = I.TINY
    w = I.make_weights(cfg, seed=0)
    prompt = torch.from_numpy(I.make_prompt(cfg, 1, 4, seed=0)).cuda()
    d = _dec(cfg, w, 1, 4)
    d.prefill(prompt)
    assert d.context_len() == [4]
    with pytest.raises(mk.MKError) as e:
        d.decode_step(prompt[:, 0].contiguous())
    assert e.value.status == mk.MK_E_CAPACITY
    assert d.context_len() == [4]
    with pytest.raises(mk.MKError) as e:
        d.prefill(prompt[:, :1].contiguous())
    assert e.value.status == mk.MK_E_CAPACITY
    d.close()


@pytest.mark.parametrize("mode", [0, 1], ids=["megakernel", "graph"])
def test_watchdog_then_reset_recovers(mode):
    """A step whose inputs never arrive ends with MK_E_DEVICE_TIMEOUT (every
    workgroup leaves on its own watchdog); the handle answers MK_E_STATE until
    mk_reset; after the reset the decoder continues from the last good position
    and matches a decoder that never failed."""
    import persistent_megakernel_02_amd.mk as mk

    torch = _torch()
    cfg = I.TINY
    w = I.make_weights(cfg, seed=3)
    prompt = torch.from_numpy(I.make_prompt(cfg, 1, 6, seed=3)).cuda()
    ref = _dec(cfg, w, 1, 16, mode=mode)
    ref.prefill(prompt)
    ref_tok, ref_log = [], []
    tok = ref.tok.clone()
    for _ in range(3):
        t, l = ref.decode_step(tok)
        tok = t.clone()
        ref_tok.append(t.cpu().numpy().copy())
        ref_log.append(l.cpu().numpy().copy())
    ref.close()

    d = _dec(cfg, w, 1, 16, mode=mode)
    d.prefill(prompt)
    first = d.tok.clone()
    print(f"case watchdog mode={mode}", flush=True)
    d.debug_inject(1)
    d.decode_step(first.clone())  # enqueued; the failure is latched by the device
    torch.cuda.synchronize()
    with pytest.raises(mk.MKError) as e:
        d.decode_step(first.clone())
    assert e.value.status == mk.MK_E_DEVICE_TIMEOUT
    with pytest.raises(mk.MKError) as e:
        d.decode_step(first.clone())
    assert e.value.status == mk.MK_E_STATE
    d.reset()
    assert d.context_len() == [6]  # the failed step did not advance the position
    tok = first.clone()
    for t_ref, l_ref in zip(ref_tok, ref_log):
        t, l = d.decode_step(tok)
        tok = t.clone()
        assert np.array_equal(t.cpu().numpy(), t_ref)
        assert np.array_equal(l.cpu().numpy(), l_ref)
    d.close()


def test_nan_logits_are_reported():
    """A NaN final-norm gain makes every logit NaN: the step completes and the
    next call reports MK_E_DEVICE_NAN (the oracle reports the same step as an
    error: its argmax has no answer there)."""
    import persistent_megakernel_02_amd.mk as mk

    torch = _torch()
    cfg = I.TINY
    w = I.make_weights(cfg, seed=4)
    w.final_norm[:] = 0x7FC0  # bf16 quiet NaN
    orc = O.Oracle(cfg, w, 1, 8)
    with pytest.raises(RuntimeError, match="code 2"):  # ORC_E_NAN
        orc.prefill(I.make_prompt(cfg, 1, 2, seed=4))
    d = _dec(cfg, w, 1, 8)
    prompt = torch.from_numpy(I.make_prompt(cfg, 1, 2, seed=4)).cuda()
    d.prefill(prompt)
    torch.cuda.synchronize()
    assert np.isnan(d.logits.cpu().numpy()).all()
    with pytest.raises(mk.MKError) as e:
        d.decode_step(d.tok.clone())
    assert e.value.status == mk.MK_E_DEVICE_NAN
    d.close()
