"""Measured error of the device math the decode step uses (expf, sqrtf, the fp32
divide and their compositions), in units in the last place of the exact result
computed in double.  The kernel's RoPE table is computed on the host in double;
the device functions are HIP's own, compiled with the kernel's flags."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _ulp_err(got, exact):
    """|got - exact| in fp32 ulps of the exact value."""
    ex32 = exact.astype(np.float32)
    ulp = np.abs(np.spacing(ex32)).astype(np.float64)
    return np.abs(got.astype(np.float64) - exact) / ulp


CASES = [
    # (fn, name, input range as (lo, hi) or a callable, exact in double, bound in ulps)
    (0, "expf (softmax, arguments <= 0)", (-87.0, 0.0), np.exp, 2.0),
    (0, "expf (silu, |z| <= 20)", (-20.0, 20.0), np.exp, 2.0),
    (1, "sqrtf", (1e-6, 1e4), np.sqrt, 1.0),
    (2, "1 / x", (1e-3, 1e6), lambda x: 1.0 / x, 1.0),
    (3, "1 / sqrtf(x) (RMSNorm scale)", (1e-6, 1e4), lambda x: 1.0 / np.sqrt(x), 2.0),
    (4, "silu z / (1 + expf(-z))", (-20.0, 20.0), lambda z: z / (1.0 + np.exp(-z)), 4.0),
]


@pytest.mark.parametrize("fn,name,rng,exact,bound", CASES, ids=[c[1] for c in CASES])
def test_device_math_ulp_error(fn, name, rng, exact, bound):
    import torch

    import persistent_megakernel_02_amd.mk as mk

    g = np.random.default_rng(fn * 7 + 1)
    lo, hi = rng
    if lo > 0:
        x = np.exp(g.uniform(np.log(lo), np.log(hi), 1 << 20)).astype(np.float32)
    else:
        x = g.uniform(lo, hi, 1 << 20).astype(np.float32)
    y = mk.device_math(fn, torch.from_numpy(x).cuda()).cpu().numpy()
    e = _ulp_err(y, exact(x.astype(np.float64)))
    if fn == 4:  # silu near its zero crossing: measure relative to |z| instead
        keep = np.abs(x) > 1e-3
        e = e[keep]
    worst = float(e.max())
    print(f"{name}: max error {worst:.3f} ulp, mean {float(e.mean()):.3f} ulp over {e.size} inputs", flush=True)
    assert worst <= bound, f"{name}: {worst:.3f} ulp"
