"""Per-element error bars shared by the GPU parity tests.

The stated tolerance is max |gpu - oracle| <= 1e-5 for fp32 outputs and
<= 2e-3 for fp16/bf16 outputs (fp32 accumulation).  A 16-bit output has to be
rounded to its storage type, and at |out| > 0.5 a bf16 half-ulp alone exceeds
2e-3, so for 16-bit outputs the bar per element is max(2e-3, one unit in the
last place of the storage type at |oracle|).  At the workload shapes |out|
stays well below 0.5, where 2e-3 is the binding bar.
"""
import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
MANT_BITS = {"f16": 10, "bf16": 7}


def bound(ref, dtype):
    tol = TOL[dtype]
    if dtype == "f32":
        return np.full(np.shape(ref), tol)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -30)))
    return np.maximum(tol, 2.0 ** (e - MANT_BITS[dtype]))


def assert_close(got, ref, dtype, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output at {np.argwhere(~np.isfinite(got))[:4]}"
    if not got.size:
        return
    diff = np.abs(got - ref)
    bad = diff > bound(ref, dtype)
    assert not bad.any(), (f"{what}: {bad.sum()} elements over the bar; max abs err "
                           f"{diff.max():.3e}, worst at {np.argwhere(bad)[:4].tolist()}")
