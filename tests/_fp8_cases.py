"""Inputs on which the E4M3 quantiser's two plausible readings disagree.

Writing x into a pool with scale s stores the code nearest x / s.  Whether
that quotient is formed in float32 (the kernel's precision, the reading the
oracle takes) or exactly (float64 of float32 inputs) changes the code when
x / s lies within a float32 rounding of a midpoint between two E4M3 values.
``divergent_inputs`` finds such x (representable in the source type) by
brute force: for every midpoint m of adjacent E4M3 magnitudes it tries the
few source values next to m * s.  The E4M3 magnitudes come from torch's
float8_e4m3fn (a library table, independent of the oracle), and the nearest
code is found by brute force over all 127 of them (ties to the even code).
"""
import numpy as np
import torch

# magnitudes of codes 0x00 .. 0x7E (0x7F is NaN)
E4M3_MAGNITUDES = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()

# Scales with many divergent inputs for every source type (found by scanning
# a list of non-power-of-two scales).
K_SCALE = 3.3
V_SCALE = 0.9


def nearest_code(a: float) -> int:
    """Code (sign bit from ``a``) of the E4M3 value nearest ``a``, ties to the
    even code, magnitudes above 448 saturated: brute force over the table."""
    mag = min(abs(a), 448.0)
    d = np.abs(E4M3_MAGNITUDES - mag)
    idx = np.nonzero(d == d.min())[0]
    code = int(idx[0]) if len(idx) == 1 else int(idx[0] if idx[0] % 2 == 0 else idx[1])
    return code | (0x80 if a < 0 else 0)


def _neighbours(t: float, src: str):
    if src == "f32":
        b = np.int64(np.float32(t).view(np.uint32))
        return [float(np.array(b + k, dtype=np.uint32).view(np.float32)) for k in range(-3, 4)]
    if src == "f16":
        b = np.int64(np.float16(t).view(np.uint16))
        return [float(np.array(b + k, dtype=np.uint16).view(np.float16)) for k in range(-3, 4)]
    b = np.int64(np.float32(t).view(np.uint32)) >> 16            # bf16: the high half of a float32
    return [float(np.array((b + k) << 16, dtype=np.uint32).view(np.float32)) for k in range(-3, 4)]


def divergent_inputs(src: str, scale: float):
    """[(x, code with the float32 quotient, code with the exact quotient)]
    for positive x representable in ``src`` where the two codes differ."""
    s32 = np.float32(scale)
    mids = (E4M3_MAGNITUDES[:-1] + E4M3_MAGNITUDES[1:]) / 2
    out, seen = [], set()
    for m in mids:
        for x in _neighbours(float(m) * float(s32), src):
            if not np.isfinite(x) or x <= 0 or x in seen:
                continue
            seen.add(x)
            c32 = nearest_code(float(np.float32(x) / s32))
            c64 = nearest_code(x / float(s32))
            if c32 != c64:
                out.append((x, c32, c64))
    return out
