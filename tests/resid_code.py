"""The forward's byte residual of a bf16 output as include/nbattn.h defines it (o_resid), on the host in float32:
with a the fp32 value, v = bf16(a) (round to nearest even) and u = 2^(max(e, 1) - 134) the ulp of v (e = v's
biased exponent field), the code is (a - v) in units of u / 254, rounded to nearest even and clamped to
[-127, 127].  Used by the GPU finalize test (bit-exact against the kernel's encoder) and by the CPU pins of the
definition's bound."""
import numpy as np
import torch


def resid_codes(acc: torch.Tensor):
    """(codes int8, ulp float32) of float32 values ``acc``."""
    a = acc.float().numpy()
    v = acc.float().to(torch.bfloat16)
    vf = v.float().numpy()
    be = (v.view(torch.int16).numpy().astype(np.int32) >> 7) & 0xFF
    e = np.maximum(be, 1) - 134
    x = np.rint(np.ldexp(a - vf, -e).astype(np.float32) * np.float32(254))
    return np.clip(x, -127, 127).astype(np.int8), np.ldexp(np.float32(1), e).astype(np.float32)


def resid_decode(v_bf16: torch.Tensor, codes: np.ndarray) -> np.ndarray:
    """v + code * u / 254 in float64."""
    be = (v_bf16.view(torch.int16).numpy().astype(np.int32) >> 7) & 0xFF
    u = np.ldexp(1.0, np.maximum(be, 1) - 134)
    return v_bf16.double().numpy() + codes.astype(np.float64) / 254.0 * u
