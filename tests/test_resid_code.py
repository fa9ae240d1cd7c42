"""CPU pins of the byte-residual definition (include/nbattn.h, o_resid; tests/resid_code.py): every code fits a
signed byte, the decoded value lies within 1/508 of the bf16 ulp of the float32 value (the bound the header
states), and the code carries the residual's sign and size -- over random values of many magnitudes and the
special cases: zero, values bf16 holds exactly, rounding ties, binade edges where rounding carries into the next
power of two, and bf16 subnormals."""
import numpy as np
import torch

from resid_code import resid_codes, resid_decode


def _values():
    g = torch.Generator("cpu").manual_seed(3)
    mags = torch.pow(2.0, torch.randint(-120, 120, (20000,), generator=g).float())
    x = torch.randn((20000,), generator=g) * mags
    specials = [0.0, -0.0, 1.0, -2.5, 3.0e-30, 1.0e30,
                1.0 + 2.0 ** -8,                      # a tie: rounds to even
                1.0 + 3 * 2.0 ** -8,                  # a tie the other way
                2.0 - 2.0 ** -9, -(2.0 - 2.0 ** -9),  # rounds up into the next binade
                2.0 ** -126 * 1.5, 2.0 ** -130, 2.0 ** -133 * 1.4, -(2.0 ** -128) * 1.3]   # near and below normal
    return torch.cat([x, torch.tensor(specials, dtype=torch.float32)])


def test_codes_fit_a_byte_and_meet_the_bound():
    a = _values()
    codes, ulp = resid_codes(a)
    assert codes.dtype == np.int8 and codes.min() >= -127 and codes.max() <= 127
    dec = resid_decode(a.to(torch.bfloat16), codes)
    err = np.abs(dec - a.double().numpy())
    # |a - v| <= u/2 and the code rounds (a - v) / u * 254 to an integer: the error is at most u / 508, plus the
    # float32 rounding of the scaled residual (far below it)
    assert np.all(err <= ulp.astype(np.float64) * (1.0 / 508 + 2.0 ** -20))


def test_codes_carry_the_residual():
    a = _values()
    v = a.to(torch.bfloat16)
    r = a.double().numpy() - v.double().numpy()
    codes, ulp = resid_codes(a)
    nz = np.abs(r) > ulp / 508
    assert np.all(np.sign(codes[nz]) == np.sign(r[nz]))
    assert np.all(codes[r == 0] == 0)
    # the decoded value is at least as close as the bf16 value alone, and strictly closer whenever the residual
    # exceeds the code's resolution
    dec = resid_decode(v, codes)
    e_dec, e_bf = np.abs(dec - a.double().numpy()), np.abs(r)
    assert np.all(e_dec <= e_bf + 1e-300)
    assert np.all(e_dec[nz] < e_bf[nz])
