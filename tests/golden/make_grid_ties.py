"""Writes grid_ties.txt: grid-packing cases whose code is decided by a tie.

Each case is a bf16 step s and a bf16 value v with v / s exactly a half-integer
h = m + 1/2, |h| <= 7.5, for which the fp32 product v * RN(1/s) rounds to a
float on the other side of h, so that rint of that product differs from rint of
the exact quotient.  The expected code is 8 + (h rounded half to even), derived
here with exact rational arithmetic (fractions.Fraction); the fp32 product is
only used to find the cases.  Nothing here calls the oracle or the GPU library.

The rule under test (grid packing of a 16-bit table, the dev.to page "Gemma 4
on a 4 GB GPU in Plain PyTorch", section "Step 2 - Keep the Vocabulary Tables
in 4-Bit"): code = clamp(rint(v / step) + 8, 0, 15) on the exact quotient.
Run:  python tests/golden/make_grid_ties.py > tests/golden/grid_ties.txt
"""

from fractions import Fraction

import numpy as np


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern (sign, 8 exponent bits, 7 fraction bits)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def bf16_bits_of(x: Fraction):
    """The bf16 pattern holding x exactly, or None."""
    f32 = np.float32(float(x))
    if Fraction(float(f32)) != x:
        return None
    b = int(np.array([f32], dtype=np.float32).view(np.uint32)[0])
    if b & 0xFFFF:
        return None
    return b >> 16


def round_half_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    r = x - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def main():
    cases = []
    # steps in [1, 4) whose reciprocal is inexact in fp32; values h * s
    for sbits in range(0x3F80, 0x4080):
        s = bf16_value(sbits)
        if s.numerator & (s.numerator - 1) == 0 and s.denominator & (s.denominator - 1) == 0:
            continue  # a power of two: its reciprocal is exact
        r = np.float32(1.0) / np.float32(float(s))
        for twice_h in range(-15, 16, 2):
            h = Fraction(twice_h, 2)
            vbits = bf16_bits_of(h * s)
            if vbits is None:
                continue
            p = np.float32(float(bf16_value(vbits))) * r
            if int(np.rint(p)) != round_half_even(h):
                cases.append((vbits, sbits, h))
    print("# grid packing ties: v / step is exactly a half-integer h; the fp32 product")
    print("# v * RN(1/step) lands on the far side of h.  Expected code = 8 + round_half_even(h),")
    print("# derived exactly (see make_grid_ties.py).  Columns: v_bits step_bits h expected_code")
    for vbits, sbits, h in cases:
        print(f"0x{vbits:04x} 0x{sbits:04x} {str(h):>6} {8 + round_half_even(h)}")


if __name__ == "__main__":
    main()
