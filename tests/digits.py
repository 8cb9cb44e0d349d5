"""Test-side model of the 8-bit operands that stage 1 writes for stage 3.

Not part of the oracle: the pages define codes, tags, the bucket order and
the exact sum S; how the HIP path splits a shift-aligned code into 8-bit MFMA
operands is its own layout.  The parity tests check that layout by identity
against the oracle's codes and tags (``check_operands``): with a = q·2^e, the
code in units of the base (the left shift of DSTAR §3.1 step 5 applied to the
code itself), the aligned code equals a where PoT ≤ 6, and elsewhere the
digits satisfy a = d0 + 2^7·d1 + 2^15·d2 with every digit in its 8-bit range.
The CPU pins in ``test_oracle_pins.py`` show that these digits reproduce S
exactly (the split identity).
"""
from __future__ import annotations

import numpy as np

from oracle import fmdq

#: Largest PoT whose shift-aligned codes fit 8 bits (|q·2^e| ≤ 2^PoT ≤ 64).
ALIGNED_POT_MAX = 6
#: Largest PoT whose shift-aligned codes need no third digit (|q·2^e| ≤ 2^13).
TWO_DIGIT_POT_MAX = 13


def pot_of(tags: np.ndarray) -> np.ndarray:
    """PoT of every sub-channel from its tag byte: e + (b − 2)."""
    return fmdq.step_exponent(fmdq.tag_of(tags)) + (fmdq.bits_of(tags) - 2)


def shifted_codes(codes: np.ndarray, tags: np.ndarray) -> np.ndarray:
    """a = q·2^e, int64 [n_t][K][T]: every code in units of the base."""
    e = fmdq.step_exponent(fmdq.tag_of(tags))
    return np.asarray(codes).astype(np.int64) * np.left_shift(np.int64(1), e)[:, :, None]


def code_digits(a: np.ndarray):
    """Signed digits a = d0 + 2^7·d1 + 2^15·d2: d0 the residue mod 2^7 in
    [−64, 63], d1 the next residue mod 2^8 in [−128, 127], d2 the rest."""
    a = np.asarray(a).astype(np.int64)
    d0 = ((a + 64) % 128) - 64
    r1 = (a - d0) // 128
    d1 = ((r1 + 128) % 256) - 128
    d2 = (r1 - d1) // 256
    return d0, d1, d2


def aligned_codes(codes: np.ndarray, tags: np.ndarray) -> np.ndarray:
    """The dense operand as this model lays it out, [n_t·T][K] int8: a where
    PoT ≤ 6, else d0 (used by the CPU split-identity pins)."""
    codes = np.asarray(codes)
    nt, K, T = codes.shape
    a = shifted_codes(codes, tags)
    d0, _, _ = code_digits(a)
    out = np.where((pot_of(tags) <= ALIGNED_POT_MAX)[:, :, None], a, d0)
    return np.ascontiguousarray(out.transpose(0, 2, 1).reshape(nt * T, K)).astype(np.int8)


def heavy_digits(codes: np.ndarray, tags: np.ndarray) -> np.ndarray:
    """Digit planes [2][n_t][K][T] int8: d1 where PoT ≥ 7, d2 where PoT ≥ 14,
    0 elsewhere (used by the CPU split-identity pins)."""
    pot = pot_of(tags)[:, :, None]
    _, d1, d2 = code_digits(shifted_codes(codes, tags))
    return np.stack([np.where(pot > ALIGNED_POT_MAX, d1, 0),
                     np.where(pot > TWO_DIGIT_POT_MAX, d2, 0)]).astype(np.int8)


def check_operands(acodes: np.ndarray, hcodes: np.ndarray, codes: np.ndarray, tags: np.ndarray,
                   what: str = "") -> None:
    """Stage 1's aligned codes ([n_t·T][K]) and digit planes ([2][n_t][K][T])
    against the oracle's codes and tags, by identity and digit ranges.  Only
    the digit-plane entries the layout defines are read (PoT ≥ 7 for the first
    plane, PoT ≥ 14 for the second)."""
    codes = np.asarray(codes)
    nt, K, T = codes.shape
    a = shifted_codes(codes, tags)                                         # [n_t][K][T]
    pot = np.broadcast_to(pot_of(tags)[:, :, None], a.shape)
    d0 = np.asarray(acodes).reshape(nt, T, K).transpose(0, 2, 1).astype(np.int64)
    light = pot <= ALIGNED_POT_MAX
    np.testing.assert_array_equal(d0[light], a[light], err_msg=f"{what}: aligned codes (PoT <= 6)")
    heavy = ~light
    d1 = np.where(heavy, np.asarray(hcodes[0]).astype(np.int64), 0)
    d2 = np.where(pot > TWO_DIGIT_POT_MAX, np.asarray(hcodes[1]).astype(np.int64), 0)
    if heavy.any():
        assert -64 <= d0[heavy].min() and d0[heavy].max() <= 63, f"{what}: d0 out of range"
        assert -128 <= d1.min() and d1.max() <= 127, f"{what}: d1 out of range"
        assert -64 <= d2.min() and d2.max() <= 64, f"{what}: d2 out of range"
        np.testing.assert_array_equal((d0 + 128 * d1 + 32768 * d2)[heavy], a[heavy],
                                      err_msg=f"{what}: a = d0 + 2^7 d1 + 2^15 d2")
