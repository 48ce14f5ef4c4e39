"""Pins for the oracle's bf16 conversions: hand-derived rounding cases and a
cross-check against torch's CPU bf16 cast (an independent implementation)."""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f32, f32_to_bf16


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


# (fp32 bits, expected bf16 bits), derived by hand from round-half-to-even
HAND_CASES = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # halfway 1.0 / 1.0078125 -> even (0x3F80)
    (0x3F818000, 0x3F82),  # halfway, lower neighbour odd -> up to even
    (0x3F808001, 0x3F81),  # just above half -> up
    (0x3F807FFF, 0x3F80),  # just below half -> down
    (0xBF808000, 0xBF80),  # negative tie -> even magnitude
    (0xBF818000, 0xBF82),
    (0x7F7FFFFF, 0x7F80),  # max finite fp32 rounds to +inf in bf16
    (0x7F7F7FFF, 0x7F7F),  # largest value that stays finite
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00008000, 0x0000),  # subnormal tie, kept part even -> down
    (0x00018000, 0x0002),  # subnormal tie, kept part odd -> up
    (0x007FFFFF, 0x0080),  # largest subnormal carries into the exponent
]


@pytest.mark.parametrize("u32,expect", HAND_CASES)
def test_f32_to_bf16_hand_cases(u32, expect):
    got = f32_to_bf16(f32_from_bits([u32]))[0]
    assert int(got) == expect, hex(int(got))


def test_nan_stays_nan():
    for u in (0x7FC00000, 0x7F800001, 0xFFC12345, 0x7FFFFFFF):
        b = int(f32_to_bf16(f32_from_bits([u]))[0])
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
        assert (b >> 15) == (u >> 31)


def test_narrow_matches_torch_random_bits():
    r = np.random.default_rng(11)
    u = r.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = f32_from_bits(u)
    finite = np.isfinite(x)
    ours = f32_to_bf16(x[finite])
    ref = torch_bf16_bits(x[finite])
    np.testing.assert_array_equal(ours, ref)


def test_narrow_matches_torch_ties_everywhere():
    # every exponent, low half exactly 0x8000 (a tie) with odd and even kept parts
    hi = np.arange(0, 0x7F7F, dtype=np.uint32)
    u = np.concatenate([(hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    u = np.concatenate([u, u | 0x80000000])
    x = f32_from_bits(u)
    np.testing.assert_array_equal(f32_to_bf16(x), torch_bf16_bits(x))


def test_widen_is_exact_and_matches_torch():
    b = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(b)
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(t)
    np.testing.assert_array_equal(np.isnan(x), nan)
    np.testing.assert_array_equal(x[~nan].view(np.uint32), t[~nan].view(np.uint32))
    # round trip of every non-NaN bf16 value is the identity
    np.testing.assert_array_equal(f32_to_bf16(x[~nan]), b[~nan])
