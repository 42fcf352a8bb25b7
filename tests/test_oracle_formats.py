"""Pins for the oracle's number formats (bf16, fp8-e4m3fn).

The oracle writes its own conversions from the format definitions. They are pinned against
hand-derived code points (tests/golden), against torch's CPU conversions (an independent
implementation) over sweeps that hit every rounding decision, and against properties of
round-to-nearest-even.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import golden_lines


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _torch_bf16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _structured_f32(max_exp_field: int) -> np.ndarray:
    """Every sign, every exponent field up to max_exp_field, every value of the top 8 mantissa
    bits, and low-15-bit patterns around the tie and sticky positions: this covers every rounding
    decision of a format that keeps at most 7 mantissa bits."""
    sign = np.array([0, 1], np.uint32)[:, None, None, None]
    ex = np.arange(0, max_exp_field + 1, dtype=np.uint32)[None, :, None, None]
    top = np.arange(256, dtype=np.uint32)[None, None, :, None]
    low = np.array([0, 1, 0x3FFF, 0x4000, 0x4001, 0x7FFE, 0x7FFF], np.uint32)[None, None, None, :]
    bits = (sign << 31) | (ex << 23) | (top << 15) | low
    return bits.reshape(-1).view(np.float32)


# ---------------------------------------------------------------------------------------- e4m3 --
def test_e4m3_golden_code_points():
    rows = [line.split() for line in golden_lines("e4m3_ocp_values.txt")]
    assert len(rows) >= 20
    codes = np.array([int(r[0], 16) for r in rows], np.uint8)
    vals = oracle.e4m3_to_f32(codes)
    for (c, bits, v), got in zip(rows, vals):
        s = bits.replace(".", "")
        assert int(s, 2) == int(c, 16), f"fixture bit string {bits} != {c}"
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), c
            if abs(float(v)) <= 448:   # encoding the exact value returns the code
                assert oracle.f32_to_e4m3(np.array([float(v)], np.float32))[0] == int(c, 16)


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2   # only S.1111.111
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_encode_structured_sweep_vs_torch():
    v = _structured_f32(135)                     # up to 2^8 * 1.99, i.e. past 448
    v = v[np.abs(v) <= 448.0]
    ours = oracle.f32_to_e4m3(v)
    assert np.array_equal(ours, _torch_e4m3(v))


def test_e4m3_encode_random_vs_torch():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2**32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    # also dense values in the magnitudes that carry scaled activations
    v2 = (rng.standard_normal(1_000_000) * rng.choice([1e-3, 1.0, 100.0], 1_000_000)).astype(
        np.float32)
    v = np.concatenate([v, v2[np.abs(v2) <= 448.0]])
    assert np.array_equal(oracle.f32_to_e4m3(v), _torch_e4m3(v))


def test_e4m3_saturates_and_keeps_nan():
    v = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert list(oracle.f32_to_e4m3(v)) == [0x7E] * 7 + [0xFE, 0xFE]
    q = oracle.f32_to_e4m3(np.array([np.nan, -np.nan], np.float32))
    assert all((c & 0x7F) == 0x7F for c in q)


def test_e4m3_round_to_nearest_property():
    """The code is the nearest representable value; on a tie the code with even mantissa wins."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    grid = np.unique(oracle.e4m3_to_f32(finite).astype(np.float64))
    rng = np.random.default_rng(7)
    v = rng.uniform(-448, 448, 200_000).astype(np.float32)
    v = np.concatenate([v, (grid[:-1] + grid[1:]).astype(np.float32) / 2])   # exact midpoints
    got = oracle.e4m3_to_f32(oracle.f32_to_e4m3(v)).astype(np.float64)
    lo = grid[np.clip(np.searchsorted(grid, v, side="right") - 1, 0, len(grid) - 1)]
    hi = grid[np.clip(np.searchsorted(grid, v, side="left"), 0, len(grid) - 1)]
    dv = v.astype(np.float64)
    best = np.minimum(np.abs(lo - dv), np.abs(hi - dv))
    assert np.all(np.abs(got - dv) == best)
    tie = np.abs(lo - dv) == np.abs(hi - dv)
    tie &= lo != hi
    codes = oracle.f32_to_e4m3(v[tie])
    assert tie.sum() > 100 and np.all((codes & 1) == 0)


@pytest.mark.skipif(os.environ.get("MOE_EXHAUSTIVE") != "1",
                    reason="exhaustive 2^32 sweep: set MOE_EXHAUSTIVE=1 (takes minutes)")
def test_e4m3_encode_exhaustive_vs_torch():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        v = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
        if v.size:
            assert np.array_equal(oracle.f32_to_e4m3(v), _torch_e4m3(v)), hex(start)


# ---------------------------------------------------------------------------------------- bf16 --
def test_bf16_golden_values():
    rows = [line.split(maxsplit=2) for line in golden_lines("bf16_values.txt")]
    assert len(rows) >= 15
    vals = np.array([float.fromhex(r[0]) for r in rows], np.float64)
    want = [int(r[1], 16) for r in rows]
    assert list(oracle.f64_to_bf16(vals)) == want
    # the same values through the fp32 entry point, where they are exact in fp32
    exact32 = vals.astype(np.float32).astype(np.float64) == vals
    assert list(oracle.f32_to_bf16(vals[exact32].astype(np.float32))) == \
        [w for w, e in zip(want, exact32) if e]


def test_bf16_structured_sweep_vs_torch():
    v = _structured_f32(254)
    assert np.array_equal(oracle.f32_to_bf16(v), _torch_bf16(v))


def test_bf16_random_and_specials_vs_torch():
    rng = np.random.default_rng(99)
    v = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = v[~np.isnan(v)]
    v = np.concatenate([v, np.array([np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45],
                                    np.float32)])
    assert np.array_equal(oracle.f32_to_bf16(v), _torch_bf16(v))
    n = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (n & 0x7F80) == 0x7F80 and (n & 0x7F) != 0


def test_bf16_from_double_is_nearest():
    """Double inputs (the combine sums): the result is one of the two bf16 neighbours and the
    nearer one; ties go to the even code. Checked with exact double arithmetic."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal(300_000) * np.exp2(rng.integers(-30, 30, 300_000))
    b = oracle.f64_to_bf16(v).astype(np.uint32)
    got = oracle.bf16_to_f32(b.astype(np.uint16)).astype(np.float64)
    # neighbours: truncation toward zero and one code up in magnitude
    trunc = (v.astype(np.float32).view(np.uint32) >> 16)
    for cand in (trunc - 1, trunc, trunc + 1):
        cv = oracle.bf16_to_f32(cand.astype(np.uint16)).astype(np.float64)
        cv = np.where(np.isnan(cv), np.inf, cv)
        assert np.all(np.abs(got - v) <= np.abs(cv - v))
