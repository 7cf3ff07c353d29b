"""Pins of the int8 quantiser: the half-step error bound, the absmax code, exact
round trips on the grid, zero and partly filled tiles."""

import numpy as np
import pytest

import oracle


def check_error_bound(seed):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        x = (rng.standard_normal((16, 32)) * rng.uniform(0.01, 30)).astype(np.float16)
        filled = int(rng.integers(1, 17))
        codes, scale = oracle.quantize_block_int8(x, filled)
        xhat = oracle.dequantize_int8(codes[:filled], scale)
        err = np.abs(x[:filled].astype(np.float64) - xhat)
        # rounding to the nearest code never errs by more than half a step
        assert err.max() <= float(scale) / 2 * (1 + 1e-12)
        # the largest magnitude maps to the end of the code range
        i = np.unravel_index(np.argmax(np.abs(x[:filled].astype(np.float32))), (filled, 32))
        assert abs(int(codes[:filled][i])) == 127
        assert np.abs(codes).max() <= 127
        assert not codes[filled:].any()


def test_error_bound_and_absmax():
    check_error_bound(1)


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(2)
    for e in range(-8, 3):
        s = np.float16(3 * 2.0**e)  # two significant bits: k * s is exact in fp16
        k = rng.integers(-127, 128, (16, 64))
        k[3, 5] = 127
        x = (k * float(s)).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), k * float(s))
        codes, scale = oracle.quantize_block_int8(x)
        assert scale == s
        assert np.array_equal(codes.astype(np.int64), k)
        assert np.array_equal(oracle.dequantize_int8(codes, scale), x.astype(np.float64))


def test_zero_tile():
    codes, scale = oracle.quantize_block_int8(np.zeros((16, 8), np.float16))
    assert scale == 0 and not codes.any()
    codes, scale = oracle.quantize_block_int8(np.ones((16, 8), np.float16), filled=0)
    assert scale == 0 and not codes.any()


def test_unfilled_rows_do_not_set_the_scale():
    x = np.ones((16, 8), np.float16)
    x[5:] = 1000
    codes, scale = oracle.quantize_block_int8(x, filled=5)
    assert scale == np.float16(1 / 127)
    assert np.all(codes[:5] == 127) and not codes[5:].any()


def test_pool_quantiser_covers_every_filled_block():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((1, 4, 2, 16, 8)).astype(np.float16)
    V = rng.standard_normal((1, 4, 2, 16, 8)).astype(np.float16)
    K8, V8, S = oracle.quantize_pool_int8(K, V, [16, 0, 3, 16])
    assert not K8[0, 1].any() and not S[0, 1].any()
    for n, f in ((0, 16), (2, 3), (3, 16)):
        for g in range(2):
            c, s = oracle.quantize_block_int8(K[0, n, g], f)
            assert np.array_equal(K8[0, n, g], c) and S[0, n, g, 0] == s
            c, s = oracle.quantize_block_int8(V[0, n, g], f)
            assert np.array_equal(V8[0, n, g], c) and S[0, n, g, 1] == s


# ---------------------------------------------------------------------------
# quantise-on-write: one token at a time into a partly filled block

def test_append_into_empty_block_matches_block_quantiser():
    """A token opening a block is quantised exactly as a one-row tile."""
    rng = np.random.default_rng(4)
    stale = rng.integers(-127, 128, (16, 32)).astype(np.int8)  # a reused block's old codes
    for _ in range(40):
        x = (rng.standard_normal(32) * rng.uniform(0.01, 50)).astype(np.float16)
        codes, scale = oracle.append_row_int8(stale, np.float16(7.0), 0, x)
        tile = np.zeros((16, 32), np.float16)
        tile[0] = x
        ref_codes, ref_scale = oracle.quantize_block_int8(tile, filled=1)
        assert scale == ref_scale and np.array_equal(codes[0], ref_codes[0])
        assert np.array_equal(codes[1:], stale[1:])  # rows past the slot untouched


def _filled_tile(rng, n, spread):
    rows = [(rng.standard_normal(24) * rng.uniform(*spread)).astype(np.float16) for _ in range(n)]
    codes, scale = np.zeros((16, 24), np.int8), np.float16(0)
    for off, x in enumerate(rows):
        codes, scale = oracle.append_row_int8(codes, scale, off, x)
    return rows, codes, scale


def test_append_within_range_keeps_earlier_codes():
    rng = np.random.default_rng(5)
    for _ in range(40):
        rows, codes, scale = _filled_tile(rng, int(rng.integers(1, 15)), (1.0, 3.0))
        off = len(rows)
        x = (rng.uniform(-1, 1, 24) * 127 * float(scale)).astype(np.float16)
        x = np.clip(x, -127 * float(scale), 127 * float(scale)).astype(np.float16)
        assert np.abs(x.astype(np.float32)).max() <= np.float32(127) * np.float32(scale)
        new_codes, new_scale = oracle.append_row_int8(codes, scale, off, x)
        assert new_scale == scale
        assert np.array_equal(new_codes[:off], codes[:off])
        err = np.abs(oracle.dequantize_int8(new_codes[off], new_scale) - x.astype(np.float64))
        assert err.max() <= float(scale) / 2 * (1 + 1e-6)


def test_append_beyond_range_requantises_the_block():
    rng = np.random.default_rng(6)
    for _ in range(40):
        rows, codes, scale = _filled_tile(rng, int(rng.integers(1, 15)), (0.5, 1.0))
        off = len(rows)
        x = (rng.standard_normal(24) * 40).astype(np.float16)
        a = float(np.abs(x.astype(np.float32)).max())
        assert a > 127 * float(scale)
        new_codes, new_scale = oracle.append_row_int8(codes, scale, off, x)
        assert new_scale == np.float16(np.float32(a) / np.float32(127)) and new_scale >= scale
        # the new row: half a step of the new scale, and its absmax at the end of the range
        err = np.abs(oracle.dequantize_int8(new_codes[off], new_scale) - x.astype(np.float64))
        assert err.max() <= float(new_scale) / 2 * (1 + 1e-6)
        assert np.abs(new_codes[off]).max() == 127
        # earlier rows move by at most half a new step from their old values
        before = oracle.dequantize_int8(codes[:off], scale)
        after = oracle.dequantize_int8(new_codes[:off], new_scale)
        assert np.abs(after - before).max() <= float(new_scale) / 2 * (1 + 1e-6)


def test_appended_block_tracks_its_data():
    """After any sequence of appends the scale has never shrunk, and each
    filled row is within its error budget of its fp16 data: half a step of
    the scale it was written with, plus half a step of every larger scale
    the block moved to afterwards (each re-expression rounds once)."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        codes, scale = np.zeros((16, 16), np.int8), np.float16(0)
        rows, scales, budget = [], [], []
        for off in range(16):
            x = (rng.standard_normal(16) * rng.choice([0.1, 1.0, 5.0, 30.0])).astype(np.float16)
            old = scale
            codes, scale = oracle.append_row_int8(codes, scale, off, x)
            if off > 0 and scale != old:
                budget = [b + float(scale) / 2 for b in budget]
            budget.append(float(scale) / 2)
            rows.append(x)
            scales.append(float(scale))
        assert all(b >= a for a, b in zip(scales, scales[1:]))
        err = np.abs(oracle.dequantize_int8(codes, scale) - np.array(rows, np.float64)).max(axis=1)
        assert np.all(err <= np.array(budget) * (1 + 1e-6))
        assert np.abs(codes.astype(np.int64)).max() <= 127


def test_append_on_a_common_grid_is_exact():
    """Rows that are integer multiples of one step, the first reaching 127
    steps, are stored exactly: no later row changes the scale."""
    rng = np.random.default_rng(8)
    s = np.float16(0.25)
    codes, scale = np.zeros((16, 8), np.int8), np.float16(0)
    ks = rng.integers(-127, 128, (16, 8))
    ks[0, 0] = 127
    for off in range(16):
        x = (ks[off] * float(s)).astype(np.float16)
        codes, scale = oracle.append_row_int8(codes, scale, off, x)
    assert scale == s
    assert np.array_equal(codes.astype(np.int64), ks)


def test_append_zero_rows_then_data():
    codes, scale = oracle.append_row_int8(np.zeros((16, 4), np.int8), np.float16(0), 0, np.zeros(4, np.float16))
    assert scale == 0 and not codes.any()
    codes, scale = oracle.append_row_int8(codes, scale, 1, np.zeros(4, np.float16))
    assert scale == 0 and not codes.any()
    x = np.array([1.0, -2.0, 0.5, 0.0], np.float16)
    codes, scale = oracle.append_row_int8(codes, scale, 2, x)
    assert scale == np.float16(np.float32(2.0) / np.float32(127))
    assert not codes[:2].any() and codes[2, 1] == -127
