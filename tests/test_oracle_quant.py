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
