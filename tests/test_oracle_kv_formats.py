"""Pins for the oracle's fp8 e5m2 and INT8 / INT4 cache formats (CPU only).

Library routine: torch's float8_e5m2 (decode of all 256 codes; fp32 ->
e5m2 casts, which round to nearest even, on a grid holding every tie).
Brute force: integer codes are the argmin of |x/s - c| over every code,
ties to the even integer.  Closed forms: explicit packed bytes, zero rows,
exactly representable rows, half-step error bounds, and a pool write/read
round trip."""
import numpy as np
import pytest
import torch

from oracle import cache, kv_formats as kf


def test_e5m2_decode_matches_torch():
    ours = kf.e5m2_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], ref[fin])
    assert kf.e5m2_decode_code(0x7B) == 57344.0 and kf.e5m2_decode_code(0x01) == 2.0 ** -16


def test_e5m2_encode_matches_torch_on_grid_with_ties():
    pos = kf.e5m2_table()[:0x7C]
    mids = (pos[:-1] + pos[1:]) / 2                              # every tie between neighbours
    rng = np.random.default_rng(3)
    rand = rng.uniform(-57344, 57344, 20000) * rng.choice([1, 1e-3, 1e-6, 1e-9], 20000)
    y = np.concatenate([pos, -pos, mids, -mids, rand, [0.0, -0.0]]).astype(np.float32)
    ours = kf.e5m2_encode_rne(y)
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def _brute_int(y, q):
    cand = np.arange(-q, q + 1, dtype=np.float64)
    d = np.abs(np.asarray(y, np.float64)[..., None] - cand)
    best = d.min(axis=-1, keepdims=True)
    ties = np.isclose(d, best, rtol=0, atol=0)
    # among equally near codes take the even one
    even = ties & (cand % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, ties)
    return cand[np.argmax(pick, axis=-1)].astype(np.int8)


@pytest.mark.parametrize("q", [kf.INT8_MAX, kf.INT4_MAX])
def test_int_codes_are_nearest_with_ties_to_even(q):
    rng = np.random.default_rng(q)
    x = rng.standard_normal((64, 4, 128)).astype(np.float32)
    # rows built so that x / s lands exactly on every half-integer: each row's
    # maximum is q * 2^-3 (s = 2^-3) and its other entries (k + 1/2) * 2^-3
    halves = (np.arange(-q, q) + 0.5).astype(np.float32) * np.float32(0.125)
    pieces = [halves[i:i + 127] for i in range(0, halves.size, 127)]
    for r, piece in enumerate(pieces):
        row = np.zeros(128, np.float32)
        row[:piece.size] = piece
        row[-1] = np.float32(q * 0.125)
        x[0, r] = row
    codes, s = kf.quantise_int_rows(x, q)
    assert all(s[0, r] == np.float32(0.125) for r in range(len(pieces)))
    y = np.clip((x / s[..., None]).astype(np.float32), -q, q)
    assert np.array_equal(codes, _brute_int(y, q))
    # the ties went to even integers
    for r, piece in enumerate(pieces):
        assert np.all(codes[0, r, :piece.size].astype(int) % 2 == 0)
    # half-step error bound
    err = np.abs(kf.dequantise_int(codes, s) - x)
    assert np.all(err <= s[..., None].astype(np.float64) / 2 * (1 + 1e-6))


def test_int4_packing_bytes():
    assert kf.pack_int4(np.array([1, -1])).tolist() == [0xF1]
    assert kf.pack_int4(np.array([-8, 7, 0, 3])).tolist() == [0x78, 0x30]
    rng = np.random.default_rng(1)
    c = rng.integers(-8, 8, size=(5, 3, 64)).astype(np.int8)
    assert np.array_equal(kf.unpack_int4(kf.pack_int4(c)), c)


def test_zero_and_exact_rows():
    z = np.zeros((2, 64), np.float32)
    for elem in ("e5m2", "i8", "i4"):
        codes, s = kf.quantise(z, elem)
        assert np.all(s == 1.0) and np.all(kf.dequantise(codes, s, elem) == 0.0)
    # integers 0..7 with max 7: s = 1, i4 exact; i8: s = 7/127, not exact
    r = np.arange(-7, 8, dtype=np.float32)[None, :].repeat(2, axis=0)
    r = np.concatenate([r, np.zeros((2, 1), np.float32)], axis=1)
    assert np.array_equal(kf.values_as_cached(r, "i4"), r.astype(np.float64))


def test_e5m2_relative_error_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((128, 128)).astype(np.float32) * 3
    codes, s = kf.quantise_e5m2_rows(x)
    deq = kf.dequantise_e5m2(codes, s)
    big = np.abs(x) > 2.0 ** -14 * s[:, None]                # normal range of the scaled value
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -3 * np.abs(x)[big] * (1 + 1e-6))


@pytest.mark.parametrize("fmt", ["fp8_e5m2", "int8_int4"])
def test_pool_round_trip(fmt):
    rng = np.random.default_rng(4)
    pool = cache.Pool(6, 2, 64, fmt)
    k = rng.standard_normal((20, 2, 64)).astype(np.float32)
    v = rng.standard_normal((20, 2, 64)).astype(np.float32)
    slots = np.concatenate([np.arange(16, 32), np.arange(80, 84)])
    pool.append(k, v, slots)
    K, V = pool.gather([1, 5], 20)
    ke, ve = kf.FORMATS[fmt]
    assert np.array_equal(K, kf.values_as_cached(k, ke)) and np.array_equal(V, kf.values_as_cached(v, ve))
    if fmt == "int8_int4":
        assert pool.v_codes.shape == (6, 2, 16, 32)
