"""Pins for the oracle's OCP e4m3 codec and per-row quantisation.

The codec is pinned against PyTorch's float8_e4m3fn dtype (a library routine,
run and compared, never read): every one of the 256 codes decodes to the same
value, and encoding agrees with torch's cast over a dense grid that contains
every representable value, every midpoint (the ties) and the subnormal range.
"""
import numpy as np
import pytest
import torch

from oracle import fp8_e4m3


def test_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8_e4m3.decode_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert sorted(np.nonzero(nan_ref)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def _torch_encode(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_grid_with_ties():
    vals = fp8_e4m3.decode_table()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2.0          # exact ties (fit in float32)
    quarter = (3 * vals[:-1] + vals[1:]) / 4.0
    three_q = (vals[:-1] + 3 * vals[1:]) / 4.0
    grid = np.concatenate([vals, mids, quarter, three_q]).astype(np.float32)
    grid = np.concatenate([grid, -grid])
    assert np.array_equal(fp8_e4m3.encode_rne(grid), _torch_encode(grid))


def test_encode_matches_torch_on_float32_bit_patterns():
    # every float32 with its 12 low mantissa bits zero, from 0 up to 448
    top = np.float32(448.0).view(np.uint32) >> 12
    bits = (np.arange(0, int(top) + 1, dtype=np.uint32) << 12)
    y = bits.view(np.float32)
    y = np.concatenate([y, -y])
    assert np.array_equal(fp8_e4m3.encode_rne(y), _torch_encode(y))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(0)
    y = np.clip(rng.standard_normal(200000).astype(np.float32) * 100, -448, 448)
    assert np.array_equal(fp8_e4m3.encode_rne(y), _torch_encode(y))


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        fp8_e4m3.encode_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        fp8_e4m3.encode_rne(np.array([np.nan]))


def test_round_trip_bound_normal_range():
    # 3 stored mantissa bits: RNE error <= half an ulp = 2^-4 relative
    rng = np.random.default_rng(1)
    y = rng.uniform(2.0 ** -6, 448, 100000).astype(np.float32)
    back = fp8_e4m3.decode_table()[fp8_e4m3.encode_rne(y)]
    assert np.all(np.abs(back - y) <= 2.0 ** -4 * np.abs(y))


def test_quantise_rows_scale_and_extremes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[5] = 0.0                                   # an all-zero row
    codes, scales = fp8_e4m3.quantise_rows(x)
    amax = np.max(np.abs(x), axis=-1)
    expect_s = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    assert scales.dtype == np.float32 and np.array_equal(scales, expect_s)
    assert np.all(codes[5] == 0)
    table = fp8_e4m3.decode_table()
    for r in range(64):
        if r == 5:
            continue
        j = int(np.argmax(np.abs(x[r])))
        # the largest element lands on +-448 (after the clamp)
        assert abs(table[codes[r, j]]) == 448.0
        assert np.sign(table[codes[r, j]]) == np.sign(x[r, j])
    deq = fp8_e4m3.dequantise(codes, scales)
    # per-element error is within half an e4m3 ulp of the scaled value (plus
    # the subnormal absolute step 2^-10 * s)
    err = np.abs(deq - x)
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scales[:, None] + 1e-12
    assert np.all(err <= bound)


def test_quantise_matches_torch_pipeline():
    # the same reading written with torch ops: float32 amax/448, float32
    # division, clamp, torch cast
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 64)) * rng.uniform(0.01, 50, (256, 1))).astype(np.float32)
    codes, scales = fp8_e4m3.quantise_rows(x)
    tx = torch.from_numpy(x)
    ts = tx.abs().amax(dim=-1) / 448.0
    ts = torch.where(ts == 0, torch.ones_like(ts), ts)
    tc = torch.clamp(tx / ts[:, None], -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(scales, ts.numpy())
    assert np.array_equal(codes, tc.numpy())
