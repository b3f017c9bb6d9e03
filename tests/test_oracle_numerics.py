"""Pins of the oracle's bf16 / fp8 e4m3 emulation against torch's CPU casts."""
import numpy as np
import torch

from oracle import (FP8_E4M3_MAX, bf16_round, fp8_block_quantize, fp8_e4m3_decode,
                    fp8_e4m3_encode)


def _wide_fp32(n, seed=0):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(-2, 2, n)
    exp = rng.integers(-140, 120, n)
    return (mant * 2.0 ** exp).astype(np.float32)


def test_bf16_round_matches_torch_cast():
    x = _wide_fp32(200000)
    # exact ties and neighbours: bf16 value +- half ulp
    base = np.float32(1.0) + np.arange(0, 64, dtype=np.float32) * np.float32(2 ** -7)
    ties = np.concatenate([base + np.float32(2 ** -8), base - np.float32(2 ** -8), -base - np.float32(2 ** -8)])
    x = np.concatenate([x, ties.astype(np.float32), np.float32([0, -0.0, 1e-45, 3e38, -3.3e38])])
    ours = bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == FP8_E4M3_MAX
    assert ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, 300000) * 2.0 ** rng.integers(-12, 9, 300000)
    x = np.clip(x, -FP8_E4M3_MAX, FP8_E4M3_MAX).astype(np.float32)
    # midpoints between neighbours exercise ties-to-even
    mags = fp8_e4m3_decode(np.arange(0x7F))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = fp8_e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_encode_saturates():
    big = np.array([448.0, 449.0, 464.0, 500.0, 1e6, -1e9, np.finfo(np.float64).max])
    out = fp8_e4m3_decode(fp8_e4m3_encode(big))
    assert np.array_equal(out, np.sign(big) * FP8_E4M3_MAX)


def test_block_quantize_scale_and_zero_block():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 16))
    x[64:128] = 0.0
    codes, sc = fp8_block_quantize(x)
    assert sc.dtype == np.float32 and sc.shape == (4,)
    assert sc[1] == 1.0 and np.all(codes[64:128] == 0)
    for b in (0, 2, 3):
        blk = x[b * 64:(b + 1) * 64]
        i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        # the block's absmax maps to +-448 (code 0x7E / 0xFE) up to fp32 scale rounding
        assert codes[b * 64:(b + 1) * 64][i] & 0x7F == 0x7E
        deq = fp8_e4m3_decode(codes[b * 64:(b + 1) * 64]) * float(sc[b])
        # e4m3: relative step 2^-3 for normals; absolute step 2^-9*s below 2^-6*s
        err = np.abs(deq - blk)
        assert np.all(err <= np.maximum(np.abs(blk) * 2 ** -4, 2.0 ** -10 * float(sc[b])) * 1.0001)
