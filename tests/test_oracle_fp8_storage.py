"""CPU pins of the oracle's fp8 storage model (storage="fp8").

The quantised QK path publishes Q and K as OCP e4m3 codes with a scale per
64-token block of each chunk (the pages name an FP8 K/V payload "and scale",
thelatestinai.com listing, Table 8, and an fp8 SageAttention backend, Table 6).
K first has its per-(chunk, head) channel mean removed, and the mean is added
back exactly: K_hat = deq(K8) + mean. Q is quantised without a mean.

Each property below follows from that definition and the e4m3 format alone:
  * the reconstruction error of every element is at most half an e4m3 step of
    (x - mean) / scale, times the scale of the element's own block, where
    scale = absmax of the block / 448 (so at most 2^-4 |x - mean| plus the
    subnormal half step 2^-10 * scale);
  * the element at a block's absmax maps to +-448 and comes back exactly (up
    to the fp32 rounding of the scale);
  * a chunk whose K is constant in every channel reconstructs exactly (the
    mean takes all of it, the codes are zero);
  * the blocks restart at each chunk start: a 72-token chunk ends in an
    8-token block with a scale of its own, whatever the chunk before it held;
  * scaling the input by a power of two scales the output by the same power
    exactly (absmax scales are exact under it).

Every check is a function of the implementation under test, so the last test
can plant a mistake in a copy of the oracle and see a pin fail.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import wf_inputs as W
from oracle import fp8_block_quantize, fp8_e4m3_decode, rotated_context
from oracle import round as oracle_round_mod

SUB_HALF_STEP = 2.0 ** -10     # half the e4m3 subnormal step 2^-9
REL_HALF_STEP = 2.0 ** -4      # half of the relative step 2^-3 of a normal e4m3 value
SLACK = 1.0 + 2.0 ** -20       # fp64 arithmetic of the reconstruction


def _block_absmax(x: np.ndarray, block: int = 64) -> np.ndarray:
    """Per-token absmax of its block's |x| over all channels, x[N, d]."""
    N = x.shape[0]
    out = np.empty(N)
    for b0 in range(0, N, block):
        out[b0:b0 + block] = np.max(np.abs(x[b0:b0 + block]))
    return out


def _half_step_bound(x: np.ndarray) -> np.ndarray:
    """Largest error a correct block quantiser may leave on x[N, d]."""
    scale = (_block_absmax(x).astype(np.float32) / np.float32(448.0)).astype(np.float64)
    return (np.abs(x) * REL_HALF_STEP + SUB_HALF_STEP * scale[:, None]) * SLACK


def _chunk(N, heads, d, seed, loc=0.0, spread=1.0):
    rng = np.random.default_rng(seed)
    return loc + spread * rng.standard_normal((N, heads, d))


# --- checks on the K model: fk(kr[N, heads, d]) -> K_hat[N, heads, d] ---------

def check_k_error_bound(fk):
    """A large per-channel offset plus noise: the mean removes the offset, so
    the error is bounded by the noise's own block scales."""
    rng = np.random.default_rng(7)
    offs = rng.uniform(-6, 6, (1, 2, 64))
    kr = offs + _chunk(200, 2, 64, 8, spread=0.5)
    out = fk(kr)
    for h in range(2):
        mu = np.mean(kr[:, h, :], axis=0)
        x = kr[:, h, :] - mu
        assert np.all(np.abs(out[:, h, :] - kr[:, h, :]) <= _half_step_bound(x) + 1e-12 * np.abs(mu)), h


def check_k_absmax_exact(fk):
    kr = _chunk(128, 1, 32, 9, loc=1.5)
    out = fk(kr)
    x = kr[:, 0, :] - np.mean(kr[:, 0, :], axis=0)
    for b0 in (0, 64):
        blk = x[b0:b0 + 64]
        i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        assert abs(out[b0 + i, 0, j] - kr[b0 + i, 0, j]) <= 2.0 ** -22 * abs(blk[i, j]) + 1e-12


def check_k_constant_channels(fk):
    """K constant along tokens in every channel (different per channel): the
    chunk mean is that constant, the remainder is zero, so K_hat == K."""
    a = ((np.arange(64) - 31.5) / 8.0)[None, None, :]
    kr = np.broadcast_to(a, (72, 1, 64)).copy()
    out = fk(kr)
    assert np.array_equal(out, kr)


def check_k_short_last_block(fk):
    """72 tokens: 64 tokens of magnitude ~1e4, then 8 of magnitude ~1e-3, each
    group zero-mean per channel, so the chunk mean is exactly 0. The last 8
    tokens are a block of their own and keep their small scale (under the big
    block's scale they would all round to zero)."""
    rng = np.random.default_rng(10)
    # integers and multiples of 2^-20: every partial sum is exact in fp64
    big = np.rint(rng.standard_normal((32, 1, 16)) * 1e4)
    small = np.rint(rng.standard_normal((4, 1, 16)) * 1e3) * 2.0 ** -20
    kr = np.concatenate([big, -big, small, -small], axis=0)
    assert np.all(np.mean(kr, axis=0) == 0)
    out = fk(kr)
    x = kr[:, 0, :]
    assert np.all(np.abs(out[:, 0, :] - x) <= _half_step_bound(x))
    assert np.max(np.abs(out[64:, 0, :] - x[64:])) <= np.max(np.abs(x[64:])) * REL_HALF_STEP * SLACK


def check_k_power_of_two(fk):
    kr = _chunk(100, 2, 32, 11, loc=0.7)
    assert np.array_equal(fk(kr * 4.0), fk(kr) * 4.0)
    assert np.array_equal(fk(kr * 2.0 ** -6), fk(kr) * 2.0 ** -6)


K_CHECKS = [check_k_error_bound, check_k_absmax_exact, check_k_constant_channels,
            check_k_short_last_block, check_k_power_of_two]


# --- checks on the Q model: fq(qr[N, heads, d]) -> Q_hat ---------------------

def check_q_error_bound(fq):
    qr = _chunk(150, 2, 64, 12, spread=2.0)
    qr[64:128, 1, :] *= 1e-3                     # one block far smaller than its neighbours
    out = fq(qr)
    for h in range(2):
        assert np.all(np.abs(out[:, h, :] - qr[:, h, :]) <= _half_step_bound(qr[:, h, :])), h


def check_q_no_mean(fq):
    """A constant offset is not removed from Q: a block holding +-3.5 in
    every element (scale 3.5 / 448 = 2^-7, exact) quantises to +-448 codes and
    comes back exactly."""
    qr = np.full((64, 1, 8), 3.5)
    qr[:, 0, 1::2] = -3.5
    assert np.array_equal(fq(qr), qr)


def check_q_zero_block_and_tail(fq):
    qr = _chunk(72, 1, 16, 13)
    qr[:64] = 0.0
    out = fq(qr)
    assert np.all(out[:64] == 0.0)
    assert np.all(np.abs(out[64:, 0, :] - qr[64:, 0, :]) <= _half_step_bound(qr[:, 0, :])[64:])


def check_q_power_of_two(fq):
    qr = _chunk(100, 2, 32, 14)
    assert np.array_equal(fq(qr * 8.0), fq(qr) * 8.0)


Q_CHECKS = [check_q_error_bound, check_q_no_mean, check_q_zero_block_and_tail, check_q_power_of_two]


# --- the chunk restart, through the context the oracle builds ----------------

SHAPE72 = dataclasses.replace(W.WORKLOADS["edge_s1_h0"], heads=1, seed=31)   # 72-token chunks, S=1, A=2


def _context_inputs(w, k):
    """Anchor/history and live chunks of very different magnitudes, each with
    its last 8 tokens 1e4 times smaller than the rest: a block that ran across
    a chunk boundary, or one block per chunk, would give those tokens a scale
    far too large for them. RoPE keeps each token's magnitude."""
    rng = np.random.default_rng(w.seed)
    mags = [1e3, 1e-3, 1e2, 1e-2]
    tok = np.where(np.arange(w.N) < 64, 1.0, 1e-4)[:, None]
    live = [tuple(rng.standard_normal((w.N, w.hd)) * tok * mags[(s + 1) % 4] for _ in range(3))
            for s in range(w.S + 1)]
    from oracle import RoundSchedule
    sch = RoundSchedule(w.S, w.A, w.H, k)
    clean = {c: tuple(rng.standard_normal((w.N, w.hd)) * tok * mags[i % 4] for _ in range(2))
             for i, c in enumerate(sch.chunk_ids()[:w.A + w.H])}
    return live, clean


def check_context_blocks_restart(ctx_fn):
    w, k = SHAPE72, SHAPE72.steady_round
    live, clean = _context_inputs(w, k)
    Qx, kx, _, _ = ctx_fn(w, k, live, clean, "exact")
    Qf, kf, _, _ = ctx_fn(w, k, live, clean, "fp8")
    for p in range(w.T):
        x = kx[p][:, 0, :] - np.mean(kx[p][:, 0, :], axis=0)
        bound = _half_step_bound(x) + 1e-12 * np.max(np.abs(kx[p]))
        assert np.all(np.abs(kf[p][:, 0, :] - kx[p][:, 0, :]) <= bound), p
    for s in range(w.S + 1):
        assert np.all(np.abs(Qf[s][:, 0, :] - Qx[s][:, 0, :]) <= _half_step_bound(Qx[s][:, 0, :])), s


# --- the oracle against its pins ---------------------------------------------

@pytest.mark.parametrize("check", K_CHECKS, ids=lambda f: f.__name__)
def test_fp8_k_model(check):
    check(oracle_round_mod._fp8_k)


@pytest.mark.parametrize("check", Q_CHECKS, ids=lambda f: f.__name__)
def test_fp8_q_model(check):
    check(oracle_round_mod._fp8_q)


def test_fp8_context_blocks_restart_at_each_chunk():
    check_context_blocks_restart(rotated_context)


# --- planted mistakes: each one fails at least one pin ------------------------

def _deq(codes, sc, n):
    return fp8_e4m3_decode(codes) * np.repeat(sc.astype(np.float64), 64)[:n, None]


def _k_without_mean_readd(kr):
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:, h, :], axis=0).astype(np.float32).astype(np.float64)
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu[None, :])
        out[:, h, :] = _deq(codes, sc, kr.shape[0])
    return out


def _k_mean_over_channels(kr):
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:, h, :], axis=1).astype(np.float32).astype(np.float64)[:, None]
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu)
        out[:, h, :] = _deq(codes, sc, kr.shape[0]) + mu
    return out


def _k_no_mean(kr):
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        codes, sc = fp8_block_quantize(kr[:, h, :])
        out[:, h, :] = _deq(codes, sc, kr.shape[0])
    return out


def _k_one_block_per_chunk(kr):
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:, h, :], axis=0).astype(np.float32).astype(np.float64)
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu[None, :], block=kr.shape[0])
        out[:, h, :] = fp8_e4m3_decode(codes) * float(sc[0]) + mu[None, :]
    return out


def _k_scales_shifted(kr):
    """Each token dequantised with the next block's scale."""
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:, h, :], axis=0).astype(np.float32).astype(np.float64)
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu[None, :])
        sc2 = np.roll(sc, -1)
        out[:, h, :] = _deq(codes, sc2, kr.shape[0]) + mu[None, :]
    return out


def _k_mean_of_half(kr):
    """Mean over the first 64 tokens only (a block, not the chunk)."""
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:64, h, :], axis=0).astype(np.float32).astype(np.float64)
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu[None, :])
        out[:, h, :] = _deq(codes, sc, kr.shape[0]) + mu[None, :]
    return out


def _q_with_mean_removed(qr):
    out = np.empty_like(qr)
    for h in range(qr.shape[1]):
        mu = np.mean(qr[:, h, :], axis=0)
        codes, sc = fp8_block_quantize(qr[:, h, :] - mu[None, :])
        out[:, h, :] = _deq(codes, sc, qr.shape[0])
    return out


def _q_one_block(qr):
    out = np.empty_like(qr)
    for h in range(qr.shape[1]):
        codes, sc = fp8_block_quantize(qr[:, h, :], block=qr.shape[0])
        out[:, h, :] = fp8_e4m3_decode(codes) * float(sc[0])
    return out


def _q_truncating(qr):
    """Codes rounded toward zero instead of to nearest."""
    from oracle.numerics import _MAGS
    out = np.empty_like(qr)
    for h in range(qr.shape[1]):
        x = qr[:, h, :]
        n = x.shape[0]
        sc = np.array([max(np.float32(np.max(np.abs(x[b:b + 64]))) / np.float32(448), np.float32(1e-30))
                       for b in range(0, n, 64)], dtype=np.float32)
        s = np.repeat(sc.astype(np.float64), 64)[:n, None]
        y = np.abs(x) / s
        idx = np.clip(np.searchsorted(_MAGS, y, side="right") - 1, 0, 0x7E)
        out[:, h, :] = np.sign(x) * _MAGS[idx] * s
    return out


def _context_across_chunks(w, k, live, clean, storage):
    """Blocks of 64 keys running through the whole context instead of
    restarting at each chunk."""
    Qs, ck, cv, ids = rotated_context(w, k, live, clean, "exact")
    if storage == "exact":
        return Qs, ck, cv, ids
    Qf, _, _, _ = rotated_context(w, k, live, clean, storage)
    T, N, h, d = ck.shape
    flat = ck.reshape(T * N, h, d)
    kf = oracle_round_mod._fp8_k(flat).reshape(T, N, h, d)
    return Qf, kf, cv, ids


@pytest.mark.parametrize("mutant", [_k_without_mean_readd, _k_mean_over_channels, _k_no_mean,
                                    _k_one_block_per_chunk, _k_scales_shifted, _k_mean_of_half],
                         ids=lambda f: f.__name__)
def test_planted_k_mistakes_fail_a_pin(mutant):
    failed = []
    for check in K_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, mutant.__name__ + " passed every K pin"


@pytest.mark.parametrize("mutant", [_q_with_mean_removed, _q_one_block, _q_truncating],
                         ids=lambda f: f.__name__)
def test_planted_q_mistakes_fail_a_pin(mutant):
    failed = []
    for check in Q_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, mutant.__name__ + " passed every Q pin"


def test_planted_context_mistake_fails_the_restart_pin():
    with pytest.raises(AssertionError):
        check_context_blocks_restart(_context_across_chunks)


def test_planted_mistakes_in_the_oracle_module_are_caught(monkeypatch):
    """The same pins through the module's own entry (store / rotated_context)
    with a mistake planted into the oracle module itself."""
    monkeypatch.setattr(oracle_round_mod, "_fp8_k", _k_without_mean_readd)
    with pytest.raises(AssertionError):
        check_context_blocks_restart(rotated_context)
    monkeypatch.setattr(oracle_round_mod, "_fp8_k", _k_one_block_per_chunk)
    with pytest.raises(AssertionError):
        check_context_blocks_restart(rotated_context)
