"""Pins of the oracle's 3D RoPE: invariants and a library 1D rotary special case."""
import numpy as np
import pytest
import torch

from oracle import rope_3d, rope_split, token_grid


def test_split_widths():
    assert rope_split(128) == (44, 42, 42)
    assert rope_split(64) == (24, 20, 20)
    for d in (64, 96, 128, 256):
        t, h, w = rope_split(d)
        assert t + h + w == d and t % 2 == h % 2 == w % 2 == 0
    with pytest.raises(ValueError):
        rope_split(128, (44, 42, 40))


def test_token_grid_matches_nested_loops():
    F, Hp, Wp, cid = 3, 5, 7, 4
    t, y, x = token_grid(cid, F, Hp, Wp)
    n = 0
    for f in range(F):
        for yy in range(Hp):
            for xx in range(Wp):
                assert (t[n], y[n], x[n]) == (F * cid + f, yy, xx)
                n += 1
    assert n == len(t)


def _rand(N, heads, d, seed=0):
    return np.random.default_rng(seed).standard_normal((N, heads, d))


def test_norm_preserved_and_zero_position_identity():
    split = rope_split(128)
    v = _rand(50, 3, 128)
    rng = np.random.default_rng(2)
    t, y, x = rng.integers(0, 4000, 50), rng.integers(0, 30, 50), rng.integers(0, 52, 50)
    r = rope_3d(v, t, y, x, split, 1e4)
    assert np.max(np.abs(np.linalg.norm(r, axis=-1) - np.linalg.norm(v, axis=-1))) <= 1e-12
    z = np.zeros(50, dtype=np.int64)
    assert np.max(np.abs(rope_3d(v, z, z, z, split, 1e4) - v)) == 0.0


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_relative_position_invariance_per_axis(axis):
    split = rope_split(128)
    q, k = _rand(20, 2, 128, 1), _rand(20, 2, 128, 2)
    rng = np.random.default_rng(3)
    pq = [rng.integers(0, 100, 20) for _ in range(3)]
    pk = [rng.integers(0, 100, 20) for _ in range(3)]
    base = np.sum(rope_3d(q, *pq, split, 1e4) * rope_3d(k, *pk, split, 1e4), axis=-1)
    pq2 = [p.copy() for p in pq]
    pk2 = [p.copy() for p in pk]
    pq2[axis] += 37
    pk2[axis] += 37
    shifted = np.sum(rope_3d(q, *pq2, split, 1e4) * rope_3d(k, *pk2, split, 1e4), axis=-1)
    assert np.max(np.abs(base - shifted)) <= 1e-10
    # a one-sided shift does change it
    pq3 = [p.copy() for p in pq]
    pq3[axis] += 37
    moved = np.sum(rope_3d(q, *pq3, split, 1e4) * rope_3d(k, *pk, split, 1e4), axis=-1)
    assert np.max(np.abs(base - moved)) > 1e-3


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_single_axis_equals_library_interleaved_rotary(axis):
    # Positions on one axis only reduce the 3D embedding to the interleaved
    # (rotate-every-two) 1D rotary on that axis's channel range, which
    # transformers ships for GPT-J (base 10000, fp32).
    from transformers.models.gptj import modeling_gptj as g
    d = 128
    split = rope_split(d)
    off = sum(split[:axis])
    da = split[axis]
    N = 64
    v = _rand(N, 1, d, 9)
    pos = np.arange(N, dtype=np.int64) * 3
    zero = np.zeros(N, dtype=np.int64)
    ps = [zero, zero, zero]
    ps[axis] = pos
    ours = rope_3d(v, *ps, split, 1e4)
    table = g.create_sinusoidal_positions(int(pos.max()) + 1, da)          # [pos, sin|cos]
    sincos = table[torch.from_numpy(pos)]
    sin, cos = torch.split(sincos, da // 2, dim=-1)
    x = torch.from_numpy(v[:, :, off:off + da]).float()[None]               # [1, N, 1, da]
    ref = g.apply_rotary_pos_emb(x, sin[None], cos[None])[0].double().numpy()
    assert np.max(np.abs(ours[:, :, off:off + da] - ref)) <= 2e-4
    # every other channel is untouched
    rest = np.ones(d, dtype=bool)
    rest[off:off + da] = False
    assert np.array_equal(ours[:, :, rest], v[:, :, rest])
