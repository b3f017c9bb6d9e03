"""Pins of the oracle's attention: brute force, library routine, closed forms, invariants."""
import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import (RoundSchedule, dense_round_attention, legal_positions,
                    masked_softmax_attention, oracle_round, round_attention,
                    rotated_context, slot_position)


def _random_ctx(S, A, H, N, heads, d, seed=0):
    rng = np.random.default_rng(seed)
    T = A + H + S + 1
    Qs = rng.standard_normal((S + 1, N, heads, d))
    ck = rng.standard_normal((T, N, heads, d))
    cv = rng.standard_normal((T, N, heads, d))
    return Qs, ck, cv


@pytest.mark.parametrize("S,A,H", [(2, 1, 2), (1, 1, 1), (3, 1, 0), (4, 2, 1)])
def test_gather_equals_dense_masked(S, A, H):
    Qs, ck, cv = _random_ctx(S, A, H, 16, 2, 8, seed=S * 10 + H)
    a = round_attention(Qs, ck, cv, S, A, H)
    b = dense_round_attention(Qs, ck, cv, S, A, H)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_dense_mask_matches_mwf_tokenwise():
    S, A, H, N = 2, 1, 2, 4
    Qs, ck, cv = _random_ctx(S, A, H, N, 1, 4)
    _, ps, mask = dense_round_attention(Qs, ck, cv, S, A, H, return_p=True)
    T = A + H + S + 1
    for s in range(S + 1):
        for p in range(T):
            blk = mask[s * N:(s + 1) * N, p * N:(p + 1) * N]
            assert blk.all() == (p in legal_positions(s, S, A, H))
            assert blk.all() or not blk.any()        # full attention inside a chunk
    P = ps[0]
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(P[~mask] == 0.0)


@pytest.mark.parametrize("S", [1, 2])
def test_each_slot_equals_library_sdpa(S):
    A, H, N, heads, d = 1, 2, 24, 3, 16
    Qs, ck, cv = _random_ctx(S, A, H, N, heads, d, seed=7 + S)
    out = round_attention(Qs, ck, cv, S, A, H)
    for s in range(S + 1):
        pos = legal_positions(s, S, A, H)
        q = torch.from_numpy(Qs[s]).permute(1, 0, 2)                       # [heads, N, d]
        k = torch.from_numpy(np.concatenate([ck[p] for p in pos], 0)).permute(1, 0, 2)
        v = torch.from_numpy(np.concatenate([cv[p] for p in pos], 0)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).numpy()
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def test_store_row_is_plain_clean_history_attention():
    # S = 1: the store (slot 1) reads anchor + history + itself only
    S, A, H, N, heads, d = 1, 1, 2, 12, 1, 8
    Qs, ck, cv = _random_ctx(S, A, H, N, heads, d, seed=3)
    out = round_attention(Qs, ck, cv, S, A, H, slots=[S])
    kk = np.concatenate([ck[p][:, 0] for p in range(A + H + 1)], 0)
    vv = np.concatenate([cv[p][:, 0] for p in range(A + H + 1)], 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qs[S][:, 0])[None], torch.from_numpy(kk)[None], torch.from_numpy(vv)[None])[0]
    assert np.max(np.abs(out[0, :, 0] - ref.numpy())) <= 1e-12


def test_softmax_rows_sum_to_one_and_scale_is_inv_sqrt_d():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((6, 32)), rng.standard_normal((40, 32)), rng.standard_normal((40, 5))
    o, p = masked_softmax_attention(q, k, v, 1 / np.sqrt(32), return_p=True)
    assert np.max(np.abs(p.sum(1) - 1)) <= 1e-12
    # brute-force one row with Python loops
    r = 2
    sc = [sum(q[r, i] * k[j, i] for i in range(32)) / 32 ** 0.5 for j in range(40)]
    m = max(sc)
    e = [np.exp(x - m) for x in sc]
    z = sum(e)
    for c in range(5):
        assert abs(sum(e[j] / z * v[j, c] for j in range(40)) - o[r, c]) <= 1e-12


def test_noisier_slots_never_change_cleaner_outputs():
    S, A, H, N, heads, d = 3, 1, 2, 8, 2, 8
    Qs, ck, cv = _random_ctx(S, A, H, N, heads, d, seed=11)
    base = round_attention(Qs, ck, cv, S, A, H)
    for s in range(1, S + 1):
        k2, v2 = ck.copy(), cv.copy()
        for j in range(s):
            p = slot_position(j, S, A, H)
            k2[p] = np.nan
            v2[p] = np.nan
        pert = round_attention(Qs, k2, v2, S, A, H)
        assert np.array_equal(pert[s:], base[s:])           # bit-identical
        assert np.isnan(pert[:s]).all()                     # noisier ones do read them
        # dense formulation, finite perturbation: masked columns have weight exactly 0
        k3, v3 = ck.copy(), cv.copy()
        for j in range(s):
            p = slot_position(j, S, A, H)
            k3[p] += 1e3
            v3[p] -= 7.0
        dn = dense_round_attention(Qs, k3, v3, S, A, H)
        db = dense_round_attention(Qs, ck, cv, S, A, H)
        assert np.array_equal(dn[s:], db[s:])


def test_zero_query_reads_exactly_the_legal_chunks():
    # Q = 0 gives uniform weights, so O_s is the mean of V over L(s). With V
    # constant per chunk (its chunk id) the result is an exact rational.
    for S, A, H in [(4, 1, 2), (5, 1, 2), (4, 1, 3), (2, 1, 2)]:
        N, heads, d = 6, 2, 4
        T = A + H + S + 1
        k = S + H + A + 3
        ids = RoundSchedule(S, A, H, k).chunk_ids()
        Qs = np.zeros((S + 1, N, heads, d))
        ck = np.random.default_rng(1).standard_normal((T, N, heads, d))
        cv = np.stack([np.full((N, heads, d), float(ids[p])) for p in range(T)])
        out = round_attention(Qs, ck, cv, S, A, H)
        for s in range(S + 1):
            legal = [ids[p] for p in range(T) if p in legal_positions(s, S, A, H)]
            assert len(legal) == A + H + S + 1 - s
            assert np.max(np.abs(out[s] - sum(legal) / len(legal))) <= 1e-12


def test_constant_values_pass_through():
    S, A, H, N, heads, d = 2, 1, 2, 8, 2, 16
    Qs, ck, _ = _random_ctx(S, A, H, N, heads, d, seed=4)
    cv = np.full(ck.shape, -2.375)
    out = round_attention(Qs, ck, cv, S, A, H)
    assert np.max(np.abs(out + 2.375)) <= 1e-12


def test_tiny_round_end_to_end_consistency():
    # full pipeline on the tiny workload: gather == dense, finite, bf16 vs exact close
    w = W.WORKLOADS["tiny"]
    k = w.steady_round + 1
    live = [W.draw(w, k, s) for s in range(w.S + 1)]
    sch = RoundSchedule(w.S, w.A, w.H, k)
    clean = {c: W.stored_draw(w, c)[1:] for c in sch.chunk_ids()[:w.A + w.H]}
    Qs, ck, cv, ids = rotated_context(w, k, live, clean, storage="exact")
    a = round_attention(Qs, ck, cv, w.S, w.A, w.H)
    b = dense_round_attention(Qs, ck, cv, w.S, w.A, w.H)
    assert np.max(np.abs(a - b)) <= 1e-12
    ob = oracle_round(w, k, live, clean, storage="bf16")
    rel = np.linalg.norm(ob - a) / np.linalg.norm(a)
    assert 0 < rel < 5e-3


def test_rope_positions_follow_the_schedule():
    # Q = K = a on every even time-axis channel: after RoPE the score of query
    # frame t_q against key frame t_k is a^2 * sum_m cos((t_q - t_k) w_m)/sqrt(d),
    # uniquely largest at t_k = t_q. With a large a the softmax picks the
    # query's own latent frame, i.e. its own chunk; V = chunk id then returns
    # the chunk id each slot was rotated as.
    w = W.WORKLOADS["ragged64"]
    k = w.steady_round + 2
    sch = RoundSchedule(w.S, w.A, w.H, k)
    d_t = w.rope_split[0]
    pat = np.zeros(w.head_dim)
    pat[0:d_t:2] = 40.0
    qk = np.tile(pat, (w.N, w.heads))

    def chunk(cid):
        return qk.copy(), qk.copy(), np.full((w.N, w.hd), float(cid))

    live = [chunk(sch.slot_chunk(s)) for s in range(w.S + 1)]
    clean = {c: chunk(c)[1:] for c in sch.chunk_ids()[:w.A + w.H]}
    out = oracle_round(w, k, live, clean, storage="exact")
    for s in range(w.S + 1):
        assert np.max(np.abs(out[s] - sch.slot_chunk(s))) <= 1e-9, s


# --- the all-live mask (bidirectional live K/V, the Rolling Forcing contrast) ---

@pytest.mark.parametrize("S,A,H", [(2, 1, 2), (3, 1, 0), (4, 2, 1)])
def test_all_live_gather_equals_dense(S, A, H):
    Qs, ck, cv = _random_ctx(S, A, H, 12, 2, 8, seed=100 + S)
    a = round_attention(Qs, ck, cv, S, A, H, kind="all")
    b = dense_round_attention(Qs, ck, cv, S, A, H, kind="all")
    assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("S", [1, 3])
def test_all_live_each_slot_is_sdpa_over_the_whole_context(S):
    # every slot attends to every context position: plain library attention
    # over the concatenation of all T chunks, no mask
    A, H, N, heads, d = 1, 1, 20, 2, 16
    Qs, ck, cv = _random_ctx(S, A, H, N, heads, d, seed=200 + S)
    T = A + H + S + 1
    out = round_attention(Qs, ck, cv, S, A, H, kind="all")
    k = torch.from_numpy(ck.reshape(T * N, heads, d)).permute(1, 0, 2)
    v = torch.from_numpy(cv.reshape(T * N, heads, d)).permute(1, 0, 2)
    for s in range(S + 1):
        q = torch.from_numpy(Qs[s]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).numpy()
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def test_noisiest_slot_reads_the_same_under_both_masks():
    # M_WF(0, j) = 1 for every live j, so slot 0 already sees everything
    S, A, H = 3, 1, 2
    Qs, ck, cv = _random_ctx(S, A, H, 10, 2, 8, seed=300)
    wf_ = round_attention(Qs, ck, cv, S, A, H)
    al = round_attention(Qs, ck, cv, S, A, H, kind="all")
    assert np.array_equal(wf_[0], al[0])
    assert all(np.max(np.abs(wf_[s] - al[s])) > 1e-3 for s in range(1, S + 1))


@pytest.mark.parametrize("S,A,H,C", [(2, 1, 2, 5), (3, 2, 1, 6)])
def test_fill_and_drain_rounds_read_exactly_the_present_chunks(S, A, H, C):
    # Q = 0 gives uniform weights, V = chunk id: each present slot's output is
    # the exact mean of the ids of the chunks it reads, which a brute-force
    # pipeline fixes (stage k - i for chunk i, clean after its store round)
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["tiny"], S=S, A=A, H=H, heads=1)
    N, hd = w.N, w.hd
    for k in range(C + S):
        sch = RoundSchedule(S, A, H, k, fill=True, total_chunks=C)
        live = [None if not sch.slot_present(s) else
                (np.zeros((N, hd)), np.zeros((N, hd)), np.full((N, hd), float(k - s))) for s in range(S + 1)]
        stored = [i for i in range(C) if i + S + 1 <= k]
        clean = {i: (np.zeros((N, hd)), np.full((N, hd), float(i))) for i in stored}
        out = oracle_round(w, k, live, clean, storage="exact", fill=True, total_chunks=C)
        hist = [i for i in stored if i >= A][-H:] if H else []
        anchors = [i for i in stored if i < A]
        for s in range(S + 1):
            if not sch.slot_present(s):
                assert np.isnan(out[s]).all()
                continue
            reads = anchors + hist + [k - j for j in range(s, S + 1) if 0 <= k - j <= C - 1]
            assert np.max(np.abs(out[s] - np.mean(reads))) <= 1e-12, (k, s)
