"""Pins of the oracle's schedule model and mask structure (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import GroupRing, RoundSchedule, legal_positions, live_mask, slot_position

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_mask_is_lower_triangular_in_context_order():
    # M_WF(s, j) = 1[j >= s]; listing the live slots cleanest first
    # (store, slot S-1, ..., slot 0) makes it the lower-triangular ones matrix.
    for S in (1, 2, 4, 5):
        M = live_mask(S)
        order = list(range(S, -1, -1))                   # cleanest first
        Mc = M[np.ix_(order, order)]
        assert np.array_equal(Mc, np.tril(np.ones((S + 1, S + 1), dtype=np.int64)))
    # literal S = 2 matrix in slot order [s][j]
    assert live_mask(2).tolist() == [[1, 1, 1], [0, 1, 1], [0, 0, 1]]


def test_legal_context_is_prefix_and_clean_parts_visible_to_all():
    for S, A, H in [(2, 1, 2), (4, 1, 2), (5, 1, 2), (4, 1, 3), (1, 1, 0), (3, 2, 1)]:
        T = A + H + S + 1
        for s in range(S + 1):
            pos = legal_positions(s, S, A, H)
            assert pos == list(range(T - s)), (S, A, H, s)
            assert set(range(A + H)) <= set(pos)           # anchor + history read by all
            assert slot_position(s, S, A, H) in pos         # itself
            for j in range(s):                              # never a noisier slot
                assert slot_position(j, S, A, H) not in pos


def test_store_reads_smallest_context_noisiest_reads_all():
    S, A, H = 4, 1, 2
    sizes = [len(legal_positions(s, S, A, H)) for s in range(S + 1)]
    assert sizes == [8, 7, 6, 5, 4]
    assert sizes[0] == A + H + S + 1


def test_round_schedule_k_equals_i_plus_s():
    S, A, H = 4, 1, 2
    sch = RoundSchedule(S, A, H, 7)
    # anchor 0 | hist 1, 2 | store 3 | slots 3, 2, 1, 0 hold chunks 4, 5, 6, 7
    assert sch.chunk_ids() == [0, 1, 2, 3, 4, 5, 6, 7]
    for k in range(7, 20):
        sch = RoundSchedule(S, A, H, k)
        for s in range(S + 1):
            assert sch.slot_chunk(s) + s == k
    with pytest.raises(ValueError):
        RoundSchedule(S, A, H, 6)


def test_fig1_one_chunk_per_round_after_fill():
    g = json.load(open(os.path.join(GOLD, "fig1_wavefront_s4.json")))
    S, A, H = g["S"], 1, 2
    k0 = S + H + A
    emitted = [RoundSchedule(S, A, H, k).chunk_at(A + H) for k in range(k0, k0 + g["rounds_observed"])]
    assert len(set(emitted)) == g["chunks_emitted"]
    assert emitted == list(range(emitted[0], emitted[0] + g["chunks_emitted"]))
    # each chunk visits stages 0..S (store) in consecutive rounds
    c = k0 + 3
    stages = []
    for k in range(c, c + S + 1):
        sch = RoundSchedule(S, A, H, max(k, k0))
        stages.append([s for s in range(S + 1) if sch.slot_chunk(s) == c])
    assert stages == [[s] for s in range(g["stages_per_chunk"])]


def test_group_ring_relabels_without_copy():
    S, A, H = 4, 1, 2
    T = A + H + S + 1
    ring = GroupRing(S, A, H)
    k0 = S + H + A
    # which chunk each physical group holds, starting from a full round k0
    held = {g: RoundSchedule(S, A, H, k0).chunk_at(p) for p, g in enumerate(ring.groups())}
    for step in range(3 * (H + S + 1)):
        k = k0 + step
        groups = ring.groups()
        assert sorted(groups) == list(range(T))                      # a permutation
        assert groups[:A] == list(range(A))                          # anchor fixed
        sch = RoundSchedule(S, A, H, k)
        # every position holds the chunk the schedule names; anchor and history
        # were never re-published, so they got there by relabelling alone
        for p in range(T):
            assert held[groups[p]] == sch.chunk_at(p), (step, p)
        ring.advance()
        g2 = ring.groups()
        # relabelling: the group at position p-1 now is the one that was at p
        for p in range(A + 1, T):
            assert g2[p - 1] == groups[p]
        # the next round re-publishes every live slot (store included)
        nxt = RoundSchedule(S, A, H, k + 1)
        for s in range(S + 1):
            held[g2[slot_position(s, S, A, H)]] = nxt.slot_chunk(s)


def test_table8_chunk_bytes():
    g = json.load(open(os.path.join(GOLD, "table8_ipc_copy.json")))
    shapes = json.load(open(os.path.join(GOLD, "table11_shapes.json")))["models"]
    N = 3 * 30 * 52                                   # 3 latent frames of 30x52 patches
    assert N == g["chunk_tokens"]
    hidden = shapes["14B"]["hidden"]
    assert N * hidden * 2 * 2 == g["bytes"]           # bf16 K and V of one chunk
    # head_dim 128 for both standard Wan2.1 models
    assert shapes["1.3B"]["hidden"] // shapes["1.3B"]["heads"] == 128
    assert shapes["14B"]["hidden"] // shapes["14B"]["heads"] == 128


def test_all_live_mask_is_all_ones_and_every_slot_reads_everything():
    for S in (1, 2, 4):
        assert (live_mask(S, "all") == 1).all()
        A, H = 1, 2
        T = A + H + S + 1
        for s in range(S + 1):
            assert legal_positions(s, S, A, H, "all") == list(range(T))
    with pytest.raises(ValueError):
        live_mask(2, "rolling")


# --- fill and drain rounds ---------------------------------------------------

def _pipeline(S, A, H, C, k):
    """Brute force: follow every chunk through the pipeline to round k.
    Chunk i is at stage k - i while 0 <= k - i <= S (stage S is the store) and
    is clean from round i + S + 1 on: an anchor if i < A, else it joins the
    history, which keeps the H most recently stored non-anchor chunks."""
    stage = {i: k - i for i in range(C) if 0 <= k - i <= S}
    stored = [i for i in range(C) if i + S + 1 <= k]
    anchors = sorted(i for i in stored if i < A)
    hist = [i for i in stored if i >= A][-H:] if H else []
    return stage, anchors, hist


@pytest.mark.parametrize("S,A,H,C", [(2, 1, 2, 6), (4, 1, 2, 9), (3, 2, 1, 7), (1, 1, 0, 4), (4, 2, 3, 3)])
def test_fill_and_drain_presence_matches_the_pipeline(S, A, H, C):
    T = A + H + S + 1
    for k in range(C + S):                                   # every round of a C-chunk video
        sch = RoundSchedule(S, A, H, k, fill=True, total_chunks=C)
        stage, anchors, hist = _pipeline(S, A, H, C, k)
        ids = sch.present_chunk_ids()
        live = {s: c for c, s in stage.items()}
        for s in range(S + 1):
            p = slot_position(s, S, A, H)
            assert (ids[p] is not None) == (s in live)
            if s in live:
                assert ids[p] == live[s]
        assert [ids[a] for a in range(A) if ids[a] is not None] == anchors
        assert sorted(c for c in ids[A:A + H] if c is not None) == hist
        for s in range(S + 1):                               # what each present slot reads
            if s not in live:
                continue
            got = sorted(ids[p] for p in sch.legal_present(s))
            want = sorted(anchors + hist + [c for c, st in stage.items() if st >= s])
            assert got == want, (k, s)
    with pytest.raises(ValueError):
        RoundSchedule(S, A, H, C + S, fill=True, total_chunks=C)


def test_steady_rounds_have_every_position():
    S, A, H = 4, 1, 2
    for k in range(S + H + A, S + H + A + 10):
        sch = RoundSchedule(S, A, H, k, fill=True)
        assert all(sch.present(p) for p in range(sch.T))
        assert sch.present_chunk_ids() == sch.chunk_ids()


def test_fig1_first_output_after_fill():
    # Figure 1 caption (S=4): the first chunk is emitted after the pipeline
    # fills, then one chunk per round
    g = json.load(open(os.path.join(GOLD, "fig1_wavefront_s4.json")))
    S, A, H = g["S"], 1, 2
    stored = []
    for k in range(S + g["rounds_observed"]):
        sch = RoundSchedule(S, A, H, k, fill=True)
        stored.append(sch.present_chunk_ids()[A + H])
    assert stored[:S] == [None] * S
    assert stored[S:] == list(range(g["chunks_emitted"]))
