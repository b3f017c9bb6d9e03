"""CPU tests of the attention launch order (wf_attention_work_list): the host
logic that cuts (slot, head, query tile) units into one piece per XCD and
packs each piece onto that XCD's CUs. No device is involved."""
import dataclasses
import heapq
import math

import pytest

import wf_inputs as W
import wavefront_causal_attention_amd as wf
from _gpu_round import config_of

XCDS = 8


def _units(w, first, n):
    qt = math.ceil(w.N / 256)
    return {(s, h, q) for s in range(first, first + n) for h in range(w.heads) for q in range(qt)}


def _cost(w, s):
    return w.T if w.live_mask == "all" else w.T - s


def _run_cost(w, s, q):
    """The packer's run-time estimate: key chunks read, with the bf16 last
    query tile discounted to 0.6 when at most 4 of its 8 waves (32 rows each)
    hold rows of the chunk, since the others skip their compute."""
    qt = math.ceil(w.N / 256)
    tail_waves = math.ceil((w.N - (qt - 1) * 256) / 32)
    tail = w.qk_dtype == "bf16" and q == qt - 1 and tail_waves <= 4
    return _cost(w, s) * (0.6 if tail else 1.0)


def _ranges(S):
    return [(f, n) for f in range(S + 1) for n in range(1, S + 2 - f)]


@pytest.mark.parametrize("name", ["tiny", "ragged128", "edge_s1_h0", "wan1.3b_s4", "wan14b_s4", "max64",
                                  "slots62"])
def test_every_unit_listed_exactly_once(name):
    w = W.WORKLOADS[name]
    ranges = _ranges(w.S) if w.S < 8 else [(0, w.S + 1), (0, 1), (w.S, 1), (3, 11), (17, 14),
                                           (31, 2), (32, 1), (w.S - 20, 21)]
    ranges = [(f, n) for f, n in ranges if f + n <= w.S + 1]
    for first, n in ranges:
        lst = wf.wf_attention_work_list(config_of(w), first, n, 32)
        assert len(lst) % XCDS == 0
        got = [u for u in lst if u is not None]
        assert len(got) == len(set(got)) and set(got) == _units(w, first, n), (first, n)


@pytest.mark.parametrize("name,mask", [("wan1.3b_s4", "wavefront"), ("wan14b_s4", "wavefront"),
                                       ("wan1.3b_s5_30", "wavefront"), ("wan1.3b_s4", "all"),
                                       ("wan1.3b_s4_fp8", "wavefront")])
def test_xcd_pieces_balanced_and_packed_order_fills_the_cus(name, mask):
    """Each XCD's share of the key-chunk cost is within one unit of an
    eighth. Handing the XCD's entries in list order to whichever of its 32
    CUs frees first (the hardware dispatcher), with the packer's run-time
    estimates, ends within one unit of the average CU load, and for the
    wavefront mask's mixed unit costs keeps the CUs >= 96% busy: a CU takes
    only 3-4 units of 2.4-8 key chunks, so the span cannot come closer to the
    average load than a fraction of a unit (all-live units cost T or 0.6 T, so
    142.5 units on 32 CUs cannot either)."""
    w = dataclasses.replace(W.WORKLOADS[name], live_mask=mask)
    lst = wf.wf_attention_work_list(config_of(w), 0, w.S + 1, 32)
    per = [[u for b, u in enumerate(lst) if b % XCDS == x and u is not None] for x in range(XCDS)]
    loads = [sum(_cost(w, s) for s, _, _ in p) for p in per]
    total = sum(loads)
    umax = max(_cost(w, s) for s in range(w.S + 1))
    assert max(loads) - total / XCDS <= umax and total / XCDS - min(loads) <= umax
    for p in per:
        free = [0] * 32
        heapq.heapify(free)
        for s, _, q in p:
            heapq.heappush(free, heapq.heappop(free) + _run_cost(w, s, q))
        span = max(free)
        work = sum(_run_cost(w, s, q) for s, _, q in p)
        assert span <= work / 32 + umax
        if mask == "wavefront":
            assert work / (32 * span) >= 0.96, (name, work / (32 * span))


def test_work_list_validation():
    w = W.WORKLOADS["ragged128"]
    for args in [(-1, 1), (0, 0), (0, w.S + 2), (w.S, 2)]:
        with pytest.raises(wf.WfError) as e:
            wf.wf_attention_work_list(config_of(w), args[0], args[1], 32)
        assert e.value.status == wf.WF_E_INVALID_ARG
    with pytest.raises(wf.WfError) as e:
        wf.wf_attention_work_list(config_of(w), 0, 1, 0)
    assert e.value.status == wf.WF_E_INVALID_ARG


@pytest.mark.parametrize("S", [31, 32, 40, 62])
def test_slots_past_31_are_listed(S):
    """Slots 32..62 fill the top bits of a work entry: every (slot, head,
    query tile) of S+1 slots is listed once and none reads as padding."""
    w = dataclasses.replace(W.WORKLOADS["slots62"], S=S, H=62 - S)
    assert w.T == 64
    lst = wf.wf_attention_work_list(config_of(w), 0, w.S + 1, 32)
    got = [u for u in lst if u is not None]
    assert len(got) == len(set(got)) == (S + 1) * w.heads
    assert set(got) == _units(w, 0, S + 1)
    assert max(s for s, _, _ in got) == S
