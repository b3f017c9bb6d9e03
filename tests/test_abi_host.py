"""CPU tests of libwf.so: exports, validation, schedule, page table and
readiness, through the C ABI on host-model handles (no device calls)."""
import os
import re

import numpy as np
import pytest

import wf_inputs as W
import wavefront_causal_attention_amd as wf
from wavefront_causal_attention_amd import _lib
from oracle import GroupRing, RoundSchedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20            # an aligned non-null address; host-model calls never touch it


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return wf.load()


def cfg_of(w, **kw):
    from _gpu_round import config_of
    return config_of(w, **kw)


def test_every_declared_symbol_is_exported(lib):
    header = open(os.path.join(ROOT, "include", "wf.h")).read()
    declared = set(re.findall(r"\b(wf_[a-z0-9_]+)\s*\(", header))
    assert {"wf_kv_publish", "wf_attention_round", "wf_round_advance"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(_lib.EXPORTED) == declared


def test_status_strings(lib):
    names = [_lib.status_string(st) for st in range(5)]
    assert all(names) and len(set(names)) == 5


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_pool_bytes_cover_pages(lib, name):
    w = W.WORKLOADS[name]
    pb, tb = wf.wf_pool_bytes(cfg_of(w))
    elems = w.T * w.N * w.heads * w.head_dim
    kbytes = elems * (1 if w.qk_dtype == "fp8" else 2)
    assert pb >= kbytes + 2 * elems
    assert tb == w.T * (w.N // w.page_tokens) * 4


def test_wan13b_pool_size_matches_pages(lib):
    w = W.WORKLOADS["wan1.3b_s4"]
    pb, _ = wf.wf_pool_bytes(cfg_of(w))
    # 8 chunks x 4680 tokens x 1536 channels x bf16, K and V = 230,031,360 B,
    # plus under 1 MiB of RoPE tables and attention work lists
    assert 8 * 4680 * 1536 * 2 * 2 == 230031360
    assert 230031360 <= pb < 230031360 + (1 << 20)


@pytest.mark.parametrize("field,value,status", [
    ("S", 0, wf.WF_E_SHAPE), ("anchor_chunks", 0, wf.WF_E_SHAPE), ("history_chunks", -1, wf.WF_E_SHAPE),
    ("head_dim", 96, wf.WF_E_SHAPE), ("heads", 0, wf.WF_E_SHAPE), ("num_layers", 0, wf.WF_E_SHAPE),
    ("page_tokens", 100, wf.WF_E_SHAPE), ("page_tokens", 4, wf.WF_E_SHAPE),
    ("in_dtype", 7, wf.WF_E_INVALID_ARG), ("qk_dtype", 1, wf.WF_E_INVALID_ARG),
    ("first_round", -1, wf.WF_E_SHAPE), ("total_chunks", -1, wf.WF_E_SHAPE),
    ("rope_theta", 0.0, wf.WF_E_INVALID_ARG),
    ("S", 70, wf.WF_E_SHAPE), ("live_mask", 2, wf.WF_E_INVALID_ARG),
])
def test_config_validation(lib, field, value, status):
    # wan1.3b_s4 bench config: first_round 7 (first full round), unbounded video
    c = cfg_of(W.WORKLOADS["wan1.3b_s4"])
    setattr(c, field, value)
    with pytest.raises(wf.WfError) as e:
        wf.wf_pool_bytes(c)
    assert e.value.status == status


def test_fp8_tile_scale_table_limit(lib):
    # fp8 attention tiles every chunk into its 64-token quantisation blocks and
    # stages one key scale per tile of the context (at most 4096) in LDS
    import dataclasses
    w = W.WORKLOADS["wan1.3b_s4_fp8"]                       # T = 8
    fits = dataclasses.replace(w, chunk_frames=21)          # 32760 tokens: 8 x 512 tiles
    wf.wf_pool_bytes(cfg_of(fits))
    big = dataclasses.replace(w, chunk_frames=22)           # 34320 tokens: 8 x 537 tiles
    with pytest.raises(wf.WfError) as e:
        wf.wf_pool_bytes(cfg_of(big))
    assert e.value.status == wf.WF_E_SHAPE
    c = cfg_of(big)
    c.qk_dtype = wf.WF_DTYPE_BF16                            # bf16 has no such table
    wf.wf_pool_bytes(c)
    small = dataclasses.replace(W.WORKLOADS["ragged_fp8_64"], chunk_frames=1, frame_h=4, frame_w=6,
                                page_tokens=24)             # a chunk shorter than one tile
    wf.wf_pool_bytes(cfg_of(small))


def test_bad_rope_split(lib):
    c = cfg_of(W.WORKLOADS["wan1.3b_s4"])
    c.rope_split[2] = 40
    with pytest.raises(wf.WfError) as e:
        wf.wf_pool_bytes(c)
    assert e.value.status == wf.WF_E_SHAPE


def test_undersized_buffers_rejected_before_any_device_access(lib):
    c = cfg_of(W.WORKLOADS["ragged128"])
    pb, tb = wf.wf_pool_bytes(c)
    for args in [(pb - 1, tb), (pb, tb - 4)]:
        with pytest.raises(wf.WfError) as e:
            wf.wf_pool_create(c, FAKE, args[0], FAKE, args[1])
        assert e.value.status == wf.WF_E_SHAPE
    with pytest.raises(wf.WfError) as e:
        wf.wf_pool_create(c, FAKE + 16, pb, FAKE, tb)          # pool not 256-byte aligned
    assert e.value.status == wf.WF_E_INVALID_ARG


@pytest.mark.parametrize("name", ["wan1.3b_s4", "wan1.3b_s5_30", "wan14b_s4", "tiny", "edge_s1_h0"])
def test_schedule_and_page_table_closed_form(lib, name):
    w = W.WORKLOADS[name]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    ring = GroupRing(w.S, w.A, w.H)
    ppc = w.N // w.page_tokens
    try:
        for step in range(3 * (w.H + w.S + 1) + 1):
            k = w.steady_round + step
            assert wf.wf_round_index(h) == k
            assert wf.wf_schedule_chunk_ids(h, w.T) == RoundSchedule(w.S, w.A, w.H, k).chunk_ids()
            table = wf.wf_page_table_host(h, w.T * ppc)
            assert table == [g * ppc + i for g in ring.groups() for i in range(ppc)]
            assert sorted(table) == list(range(w.T * ppc))           # a permutation of the pages
            # every live slot and the store publish, then the round ends
            wf.wf_kv_publish(h, 0, 0, w.S + 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
            wf.wf_round_advance(h, None)
            ring.advance()
    finally:
        wf.wf_pool_destroy(h)


def test_readiness_and_failure_forcing(lib):
    w = W.WORKLOADS["wan1.3b_s4"]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    T, S, A, H = w.T, w.S, w.A, w.H
    try:
        # nothing published: attention and advance refuse
        for call in (lambda: wf.wf_attention_round(h, 0, 0, S + 1, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None),
                     lambda: wf.wf_round_advance(h, None)):
            with pytest.raises(wf.WfError) as e:
                call()
            assert e.value.status == wf.WF_E_NOT_READY
        # clean positions (slots S+1..T-1) published with K/V only
        wf.wf_kv_publish(h, 0, S + 1, T - S - 1, None, FAKE, FAKE, w.hd, None, None, None, None)
        assert wf.wf_ready_mask(h, 0) == (1 << (A + H)) - 1
        # the store alone makes slot S attendable, not slot S-1
        wf.wf_kv_publish(h, 0, S, 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)
        wf.wf_attention_round(h, 0, S, 1, FAKE, None, FAKE, wf.WF_DTYPE_BF16, None)
        with pytest.raises(wf.WfError) as e:
            wf.wf_attention_round(h, 0, S - 1, 2, FAKE, None, FAKE, wf.WF_DTYPE_BF16, None)
        assert e.value.status == wf.WF_E_NOT_READY
        # slots 1..S-1: slot 1 is attendable, slot 0 is not
        wf.wf_kv_publish(h, 0, 1, S - 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)
        wf.wf_attention_round(h, 0, 1, S, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None)
        with pytest.raises(wf.WfError) as e:
            wf.wf_attention_round(h, 0, 0, S + 1, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None)
        assert e.value.status == wf.WF_E_NOT_READY
        wf.wf_kv_publish(h, 0, 0, 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)
        wf.wf_attention_round(h, 0, 0, S + 1, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None)
        assert wf.wf_ready_mask(h, 0) == (1 << T) - 1
        # advance: history and anchor stay published, live slots need re-publishing
        wf.wf_round_advance(h, None)
        assert wf.wf_ready_mask(h, 0) == (1 << (A + H)) - 1
        with pytest.raises(wf.WfError) as e:
            wf.wf_round_advance(h, None)
        assert e.value.status == wf.WF_E_NOT_READY
        assert wf.wf_round_index(h) == w.steady_round + 1
    finally:
        wf.wf_pool_destroy(h)


def test_store_required_in_every_layer(lib):
    w = W.WORKLOADS["ragged128"]
    h = wf.wf_pool_create_host_model(cfg_of(w, num_layers=3))
    try:
        for layer in (0, 1):
            wf.wf_kv_publish(h, layer, 0, w.S + 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)
        with pytest.raises(wf.WfError) as e:
            wf.wf_round_advance(h, None)
        assert e.value.status == wf.WF_E_NOT_READY
        wf.wf_kv_publish(h, 2, w.S, 1, None, FAKE, FAKE, w.hd, None, None, None, None)
        wf.wf_round_advance(h, None)
    finally:
        wf.wf_pool_destroy(h)


@pytest.mark.parametrize("args", [
    dict(layer=1), dict(layer=-1), dict(slot_first=-1), dict(nslots=0), dict(nslots=9),
    dict(k=None), dict(v=None), dict(stride=100), dict(q_out=None),
    dict(slot_first=4, nslots=2),          # q given but range includes a clean slot
    dict(q=FAKE + 2),                      # misaligned
])
def test_publish_invalid_args(lib, args):
    w = W.WORKLOADS["wan1.3b_s4"]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    a = dict(layer=0, slot_first=0, nslots=w.S + 1, q=FAKE, k=FAKE, v=FAKE, stride=w.hd, q_out=FAKE)
    a.update(args)
    try:
        with pytest.raises(wf.WfError) as e:
            wf.wf_kv_publish(h, a["layer"], a["slot_first"], a["nslots"], a["q"], a["k"], a["v"],
                             a["stride"], None, a["q_out"], None, None)
        assert e.value.status == wf.WF_E_INVALID_ARG
        assert wf.wf_ready_mask(h, 0) == 0               # nothing changed
    finally:
        wf.wf_pool_destroy(h)


@pytest.mark.parametrize("noalloc", [False, True])
def test_publish_noalloc_checks_like_publish_and_bounds_its_scratch(lib, noalloc):
    """wf_kv_publish_noalloc takes wf_kv_publish's arguments and checks; on an
    fp8 pool whose K-mean block sums (nslots * heads * ceil(N/64) * d * 8
    bytes) exceed its static 16 MiB array it returns WF_E_SHAPE, launches
    nothing and marks nothing published; bf16 pools need no scratch."""
    import dataclasses
    w = W.WORKLOADS["wan1.3b_s4_fp8"]
    big = dataclasses.replace(w, heads=48)            # 5 slots x 48 heads x 74 blocks x 1 KiB > 16 MiB
    h = wf.wf_pool_create_host_model(cfg_of(big))
    try:
        args = (h, 0, 0, big.S + 1, FAKE, FAKE, FAKE, 3 * big.hd, None, FAKE, FAKE, None)
        if noalloc:
            with pytest.raises(wf.WfError) as e:
                wf.wf_kv_publish(*args, noalloc=True)
            assert e.value.status == wf.WF_E_SHAPE and "scratch" in str(e.value)
            assert wf.wf_ready_mask(h, 0) == 0
            # a smaller range fits: 2 slots x 48 heads x 74 blocks x 1 KiB
            wf.wf_kv_publish(h, 0, 0, 2, FAKE, FAKE, FAKE, 3 * big.hd, None, FAKE, FAKE, None, noalloc=True)
            assert wf.wf_ready_mask(h, 0) == sum(1 << (big.T - 1 - s) for s in range(2))
        else:
            wf.wf_kv_publish(*args)
        with pytest.raises(wf.WfError) as e:           # the shared argument checks
            wf.wf_kv_publish(h, 1, 0, 1, FAKE, FAKE, FAKE, 3 * big.hd, None, FAKE, FAKE, None, noalloc=noalloc)
        assert e.value.status == wf.WF_E_INVALID_ARG
    finally:
        wf.wf_pool_destroy(h)
    hb = wf.wf_pool_create_host_model(cfg_of(dataclasses.replace(W.WORKLOADS["wan1.3b_s4"], heads=64)))
    try:
        wf.wf_kv_publish(hb, 0, 0, 5, FAKE, FAKE, FAKE, 64 * 128, None, FAKE, None, None, noalloc=noalloc)
    finally:
        wf.wf_pool_destroy(hb)


@pytest.mark.parametrize("args", [
    dict(layer=2), dict(slot_first=5), dict(nslots=6), dict(q=None), dict(out=None),
    dict(out_dtype=wf.WF_DTYPE_FP8_E4M3), dict(out=FAKE + 8),
])
def test_attention_invalid_args(lib, args):
    w = W.WORKLOADS["wan1.3b_s4"]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    wf.wf_kv_publish(h, 0, w.S + 1, w.T - w.S - 1, None, FAKE, FAKE, w.hd, None, None, None, None)
    wf.wf_kv_publish(h, 0, 0, w.S + 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)
    a = dict(layer=0, slot_first=0, nslots=w.S + 1, q=FAKE, out=FAKE, out_dtype=wf.WF_DTYPE_FP32)
    a.update(args)
    try:
        with pytest.raises(wf.WfError) as e:
            wf.wf_attention_round(h, a["layer"], a["slot_first"], a["nslots"], a["q"], None,
                                  a["out"], a["out_dtype"], None)
        assert e.value.status == wf.WF_E_INVALID_ARG
    finally:
        wf.wf_pool_destroy(h)


def test_explicit_rope_offsets_validated(lib):
    w = W.WORKLOADS["tiny"]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    try:
        with pytest.raises(wf.WfError) as e:
            wf.wf_kv_publish(h, 0, 0, 1, FAKE, FAKE, FAKE, w.hd, [-3], FAKE, None, None)
        assert e.value.status == wf.WF_E_INVALID_ARG
        wf.wf_kv_publish(h, 0, 0, 2, FAKE, FAKE, FAKE, w.hd, [5, 6], FAKE, None, None)
    finally:
        wf.wf_pool_destroy(h)


def test_all_live_attention_needs_the_whole_context(lib):
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["wan1.3b_s4"], live_mask="all")
    h = wf.wf_pool_create_host_model(cfg_of(w))
    T, S = w.T, w.S
    try:
        # clean positions and the store only: under M_WF the store would be
        # ready, under the all-live mask it reads every live slot too
        wf.wf_kv_publish(h, 0, S + 1, T - S - 1, None, FAKE, FAKE, w.hd, None, None, None, None)
        wf.wf_kv_publish(h, 0, S, 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
        with pytest.raises(wf.WfError) as e:
            wf.wf_attention_round(h, 0, S, 1, FAKE, FAKE, FAKE, wf.WF_DTYPE_BF16, None)
        assert e.value.status == wf.WF_E_NOT_READY
        wf.wf_kv_publish(h, 0, 0, S, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
        wf.wf_attention_round(h, 0, S, 1, FAKE, FAKE, FAKE, wf.WF_DTYPE_BF16, None)
        assert wf.wf_ready_mask(h, 0) == (1 << T) - 1
    finally:
        wf.wf_pool_destroy(h)
    # the wavefront mask accepts the store with only its prefix published
    h = wf.wf_pool_create_host_model(cfg_of(W.WORKLOADS["wan1.3b_s4"]))
    try:
        wf.wf_kv_publish(h, 0, S + 1, T - S - 1, None, FAKE, FAKE, w.hd, None, None, None, None)
        wf.wf_kv_publish(h, 0, S, 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
        wf.wf_attention_round(h, 0, S, 1, FAKE, FAKE, FAKE, wf.WF_DTYPE_BF16, None)
    finally:
        wf.wf_pool_destroy(h)


def test_first_round_past_the_video_is_rejected(lib):
    c = cfg_of(W.WORKLOADS["wan1.3b_s4"], first_round=10)
    c.total_chunks = 7                         # last round 7 - 1 + S = 10
    wf.wf_pool_bytes(c)
    c.first_round = 11
    with pytest.raises(wf.WfError) as e:
        wf.wf_pool_bytes(c)
    assert e.value.status == wf.WF_E_SHAPE


@pytest.mark.parametrize("S,A,H,C", [(2, 1, 2, 6), (4, 1, 2, 9), (3, 2, 1, 7), (2, 2, 0, 5)])
def test_fill_and_drain_whole_video(lib, S, A, H, C):
    """Host state over every round of a C-chunk video: chunk ids follow the
    oracle's occupancy, occupied positions never share pages, a stored chunk
    is read later from the pages it was written to (anchors included), empty
    slots refuse publish and attention, and the video ends after C-1+S."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["tiny"], S=S, A=A, H=H)
    c = cfg_of(w, first_round=0)
    c.total_chunks = C
    h = wf.wf_pool_create_host_model(c)
    T, ppc = w.T, w.N // w.page_tokens
    written = {}                                   # chunk -> page group its store wrote
    try:
        for k in range(C + S):
            assert wf.wf_round_index(h) == k
            sch = RoundSchedule(S, A, H, k, fill=True, total_chunks=C)
            ids = [-1 if x is None else x for x in sch.present_chunk_ids()]
            assert wf.wf_schedule_chunk_ids(h, T) == ids
            table = wf.wf_page_table_host(h, T * ppc)
            group = [table[p * ppc] // ppc for p in range(T)]
            occupied = [p for p in range(T) if ids[p] >= 0]
            assert len({group[p] for p in occupied}) == len(occupied)
            for p in range(A + H):                 # clean chunks sit where their store wrote them
                if ids[p] >= 0:
                    assert group[p] == written[ids[p]], (k, p)
            present = [s for s in range(S + 1) if sch.slot_present(s)]
            for s in range(S + 1):
                if s not in present:
                    with pytest.raises(wf.WfError) as e:
                        wf.wf_kv_publish(h, 0, s, 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
                    assert e.value.status == wf.WF_E_INVALID_ARG
            lo, hi = present[0], present[-1]
            wf.wf_kv_publish(h, 0, lo, hi - lo + 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, FAKE, None)
            wf.wf_attention_round(h, 0, lo, hi - lo + 1, FAKE, FAKE, FAKE, wf.WF_DTYPE_BF16, None)
            if lo > 0:
                with pytest.raises(wf.WfError) as e:
                    wf.wf_attention_round(h, 0, 0, lo + 1, FAKE, FAKE, FAKE, wf.WF_DTYPE_BF16, None)
                assert e.value.status == wf.WF_E_INVALID_ARG
            if S in present:
                written[ids[A + H]] = group[A + H]
            if k < C - 1 + S:
                wf.wf_round_advance(h, None)
                mask = wf.wf_ready_mask(h, 0)
                nxt = RoundSchedule(S, A, H, k + 1, fill=True, total_chunks=C).present_chunk_ids()
                for p in range(A + H):             # clean positions with a chunk stay published
                    assert bool(mask >> p & 1) == (nxt[p] is not None), (k, p)
        with pytest.raises(wf.WfError) as e:
            wf.wf_round_advance(h, None)
        assert e.value.status == wf.WF_E_INVALID_ARG
    finally:
        wf.wf_pool_destroy(h)


def _proj(h, w, **kw):
    args = dict(layer=0, slot_first=0, nslots=w.S + 1, x=FAKE, stride=w.hd, hidden=w.hd, wt=FAKE, bias=None,
                q_out=FAKE)
    args.update(kw)
    wf.wf_qkv_project_publish(h, args["layer"], args["slot_first"], args["nslots"], args["x"], args["stride"],
                              args["hidden"], args["wt"], args["bias"], None, args["q_out"], None)


def test_project_publish_marks_live_slots_and_validates(lib):
    w = W.WORKLOADS["ragged128"]
    h = wf.wf_pool_create_host_model(cfg_of(w))
    try:
        bad = [dict(slot_first=1, nslots=w.S + 1), dict(nslots=0), dict(x=None), dict(wt=None), dict(q_out=None),
               dict(hidden=w.hd + 32), dict(stride=w.hd - 64), dict(stride=w.hd + 4), dict(x=FAKE + 8),
               dict(layer=1)]
        for kw in bad:
            with pytest.raises(wf.WfError) as e:
                _proj(h, w, **kw)
            assert e.value.status == wf.WF_E_INVALID_ARG, kw
            assert wf.wf_ready_mask(h, 0) == 0
        _proj(h, w, slot_first=1, nslots=w.S)            # slots 1..S
        live = sum(1 << (w.T - 1 - s) for s in range(1, w.S + 1))
        assert wf.wf_ready_mask(h, 0) == live
        _proj(h, w, slot_first=0, nslots=1, hidden=2 * w.hd, stride=2 * w.hd, bias=FAKE)
        assert wf.wf_ready_mask(h, 0) == live | 1 << (w.T - 1)
    finally:
        wf.wf_pool_destroy(h)


@pytest.mark.parametrize("change", [dict(qk_dtype="fp8"), dict(heads=3, head_dim=64),
                                    dict(frame_h=1, frame_w=8, chunk_frames=8, page_tokens=64)])
def test_project_publish_rejects_unsupported_shapes(lib, change):
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["tiny"], **change)
    if change.get("heads") == 3:
        w = dataclasses.replace(w, rope_split=(24, 20, 20))
    h = wf.wf_pool_create_host_model(cfg_of(w))
    try:
        with pytest.raises(wf.WfError) as e:
            _proj(h, w)
        assert e.value.status == wf.WF_E_SHAPE
    finally:
        wf.wf_pool_destroy(h)


def test_project_publish_rejects_empty_slots_in_fill_rounds(lib):
    w = W.WORKLOADS["tiny"]
    h = wf.wf_pool_create_host_model(cfg_of(w, first_round=0))
    try:
        with pytest.raises(wf.WfError) as e:
            _proj(h, w)                                    # round 0: only slot 0 holds a chunk
        assert e.value.status == wf.WF_E_INVALID_ARG
        _proj(h, w, nslots=1)
        assert wf.wf_ready_mask(h, 0) == 1 << (w.T - 1)
    finally:
        wf.wf_pool_destroy(h)


def _proj8(h, w, **kw):
    args = dict(layer=0, slot_first=0, nslots=w.S + 1, x=FAKE, stride=w.hd, xs=FAKE, hidden=w.hd, wt=FAKE,
                ws=FAKE, bias=None, q_out=FAKE)
    args.update(kw)
    wf.wf_qkv_project_publish_w8a8(h, args["layer"], args["slot_first"], args["nslots"], args["x"], args["stride"],
                                   args["xs"], args["hidden"], args["wt"], args["ws"], args["bias"], None,
                                   args["q_out"], None)


def test_w8a8_project_publish_marks_live_slots_and_validates(lib):
    w = W.WORKLOADS["ragged128"]                      # h*d = 384: three 128-code stages
    h = wf.wf_pool_create_host_model(cfg_of(w))
    try:
        bad = [dict(slot_first=1, nslots=w.S + 1), dict(nslots=0), dict(x=None), dict(wt=None), dict(q_out=None),
               dict(xs=None), dict(ws=None), dict(xs=FAKE + 4), dict(ws=FAKE + 8),
               dict(hidden=w.hd + 64),                # not a multiple of 128 codes
               dict(stride=w.hd - 128), dict(stride=w.hd + 8), dict(x=FAKE + 8), dict(layer=1)]
        for kw in bad:
            with pytest.raises(wf.WfError) as e:
                _proj8(h, w, **kw)
            assert e.value.status == wf.WF_E_INVALID_ARG, kw
            assert wf.wf_ready_mask(h, 0) == 0
        _proj8(h, w, slot_first=1, nslots=w.S)
        live = sum(1 << (w.T - 1 - s) for s in range(1, w.S + 1))
        assert wf.wf_ready_mask(h, 0) == live
        _proj8(h, w, slot_first=0, nslots=1, hidden=2 * w.hd, stride=2 * w.hd + 16, bias=FAKE)
        assert wf.wf_ready_mask(h, 0) == live | 1 << (w.T - 1)
    finally:
        wf.wf_pool_destroy(h)


@pytest.mark.parametrize("change", [dict(qk_dtype="fp8"), dict(heads=3, head_dim=64)])
def test_w8a8_project_publish_rejects_unsupported_shapes(lib, change):
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["tiny"], **change)
    if change.get("heads") == 3:
        w = dataclasses.replace(w, rope_split=(24, 20, 20))
    h = wf.wf_pool_create_host_model(cfg_of(w))
    try:
        with pytest.raises(wf.WfError) as e:
            _proj8(h, w, hidden=128, stride=128)
        assert e.value.status == wf.WF_E_SHAPE
    finally:
        wf.wf_pool_destroy(h)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), "INVALID_ARG"), (dict(codes=None), "INVALID_ARG"), (dict(scales=None), "INVALID_ARG"),
    (dict(rows=-1), "INVALID_ARG"), (dict(cols=0), "SHAPE"), (dict(cols=12), "SHAPE"), (dict(cols=8200), "SHAPE"),
    (dict(x_stride=8), "INVALID_ARG"), (dict(x_stride=36), "INVALID_ARG"), (dict(code_stride=12), "INVALID_ARG"),
    (dict(code_stride=36), "INVALID_ARG"), (dict(x=FAKE + 8), "INVALID_ARG"), (dict(codes=FAKE + 4), "INVALID_ARG"),
    (dict(scales=FAKE + 2), "INVALID_ARG"), (dict(rows=1 << 31), "SHAPE"),
])
def test_quantize_rows_validates_before_any_launch(lib, kw, status):
    args = dict(x=FAKE, rows=10, cols=32, x_stride=32, codes=FAKE, code_stride=32, scales=FAKE)
    args.update(kw)
    with pytest.raises(wf.WfError) as e:
        wf.wf_quantize_rows_fp8(args["x"], args["rows"], args["cols"], args["x_stride"], args["codes"],
                                args["code_stride"], args["scales"], 0)
    assert e.value.status == getattr(wf, "WF_E_" + status)


def test_quantize_rows_zero_rows_launches_nothing(lib):
    wf.wf_quantize_rows_fp8(FAKE, 0, 64, 64, FAKE, 64, FAKE, 0)


def _publish_live(h, w, layers=1):
    for layer in range(layers):
        wf.wf_kv_publish(h, layer, 0, w.S + 1, FAKE, FAKE, FAKE, w.hd, None, FAKE, None, None)


@pytest.mark.parametrize("layers", [1, 2])
def test_round_replayed_leaves_the_host_where_eager_rounds_do(lib, layers):
    """A captured round publishes every live slot, attends and advances once;
    its replays run without the host. After each replay wf_round_replayed must
    leave the host state (round, readiness per layer, page groups) exactly where
    the same rounds run eagerly leave it."""
    w = W.WORKLOADS["ragged128"]
    eager = wf.wf_pool_create_host_model(cfg_of(w, num_layers=layers))
    graph = wf.wf_pool_create_host_model(cfg_of(w, num_layers=layers))
    try:
        npages = w.T * (w.N // w.page_tokens)
        for h in (eager, graph):                       # seed anchor and history
            for layer in range(layers):
                wf.wf_kv_publish(h, layer, w.S + 1, w.T - w.S - 1, None, FAKE, FAKE, w.hd, None, None, None, None)
        _publish_live(graph, w, layers)                # the captured round's publishes
        for r in range(2 * w.T + 1):
            _publish_live(eager, w, layers)
            for layer in range(layers):
                wf.wf_attention_round(eager, layer, 0, w.S + 1, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None)
            wf.wf_round_advance(eager, None)
            wf.wf_round_replayed(graph)
            assert wf.wf_round_index(graph) == wf.wf_round_index(eager)
            for layer in range(layers):
                assert wf.wf_ready_mask(graph, layer) == wf.wf_ready_mask(eager, layer), (r, layer)
            assert wf.wf_page_table_host(graph, npages) == wf.wf_page_table_host(eager, npages)
            assert wf.wf_schedule_chunk_ids(graph, w.T) == wf.wf_schedule_chunk_ids(eager, w.T)
        # after the replays the graph pool's host state takes eager calls again
        _publish_live(graph, w, layers)
        wf.wf_attention_round(graph, 0, 0, w.S + 1, FAKE, None, FAKE, wf.WF_DTYPE_FP32, None)
        wf.wf_round_advance(graph, None)
    finally:
        wf.wf_pool_destroy(eager)
        wf.wf_pool_destroy(graph)


def test_round_replayed_only_in_steady_rounds(lib):
    w = W.WORKLOADS["tiny"]
    fill = wf.wf_pool_create_host_model(cfg_of(w, first_round=0))      # fill rounds: positions empty
    last = wf.wf_pool_create_host_model(cfg_of(w, first_round=w.S + w.H + w.A, total_chunks=w.S + w.H + w.A + 1))
    try:
        with pytest.raises(wf.WfError) as e:
            wf.wf_round_replayed(fill)
        assert e.value.status == wf.WF_E_INVALID_ARG and wf.wf_round_index(fill) == 0
        # steady now, but the next round starts the drain: not replayable
        with pytest.raises(wf.WfError) as e:
            wf.wf_round_replayed(last)
        assert e.value.status == wf.WF_E_INVALID_ARG
    finally:
        wf.wf_pool_destroy(fill)
        wf.wf_pool_destroy(last)


@pytest.mark.parametrize("blocks,steps,out", [(0, 1, FAKE), (1, 0, FAKE), (-3, 8, FAKE), (1, 1, None)])
def test_mfma_calibrate_rejects_bad_arguments_before_any_launch(lib, blocks, steps, out):
    """The calibration entry checks its arguments on the host: no workgroups,
    no steps or no output buffer return WF_E_INVALID_ARG and launch nothing
    (the fake address is never touched)."""
    with pytest.raises(wf.WfError) as e:
        _lib.wf_mfma_calibrate(blocks, steps, out, stream=0)
    assert e.value.status == _lib.WF_E_INVALID_ARG


@pytest.mark.parametrize("src,dst,nbytes", [(None, FAKE, 64), (FAKE, None, 64), (FAKE, FAKE + 16, 0),
                                            (FAKE, FAKE + 64, -16), (FAKE, FAKE + 64, 24), (FAKE + 8, FAKE + 64, 32),
                                            (FAKE, FAKE + 68, 32)])
def test_stream_copy_calibrate_rejects_bad_arguments_before_any_launch(lib, src, dst, nbytes):
    """Null pointers, sizes that are not a positive multiple of 16 and pointers
    that are not 16-byte aligned return WF_E_INVALID_ARG and launch nothing
    (the fake addresses are never touched)."""
    with pytest.raises(wf.WfError) as e:
        _lib.wf_stream_copy_calibrate(src, dst, nbytes, stream=0)
    assert e.value.status == _lib.WF_E_INVALID_ARG
