"""GPU parity of the fused QKV projection + RoPE + publish (wf_qkv_project_publish)
against the fp64 oracle, through the C ABI.

The oracle projects the same bf16 hidden states with the same bf16 weights in
fp64 (oracle.project_qkv), rotates Q and K in fp64 and rounds the pages to
bf16. The kernel accumulates in fp32, rotates in fp32 and rounds once, so every
published element is within one bf16 ulp of the oracle's and almost all are
equal. End to end, attention over the fused publish meets the bf16 bar
(max-abs 1e-2, rel-L2 5e-3, fp32 output mode).
"""
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import RoundSchedule, bf16_round, oracle_round, project_qkv, rope_3d, rotate_chunk, split_qkv, token_grid

from _gpu_round import (RoundRunner, bf16_dev_bits_to_f32, err_stats, gpu_rows, oracle_rows, position_rows,
                        read_pages, to_dev)
from _gpu_round import bf16_ulps as _bf16_ulps, worst_ulp as _worst

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import wavefront_causal_attention_amd as wf
    wf.load()
    yield


def _project_round(r: RoundRunner, slot_first=0, nslots=None):
    """Fused projection + publish of live slots [slot_first, +nslots) with the
    workload's seeded hidden states and weights; returns the fp64 (q, k, v) the
    oracle projects for every live slot."""
    w = r.w
    nslots = w.S + 1 - slot_first if nslots is None else nslots
    xs = [W.draw_hidden(w, r.k, s) for s in range(w.S + 1)]
    wt, b = W.projection_weights(w)
    xd = to_dev(np.concatenate(xs[slot_first:slot_first + nslots], 0), "bf16")
    wd, bd = to_dev(wt, "bf16"), to_dev(b, "bf16")
    r.pool.project_publish(0, slot_first, nslots, xd, w.hd, w.hd, wd, bd, q_out=r.q)
    torch.cuda.synchronize()
    live = [tuple(split_qkv(project_qkv(x, wt, b), w.hd)) for x in xs]
    r.live = live
    return live


@pytest.mark.parametrize("name", ["tiny", "ragged128", "ragged64", "edge_s1_h0"])
def test_project_publish_pages_match_oracle(name):
    w = W.WORKLOADS[name]
    say("case", name, "fused projection: Q and pages")
    r = RoundRunner(w)
    live = _project_round(r)
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    kp, vp = read_pages(r.pool, w)
    table = r.pool.table.cpu().numpy()
    qf = bf16_dev_bits_to_f32(r.q)                      # [S+1, heads, N, d]
    total = diff = 0
    for s in range(w.S + 1):
        c = sch.slot_chunk(s)
        q, k, v = live[s]
        p = w.T - 1 - s
        refs = [(qf[s], bf16_round(rotate_chunk(w, c, q)).transpose(1, 0, 2)),
                (position_rows(kp, table, p, r.pool.ppc), bf16_round(rotate_chunk(w, c, k)).transpose(1, 0, 2)),
                (position_rows(vp, table, p, r.pool.ppc),
                 bf16_round(v.reshape(w.N, w.heads, w.head_dim)).transpose(1, 0, 2))]
        for got, ref in refs:
            ulp = _bf16_ulps(got, ref)
            assert ulp.max() <= 1, (s, _worst(got, ref))
            total += ulp.size
            diff += int(np.count_nonzero(ulp))
    say(name, "elements 1 ulp from the oracle: %d of %d" % (diff, total))
    assert diff <= 1e-3 * total


@pytest.mark.parametrize("name", ["tiny", "ragged128", "edge_s1_h0"])
def test_project_publish_round_parity(name):
    w = W.WORKLOADS[name]
    say("case", name, "fused projection: full round")
    r = RoundRunner(w)
    r.seed_clean()
    live = _project_round(r)
    out = r.attention("fp32")
    ref = oracle_round(w, r.k, live, r.clean_for_round(), storage="bf16")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    mx, rel = err_stats(g, ref)
    say(name, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2


def test_project_publish_slot_subset_equals_full_launch():
    w = W.WORKLOADS["ragged128"]
    say("case ragged128, fused projection: slot subset")
    ra, rb = RoundRunner(w), RoundRunner(w)
    _project_round(ra)
    _project_round(rb, slot_first=1, nslots=w.S - 1)
    ka, va = read_pages(ra.pool, w)
    kb, vb = read_pages(rb.pool, w)
    table = ra.pool.table.cpu().numpy()
    for s in range(1, w.S):
        p = w.T - 1 - s
        assert np.array_equal(position_rows(ka, table, p, ra.pool.ppc), position_rows(kb, table, p, rb.pool.ppc))
        assert np.array_equal(position_rows(va, table, p, ra.pool.ppc), position_rows(vb, table, p, rb.pool.ppc))
        assert torch.equal(ra.q[s], rb.q[s])


def test_project_publish_full_size_sampled():
    """Wan2.1-1.3B S = 4: fused projection of all five live slots, pages on
    sampled tokens against the oracle's projection, attention on sampled rows
    and heads against the oracle over the full projected context."""
    w = W.WORKLOADS["wan1.3b_s4"]
    say("case wan1.3b_s4, fused projection, full size")
    r = RoundRunner(w)
    r.seed_clean()
    live = _project_round(r)
    out = r.attention("fp32")
    rng = np.random.default_rng(21)
    toks = np.array(sorted(set([0, 1, 255, 256, 4607, 4608, w.N - 1] + list(rng.integers(0, w.N, 40)))))
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    kp, vp = read_pages(r.pool, w)
    table = r.pool.table.cpu().numpy()
    qf = bf16_dev_bits_to_f32(r.q)
    diff = total = 0
    for s in range(w.S + 1):
        c = sch.slot_chunk(s)
        t, y, x = token_grid(c, w.chunk_frames, w.frame_h, w.frame_w)
        q, k, v = (a.reshape(w.N, w.heads, w.head_dim)[toks] for a in live[s])
        qr = bf16_round(rope_3d(q, t[toks], y[toks], x[toks], w.rope_split, w.rope_theta))
        kr = bf16_round(rope_3d(k, t[toks], y[toks], x[toks], w.rope_split, w.rope_theta))
        p = w.T - 1 - s
        for got, ref in ((qf[s][:, toks], qr.transpose(1, 0, 2)),
                         (position_rows(kp, table, p, r.pool.ppc)[:, toks], kr.transpose(1, 0, 2)),
                         (position_rows(vp, table, p, r.pool.ppc)[:, toks], bf16_round(v).transpose(1, 0, 2))):
            ulp = _bf16_ulps(got, ref)
            assert ulp.max() <= 1, (s, _worst(got, ref))
            diff += int(np.count_nonzero(ulp))
            total += ulp.size
    say("sampled elements 1 ulp from the oracle: %d of %d" % (diff, total))
    assert diff <= 1e-3 * total
    rows = np.array(sorted(set([0, 255, 256, 4607, 4608, w.N - 1] + list(rng.integers(0, w.N, 10)))))
    heads = [0, 5, 11]
    ref = oracle_rows(w, r.k, live, r.clean_for_round(), rows, heads=heads)
    g = gpu_rows(out, w, rows, heads=heads)
    mx, rel = err_stats(g, ref)
    say("attention rows", len(rows), "heads", heads, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
    assert torch.isfinite(out).all().item()


@pytest.mark.parametrize("name,C,with_bias", [("tiny", 5, True), ("edge_s1_h0", 5, False)])
def test_project_publish_whole_video(name, C, with_bias):
    """Every round of a short video published through the fused projection:
    the store's projected K/V becomes anchor or history (an anchor chunk is
    written straight into the anchor's pages), and each occupied slot matches
    the oracle's fill schedule over the positions that hold a chunk."""
    from _gpu_round import config_of
    import wavefront_causal_attention_amd as wf
    w = W.WORKLOADS[name]
    say("case", name, "fused projection, whole video of", C, "chunks, bias", with_bias)
    pool = wf.Pool(config_of(w, first_round=0, total_chunks=C))
    q = pool.q_buffer()
    wt, b = W.projection_weights(w)
    b = b if with_bias else None
    wd = to_dev(wt, "bf16")
    bd = to_dev(b, "bf16") if with_bias else None
    clean = {}
    for k in range(C + w.S):
        sch = RoundSchedule(w.S, w.A, w.H, k, fill=True, total_chunks=C)
        present = [s for s in range(w.S + 1) if sch.slot_present(s)]
        lo, hi = present[0], present[-1]
        xs = {s: W.draw_hidden(w, k, s) for s in present}
        xd = to_dev(np.concatenate([xs[s] for s in present], 0), "bf16")
        pool.project_publish(0, lo, hi - lo + 1, xd, w.hd, w.hd, wd, bd, q_out=q)
        out = pool.out_buffer("fp32")
        out.fill_(float("nan"))
        pool.attention(0, lo, hi - lo + 1, q, out)
        torch.cuda.synchronize()
        live = [tuple(split_qkv(project_qkv(xs[s], wt, b), w.hd)) if s in xs else None for s in range(w.S + 1)]
        cl = {c: clean[c] for c in sch.present_chunk_ids()[:w.A + w.H] if c is not None}
        ref = oracle_round(w, k, live, cl, storage="bf16", fill=True, total_chunks=C, slots=range(lo, hi + 1))
        o = out.cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim).astype(np.float64)
        assert np.isnan(np.delete(o, list(range(lo, hi + 1)), axis=0)).all()
        mx, rel = err_stats(o[lo:hi + 1], ref)
        say(name, "round", k, "slots", lo, "..", hi, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, (k, mx, rel)
        if w.S in present:
            clean[sch.slot_chunk(w.S)] = tuple(live[w.S][1:])
        if k < C - 1 + w.S:
            pool.advance()
