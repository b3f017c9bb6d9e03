"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Floating-point bar (bf16 path): max-abs <= 1e-2 and relative L2 <= 5e-3 on the
fp32 output mode, against the oracle with bf16 storage of the published Q/K
(the pages' BF16 backend publishes bf16 pages). Integer work (page table,
placement, schedule) is compared bit for bit, and so are the published pages:
each is the round-to-nearest-even of the fp64 rotation (V: of the input).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import GroupRing, RoundSchedule, bf16_round, oracle_round, rotate_chunk

from _gpu_round import RoundRunner, err_stats, gpu_rows, oracle_rows, run_whole_video

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
    wf.load()                      # fails loudly if libwf.so is missing
    yield


def _bf16_dev_to_np(t):
    return t.view(torch.int16).cpu().numpy().astype(np.int32).astype(np.uint32) << 16


def _bf16_ulps(a, b):
    """Distance in bf16 ulps between two arrays of bf16-exact values (same sign)."""
    ia = (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
    ib = (np.asarray(b, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("name", ["tiny", "ragged128", "ragged64", "edge_s1_h0"])
def test_round_parity_full(name):
    w = W.WORKLOADS[name]
    say("case", name, "full round")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32")
    ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="bf16")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    mx, rel = err_stats(g, ref)
    say(name, "fp32-out max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
    # bf16 output mode: same bound plus the output's own rounding
    outb = r.attention("bf16")
    gb = gpu_rows(outb, w, np.arange(w.N))
    mxb, relb = err_stats(gb, ref)
    say(name, "bf16-out max_abs %.3e rel_l2 %.3e" % (mxb, relb))
    assert mxb <= BF16_MAX_ABS and relb <= BF16_REL_L2
    # the bf16 output is the fp32 output rounded once
    assert np.array_equal(gb, bf16_round(g))


# The publish groups up to 4 heads per block (4 where they divide the head
# count, else 2, else 1) and takes 256 / (head_dim / 8) tokens a block: these
# variants of the mid-size shapes reach each grouping at both head sizes, with
# a partial last token block (312 and 216 tokens), and a fused [tokens, 3*h*d]
# input row.
PLACEMENT_VARIANTS = {
    "ragged128_h2": ("ragged128", {"heads": 2}),
    "ragged128_h4_fused": ("ragged128", {"heads": 4, "fused_qkv": True}),
    "ragged64_h4": ("ragged64", {"heads": 4}),
    "ragged64_h3": ("ragged64", {"heads": 3}),
}


def _placement_workload(name):
    if name in PLACEMENT_VARIANTS:
        base, kw = PLACEMENT_VARIANTS[name]
        return dataclasses.replace(W.WORKLOADS[base], name=name, **kw)
    return W.WORKLOADS[name]


@pytest.mark.parametrize("name", ["tiny", "ragged128", "ragged64", "edge_s1_h0", "wan1.3b_s4", "wan14b_s4"]
                         + list(PLACEMENT_VARIANTS))
def test_page_table_and_publish_placement(name):
    """Page table against the closed form; every published Q, K and V element
    equal, bit for bit, to the bf16 rounding of the oracle's fp64 RoPE (V: of
    the input), at its closed-form place in the pages."""
    w = _placement_workload(name)
    say("case", name, "placement")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
    torch.cuda.synchronize()
    pool = r.pool
    ppc = pool.ppc
    # device page table == host closed form == oracle's rotation model
    ring = GroupRing(w.S, w.A, w.H)
    dev_table = pool.table.cpu().numpy().tolist()
    expect = [g * ppc + i for g in ring.groups() for i in range(ppc)]
    assert dev_table == expect == pool.page_table_host()
    assert pool.chunk_ids() == RoundSchedule(w.S, w.A, w.H, r.k).chunk_ids()
    # read the pages back
    g = pool.geometry
    npages = w.T * ppc
    # K pages [page][head][D/8][tok][8], V pages [page][head][tok/8][D][8]
    D, pt = w.head_dim, w.page_tokens
    kp = pool.pool[g["k_off"]:g["k_off"] + npages * w.heads * pt * D * 2]
    kp = kp.view(torch.int16).view(npages, w.heads, D // 8, pt, 8).permute(0, 1, 3, 2, 4)
    vp = pool.pool[g["v_off"]:g["v_off"] + npages * w.heads * pt * D * 2]
    vp = vp.view(torch.int16).view(npages, w.heads, pt // 8, D, 8).permute(0, 1, 2, 4, 3)
    kbits = _bf16_dev_to_np(kp.reshape(npages, w.heads, pt, D))     # [page, head, tok, d]
    vbits = _bf16_dev_to_np(vp.reshape(npages, w.heads, pt, D))
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    clean = r.clean_for_round()
    pos_slot = {w.T - 1 - s: s for s in range(w.S + 1)}
    total = diff = 0
    for p in range(w.T):
        c = sch.chunk_at(p)
        kk, vv = (r.live[pos_slot[p]][1:] if p in pos_slot else clean[c])
        pages = [dev_table[p * ppc + i] for i in range(ppc)]
        kg = np.concatenate([kbits[pg] for pg in pages], axis=1).view(np.float32)   # [heads, N, d]
        vg = np.concatenate([vbits[pg] for pg in pages], axis=1).view(np.float32)   # [heads, N, d]
        kref = bf16_round(rotate_chunk(w, c, kk)).transpose(1, 0, 2)
        vref = np.asarray(vv, dtype=np.float64).reshape(w.N, w.heads, w.head_dim).transpose(1, 0, 2)
        assert np.array_equal(vg.astype(np.float64), bf16_round(vref)), p        # V bit-exact
        ulp = _bf16_ulps(kg, kref)
        total += ulp.size
        diff += int(np.count_nonzero(ulp))
    # Q rows of the live slots
    qbits = _bf16_dev_to_np(r.q).view(np.float32)               # [S+1, heads, N, d]
    for s in range(w.S + 1):
        qref = bf16_round(rotate_chunk(w, sch.slot_chunk(s), r.live[s][0])).transpose(1, 0, 2)
        ulp = _bf16_ulps(qbits[s], qref)
        total += ulp.size
        diff += int(np.count_nonzero(ulp))
    say(name, "Q/K elements differing from RNE(fp64 RoPE): %d of %d" % (diff, total))
    assert diff == 0


@pytest.mark.parametrize("name", ["ragged128", "tiny", "edge_s1_h0"])
def test_noisier_slots_poisoned_with_nan_do_not_change_cleaner_outputs(name):
    w = W.WORKLOADS[name]
    say("case", name, "nan poison")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    base = r.attention("fp32").cpu().numpy()
    live = list(r.live)
    for s in range(1, w.S + 1):
        nan = np.full((w.N, w.hd), np.nan, dtype=np.float32)
        poisoned = [(nan, nan, nan)] * s
        r.publish_live(live=poisoned + live[s:], slot_first=0, nslots=s)
        out = r.attention("fp32").cpu().numpy()
        assert np.array_equal(out[s:], base[s:]), s            # bit-identical
        assert np.isnan(out[:s]).all()
        r.publish_live(live=live, slot_first=0, nslots=s)      # restore


def test_zero_query_reads_exactly_the_legal_chunks():
    w = W.WORKLOADS["ragged128"]
    say("case zero-query chunk means")
    rng = np.random.default_rng(0)

    def draw(k, s):
        c = k - s
        return (np.zeros((w.N, w.hd), np.float32), W.round_to_bf16(rng.standard_normal((w.N, w.hd), dtype=np.float32)),
                np.full((w.N, w.hd), float(c), np.float32))

    def stored(c):
        return (None, W.round_to_bf16(rng.standard_normal((w.N, w.hd), dtype=np.float32)),
                np.full((w.N, w.hd), float(c), np.float32))

    r = RoundRunner(w, draw=draw, stored=stored)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32").cpu().numpy().reshape(w.S + 1, w.N, w.hd)
    ids = RoundSchedule(w.S, w.A, w.H, r.k).chunk_ids()
    for s in range(w.S + 1):
        legal = ids[:w.T - s]
        expect = sum(legal) / len(legal)
        assert np.max(np.abs(out[s] - expect)) <= 2e-6 * abs(expect), s


def test_constant_values_pass_through():
    w = W.WORKLOADS["ragged64"]
    say("case V constant")

    def draw(k, s):
        q, kk, _ = W.draw(w, k, s)
        return q, kk, np.full((w.N, w.hd), -2.375, np.float32)

    def stored(c):
        _, kk, _ = W.stored_draw(w, c)
        return None, kk, np.full((w.N, w.hd), -2.375, np.float32)

    r = RoundRunner(w, draw=draw, stored=stored)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32").cpu().numpy()
    assert np.max(np.abs(out + 2.375)) <= 2.375 * 2 ** -7      # P in bf16, sums in fp32


def test_slot_subset_launch_matches_full_round():
    w = W.WORKLOADS["ragged128"]
    say("case slot subsets")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    full = r.attention("fp32").cpu().numpy()
    for first, n in [(0, 1), (1, 2), (w.S, 1), (2, w.S - 1)]:
        part = r.attention("fp32", slot_first=first, nslots=n).cpu().numpy()
        assert np.array_equal(part[first:first + n], full[first:first + n])
        others = [i for i in range(w.S + 1) if not first <= i < first + n]
        assert np.isnan(part[others]).all()


def _sample_rows(N, seed, extra=16):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, 129, 255, 256, 257, N // 2, N - 73, N - 72, N - 71, N - 2, N - 1]
    fixed += [(N // 128) * 128 - 1, (N // 128) * 128, (N // 256) * 256 - 1, (N // 256) * 256]
    return np.array(sorted(set(int(x) for x in fixed + list(rng.integers(0, N, extra)) if 0 <= x < N)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["wan1.3b_s4", "wan14b_s4"])
def test_full_size_round_every_output(name):
    """Every output row of every head and slot of a full-size round (fp32
    output mode) against the oracle, which runs on the host's cores."""
    from oracle.parallel import compare_every_output, host_workers
    w = W.WORKLOADS[name]
    say("case", name, "full size, every output;", host_workers(), "oracle workers")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
    out = r.attention("fp32").cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim)
    assert np.isfinite(out).all()
    mx, rel, worst, n = compare_every_output(out, w, r.k, "bf16", say=say)
    say(name, "every output (%d slot-head units): max_abs %.3e rel_l2 %.3e worst unit rel_l2 %.3e"
        % (n, mx, rel, worst))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2 and worst <= BF16_REL_L2


@pytest.mark.timeout(900)
def test_thirty_layer_rounds_with_rotation():
    """30 consecutive layer-rounds of one pool, advancing in between: every
    output of the first and the last round, sampled rows of one head in the
    rounds between, and the device page table after every advance."""
    from oracle.parallel import compare_every_output
    w = W.WORKLOADS["wan1.3b_s5_30"]
    say("case", w.name, "30 consecutive layer-rounds")
    r = RoundRunner(w)
    r.seed_clean()
    worst = (0.0, 0.0)
    for i in range(w.layer_rounds):
        r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
        out = r.attention("fp32")
        assert r.pool.round_index() == r.k
        assert r.pool.chunk_ids() == RoundSchedule(w.S, w.A, w.H, r.k).chunk_ids()
        if i in (0, w.layer_rounds - 1):
            o = out.cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim)
            mx, rel, wu, n = compare_every_output(o, w, r.k, "bf16", say=say)
            say("round", r.k, "every output (%d units): worst unit rel_l2 %.3e" % (n, wu))
            assert wu <= BF16_REL_L2
        else:
            rows = _sample_rows(w.N, 100 + i, extra=2)[::3]
            heads = [i % w.heads]
            ref = oracle_rows(w, r.k, r.live, r.clean_for_round(), rows, heads=heads)
            g = gpu_rows(out, w, rows, heads=heads)
            mx, rel = err_stats(g, ref)
        worst = (max(worst[0], mx), max(worst[1], rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, (i, mx, rel)
        ring = GroupRing(w.S, w.A, w.H)
        for _ in range(i):
            ring.advance()
        dev = r.pool.table.cpu().numpy().tolist()
        assert dev == [g_ * r.pool.ppc + j for g_ in ring.groups() for j in range(r.pool.ppc)]
        r.advance()
        say("round", i, "ok max_abs %.2e rel %.2e" % (mx, rel))
    say("30 rounds worst max_abs %.3e rel_l2 %.3e" % worst)


@pytest.mark.parametrize("name", ["edge_s1_h0", "tiny"])
def test_rotated_rounds_full_output(name):
    """Every output row of several consecutive rounds, advancing in between,
    so each page group visits every position of the ring."""
    w = W.WORKLOADS[name]
    say("case", name, "rotated rounds, full output")
    r = RoundRunner(w)
    r.seed_clean()
    for i in range(2 * (w.H + w.S + 1) + 1):
        r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
        out = r.attention("fp32")
        ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="bf16")
        g = gpu_rows(out, w, np.arange(w.N))
        mx, rel = err_stats(g, ref)
        say(name, "round", r.k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, (i, mx, rel)
        r.advance()


@pytest.mark.parametrize("name", ["tiny", "ragged128", "edge_s1_h0"])
def test_all_live_mask_round_parity(name):
    """Every live slot sees every live slot (bidirectional live K/V): parity
    against the oracle's all-live mask; the noisiest slot reads the whole
    context under either mask, so its output is the wavefront pool's, bit for
    bit."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS[name], live_mask="all")
    say("case", name, "all-live mask")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32")
    ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="bf16", mask="all")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    mx, rel = err_stats(g, ref)
    say(name, "all-live fp32-out max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
    rw = RoundRunner(W.WORKLOADS[name])
    rw.seed_clean()
    rw.publish_live(live=r.live)
    outw = rw.attention("fp32")
    assert torch.equal(outw[0], out[0])
    assert not torch.equal(outw[1:], out[1:])


def test_two_layers_share_one_page_table():
    """A pool of two layers with one page table: each layer's round equals the
    oracle on its own data, across an advance (which needs the store of every
    layer), and the layers' pages never mix."""
    import dataclasses
    from _gpu_round import config_of, stack_dev
    import wavefront_causal_attention_amd as wf
    base = W.WORKLOADS["ragged128"]
    ws = [dataclasses.replace(base, seed=base.seed + 100 * l) for l in range(2)]
    k0 = base.steady_round
    pool = wf.Pool(config_of(base, first_round=k0, num_layers=2))
    q = pool.q_buffer()
    clean = [{}, {}]
    for l, w in enumerate(ws):                                   # seed anchor + history per layer
        sch = RoundSchedule(w.S, w.A, w.H, k0)
        ks, vs = [], []
        for slot in range(w.S + 1, w.T):
            c = sch.chunk_at(w.T - 1 - slot)
            _, kk, vv = W.stored_draw(w, c)
            clean[l][c] = (kk, vv)
            ks.append(kk)
            vs.append(vv)
        pool.publish(l, w.S + 1, w.T - w.S - 1, None, stack_dev(ks, w.in_dtype), stack_dev(vs, w.in_dtype), w.hd)
    for rnd in range(2):
        k = k0 + rnd
        say("case two layers, round", k)
        outs, lives = [], []
        for l, w in enumerate(ws):
            live = W.draw_slots(w, k, range(w.S + 1))
            lives.append(live)
            pool.publish(l, 0, w.S + 1, stack_dev([x[0] for x in live], w.in_dtype),
                         stack_dev([x[1] for x in live], w.in_dtype), stack_dev([x[2] for x in live], w.in_dtype),
                         w.hd, q_out=q)
            out = pool.out_buffer("fp32")
            out.fill_(float("nan"))
            pool.attention(l, 0, w.S + 1, q, out)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        for l, w in enumerate(ws):
            sch = RoundSchedule(w.S, w.A, w.H, k)
            ref = oracle_round(w, k, lives[l], {c: clean[l][c] for c in sch.chunk_ids()[:w.A + w.H]},
                               storage="bf16")
            g = outs[l].reshape(w.S + 1, w.N, w.heads, w.head_dim)
            mx, rel = err_stats(g, ref)
            say("layer", l, "round", k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
            assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
        assert not np.allclose(outs[0], outs[1])
        for l, w in enumerate(ws):                               # the store becomes history
            c = RoundSchedule(w.S, w.A, w.H, k).chunk_at(w.A + w.H)
            clean[l][c] = tuple(lives[l][w.S][1:])
        pool.advance()


@pytest.mark.parametrize("name,C", [("tiny", 6), ("edge_s1_h0", 5), ("ragged128", 7)])
def test_fill_and_drain_whole_video(name, C):
    """Every round of a short video, the pipeline filling and draining: each
    slot that holds a chunk matches the oracle over the positions that hold
    one; slots without a chunk are left untouched."""
    w = W.WORKLOADS[name]
    say("case", name, "whole video of", C, "chunks")

    def check(k, out, live, clean, lo, hi):
        ref = oracle_round(w, k, live, clean, storage="bf16", fill=True, total_chunks=C,
                           slots=range(lo, hi + 1))
        o = out.cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim).astype(np.float64)
        untouched = np.delete(o, list(range(lo, hi + 1)), axis=0)
        assert np.isnan(untouched).all()
        g = o[lo:hi + 1]
        assert not np.isnan(g).any()
        mx, rel = err_stats(g, ref)
        say(name, "round", k, "slots", lo, "..", hi, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, (k, mx, rel)

    run_whole_video(w, C, check)


def test_fill_rounds_of_an_open_ended_video_reach_the_steady_state():
    """With no video length the pool starts in the first fill round and, once
    the ring is full, runs the same rounds as a pool created steady."""
    w = W.WORKLOADS["tiny"]
    say("case tiny, open-ended video from round 0")
    from _gpu_round import config_of, stack_dev
    import wavefront_causal_attention_amd as wf
    pool = wf.Pool(config_of(w, first_round=0))
    q = pool.q_buffer()
    clean = {}
    for k in range(w.steady_round + 2):
        sch = RoundSchedule(w.S, w.A, w.H, k, fill=True)
        present = [s for s in range(w.S + 1) if sch.slot_present(s)]
        lo, hi = present[0], present[-1]
        live = [W.draw(w, k, s) if s in present else None for s in range(w.S + 1)]
        sel = live[lo:hi + 1]
        pool.publish(0, lo, hi - lo + 1, stack_dev([x[0] for x in sel], w.in_dtype),
                     stack_dev([x[1] for x in sel], w.in_dtype), stack_dev([x[2] for x in sel], w.in_dtype),
                     w.hd, q_out=q)
        out = pool.out_buffer("fp32")
        out.fill_(float("nan"))
        pool.attention(0, lo, hi - lo + 1, q, out)
        torch.cuda.synchronize()
        cl = {c: clean[c] for c in sch.present_chunk_ids()[:w.A + w.H] if c is not None}
        ref = oracle_round(w, k, live, cl, storage="bf16", fill=True, slots=range(lo, hi + 1))
        g = out.cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim)[lo:hi + 1].astype(np.float64)
        mx, rel = err_stats(g, ref)
        say("round", k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, (k, mx, rel)
        if k >= w.steady_round:
            assert (lo, hi) == (0, w.S)
            steady = oracle_round(w, k, live, cl, storage="bf16")
            assert np.allclose(steady, ref, equal_nan=False)
        if w.S in present:
            clean[sch.slot_chunk(w.S)] = tuple(live[w.S][1:])
        pool.advance()


def test_maximum_positions_and_table_pages():
    """T = 64 context positions and 1024 table pages (the library's limits):
    every output of two consecutive rounds against the oracle, across an
    advance, with all 64 readiness bits in use."""
    w = W.WORKLOADS["max64"]
    assert w.T == 64 and w.T * (w.N // w.page_tokens) == 1024
    say("case max64: T = 64, 1024 pages")
    r = RoundRunner(w)
    r.seed_clean()
    for i in range(2):
        r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
        assert r.pool.ready_mask(0) == (1 << 64) - 1
        out = r.attention("fp32")
        ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="bf16")
        g = gpu_rows(out, w, np.arange(w.N))
        assert not np.isnan(g).any()
        mx, rel = err_stats(g, ref)
        say("max64 round", r.k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
        dev = r.pool.table.cpu().numpy().tolist()
        assert dev == r.pool.page_table_host()
        r.advance()


def test_sixty_three_query_slots():
    """S = 62: query slots 32..62 sit in the high bits of their work entries;
    every output of every slot of two rounds, across an advance."""
    w = W.WORKLOADS["slots62"]
    say("case slots62: 63 query slots")
    r = RoundRunner(w)
    r.seed_clean()
    for i in range(2):
        r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
        out = r.attention("fp32")
        ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="bf16")
        g = gpu_rows(out, w, np.arange(w.N))
        assert not np.isnan(g).any()
        mx, rel = err_stats(g, ref)
        say("slots62 round", r.k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
        r.advance()


@pytest.mark.parametrize("path", ["publish", "project"])
def test_explicit_rope_time_offsets(path):
    """chunk_t0_host given explicitly: the schedule's own offsets publish
    exactly what the default (the pool's round counter) does; offsets shifted
    by 7 frames rotate Q and K by the time positions shifted by 7, as the
    oracle's RoPE does (within one bf16 ulp)."""
    import wavefront_causal_attention_amd as wf
    from oracle import project_qkv, rope_3d, split_qkv, token_grid
    from _gpu_round import bf16_dev_bits_to_f32, bf16_ulps, position_rows, read_pages, stack_dev, to_dev
    w = W.WORKLOADS["ragged128"]
    k = w.steady_round
    sch = RoundSchedule(w.S, w.A, w.H, k)
    t0 = [w.chunk_frames * sch.slot_chunk(s) for s in range(w.S + 1)]
    if path == "publish":
        live = [W.draw(w, k, s) for s in range(w.S + 1)]
        qd, kd, vd = (stack_dev([x[i] for x in live], w.in_dtype) for i in range(3))
        run = lambda r, t: r.pool.publish(0, 0, w.S + 1, qd, kd, vd, w.hd, q_out=r.q, chunk_t0=t)
    else:
        xs = [W.draw_hidden(w, k, s) for s in range(w.S + 1)]
        wt, b = W.projection_weights(w)
        xd, wd, bd = to_dev(np.concatenate(xs, 0), "bf16"), to_dev(wt, "bf16"), to_dev(b, "bf16")
        live = [tuple(split_qkv(project_qkv(x, wt, b), w.hd)) for x in xs]
        run = lambda r, t: r.pool.project_publish(0, 0, w.S + 1, xd, w.hd, w.hd, wd, bd, q_out=r.q, chunk_t0=t)
    say("case ragged128,", path, "explicit RoPE time offsets", t0)
    res = []
    for t in (None, t0, [x + 7 for x in t0]):
        r = RoundRunner(w)
        run(r, t)
        torch.cuda.synchronize()
        kp, vp = read_pages(r.pool, w)
        res.append((r.q.clone(), kp, vp, r.pool.table.cpu().numpy(), r.pool.ppc))
    assert torch.equal(res[0][0], res[1][0])
    for s in range(w.S + 1):                       # the published positions (anchor and history are not)
        p = w.T - 1 - s
        for i in (1, 2):
            assert np.array_equal(position_rows(res[0][i], res[0][3], p, res[0][4]),
                                  position_rows(res[1][i], res[1][3], p, res[1][4])), (s, i)
    q_sh, kp, vp, table, ppc = res[2]
    qf = bf16_dev_bits_to_f32(q_sh)
    for s in range(w.S + 1):
        t, y, x = token_grid(sch.slot_chunk(s), w.chunk_frames, w.frame_h, w.frame_w)
        q, kk, v = (a.reshape(w.N, w.heads, w.head_dim) for a in live[s])
        qr = bf16_round(rope_3d(q, t + 7, y, x, w.rope_split, w.rope_theta)).transpose(1, 0, 2)
        kr = bf16_round(rope_3d(kk, t + 7, y, x, w.rope_split, w.rope_theta)).transpose(1, 0, 2)
        p = w.T - 1 - s
        assert bf16_ulps(qf[s], qr).max() <= 1, s
        assert bf16_ulps(position_rows(kp, table, p, ppc), kr).max() <= 1, s
        assert np.array_equal(position_rows(vp, table, p, ppc), position_rows(res[0][2], table, p, ppc))
