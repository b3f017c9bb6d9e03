"""GPU parity of the W8A8 path against the fp64 oracle, through the C ABI:
the per-row e4m3 quantiser (wf_quantize_rows_fp8) and the fused projection +
RoPE + publish over e4m3 operands (wf_qkv_project_publish_w8a8).

The quantiser decides integers from floating point, so both sides decide in
the same precision (the IEEE fp32 quotient x / scale) and codes and scales
must be bit-identical. The projection then starts from the same codes on both
sides: the oracle sums the dequantised products in fp64; the kernel sums code
products on the e4m3 MFMA, which does not add its 64 products exactly: small
products lose bits below a fixed distance from the instruction's largest one
(test_e4m3_mfma_summation_on_controlled_codes: 448 - 448 + 62 x 2^-9 comes
back as 0.109375 instead of 0.12109375, 448 x 2 - 448 x 2 + 60 x 2^-6 as
0.875 instead of 0.9375), while the fp32 accumulator add is exact. So each
element of the projection may differ from the exact one by up to ACC_REL *
sum_c |x^_c w^_c|, and a published element is bounded by that (after RoPE:
the sum over its channel pair) plus one bf16 ulp. Random full-range codes use
up to 0.92 of that allowance, data drawn like the workloads' up to 0.8. End
to end, attention over the W8A8 publish meets the bf16 bar (max-abs 1e-2,
rel-L2 5e-3, fp32 output mode) against the oracle's attention over the
oracle's W8A8 projection.
"""
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import (RoundSchedule, bf16_round, fp8_e4m3_decode, oracle_round, project_qkv_w8a8,
                    quantize_rows_fp8, rope_3d, rotate_chunk, split_qkv, token_grid)

from _gpu_round import (RoundRunner, bf16_dev_bits_to_f32, err_stats, gpu_rows, oracle_rows, position_rows,
                        read_pages, to_dev)

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
ACC_REL = 2.0 ** -11      # e4m3 MFMA summation error per sum of |products|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import wavefront_causal_attention_amd as wf
    wf.load()
    yield


def _rows(seed, rows, cols):
    """bf16-exact rows over many binades, with an all-zero row, a row whose one
    outlier sends the rest to e4m3 subnormals, and rows whose quotients sit
    next to e4m3 midpoints (the fp32 reciprocal would round them one code up)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    if rows > 1:
        x[1] = rng.standard_normal(cols).astype(np.float32) * np.float32(1e-3)
        x[1, cols // 2] = 9.0
    if rows > 4:
        for r, (amax, v) in zip((2, 3, 4), ((1.1875, 0.111328125), (2.375, 0.890625),
                                            (0.0673828125, -0.050537109375))):
            x[r] = rng.uniform(-0.5, 0.5, cols).astype(np.float32) * np.float32(amax)
            x[r, 0], x[r, 1:8] = amax, v
    return W.round_to_bf16(x)


@pytest.mark.parametrize("rows,cols,x_stride,code_stride", [
    (37, 1536, 1536, 1536),       # Wan2.1-1.3B width, a partial last workgroup of rows
    (3, 8, 16, 16),               # the narrowest row, padded strides
    (11, 3072, 3080, 3088),       # 8 vectors per lane
    (9, 8192, 8192, 8192),        # the widest row the quantiser holds
    (130, 5120, 5128, 5136),      # Wan2.1-14B width, padded strides
])
def test_quantize_rows_bit_exact(rows, cols, x_stride, code_stride):
    import wavefront_causal_attention_amd as wf
    say("case quantize rows", rows, "cols", cols, "strides", x_stride, code_stride)
    x = _rows(40 + rows, rows, cols)
    xp = np.full((rows, x_stride), 3.0e38, dtype=np.float32)       # padding the kernel must not read
    xp[:, :cols] = x
    xd = to_dev(xp, "bf16")
    codes = torch.full((rows, code_stride), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows + 1,), -7.0, dtype=torch.float32, device="cuda")
    wf.wf_quantize_rows_fp8(xd, rows, cols, x_stride, codes, code_stride, scales, None)
    torch.cuda.synchronize()
    ref_c, ref_s = quantize_rows_fp8(x)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy()
    bad = np.argwhere(got_c[:, :cols] != ref_c)
    assert len(bad) == 0, "%d codes differ, first at %s: got %d ref %d" % (
        len(bad), tuple(bad[0]), got_c[tuple(bad[0])], ref_c[tuple(bad[0])])
    assert np.array_equal(got_s[:rows].view(np.uint32), ref_s.view(np.uint32))
    assert (got_c[:, cols:] == 0xAB).all() and got_s[rows] == -7.0


def _w8a8_round(r: RoundRunner, slot_first=0, nslots=None, with_bias=True):
    """W8A8 projection + publish of live slots [slot_first, +nslots): the
    hidden states and the weight are quantised on the GPU, checked bit-exact
    against the oracle's quantiser, and the oracle's fp64 (q, k, v) of every
    live slot is returned."""
    import wavefront_causal_attention_amd as wf
    w = r.w
    nslots = w.S + 1 - slot_first if nslots is None else nslots
    xs = [W.draw_hidden(w, r.k, s) for s in range(w.S + 1)]
    wt, b = W.projection_weights(w)
    b = b if with_bias else None
    xd = to_dev(np.concatenate(xs[slot_first:slot_first + nslots], 0), "bf16")
    x8, sx = wf.quantize_rows_fp8(xd)
    w8, sw = wf.quantize_rows_fp8(to_dev(wt, "bf16"))
    bd = to_dev(b, "bf16") if with_bias else None
    r.pool.project_publish_w8a8(0, slot_first, nslots, x8, x8.stride(0), sx, w.hd, w8, sw, bd, q_out=r.q)
    torch.cuda.synchronize()
    wc, ws = quantize_rows_fp8(wt)
    assert np.array_equal(w8.cpu().numpy(), wc) and np.array_equal(sw.cpu().numpy(), ws)
    q8 = [quantize_rows_fp8(x) for x in xs]
    assert np.array_equal(x8.cpu().numpy(), np.concatenate([q8[s][0] for s in range(slot_first, slot_first + nslots)]))
    assert np.array_equal(sx.cpu().numpy(), np.concatenate([q8[s][1] for s in range(slot_first, slot_first + nslots)]))
    live = [tuple(split_qkv(project_qkv_w8a8(q8[s][0], q8[s][1], wc, ws, b), w.hd)) for s in range(w.S + 1)]
    r.live = live
    wabs = np.abs(fp8_e4m3_decode(wc) * ws.astype(np.float64)[:, None])
    r.absum = lambda s, rows=slice(None): (np.abs(fp8_e4m3_decode(q8[s][0][rows]) *
                                                  q8[s][1][rows].astype(np.float64)[:, None]) @ wabs.T)
    return live


def _bf16_ulp(v):
    """Spacing of bfloat16 values at |v| (normal range)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def _pair_sum(a):
    """Per channel, the sum over its RoPE pair (2m, 2m+1) along the last axis."""
    p = a.reshape(a.shape[:-1] + (a.shape[-1] // 2, 2)).sum(-1)
    return np.repeat(p, 2, axis=-1)


def _bound_check(got, ref, acc_bound, what):
    """|got - ref| <= one bf16 ulp + the e4m3 MFMA summation bound; returns
    (elements that differ, elements, worst share of the allowance used)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    allow = _bf16_ulp(np.maximum(np.abs(got), np.abs(ref))) + acc_bound
    use = err / allow
    i = np.unravel_index(int(np.argmax(use)), use.shape)
    assert use[i] <= 1.0, "%s: %s got %r ref %r err %.3e allowed %.3e (acc %.3e)" % (
        what, i, got[i], ref[i], err[i], allow[i], acc_bound[i])
    return int(np.count_nonzero(err)), err.size, float(use[i])


def _check_pages(r, live, slots):
    w = r.w
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    kp, vp = read_pages(r.pool, w)
    table = r.pool.table.cpu().numpy()
    qf = bf16_dev_bits_to_f32(r.q)
    total = diff = 0
    worst = 0.0
    for s in slots:
        c = sch.slot_chunk(s)
        q, k, v = live[s]
        a = getattr(r, "acc_rel", ACC_REL) * r.absum(s)    # [N, 3 h d]
        heads = lambda m: m.reshape(w.N, w.heads, w.head_dim).transpose(1, 0, 2)
        p = w.T - 1 - s
        refs = [(qf[s], bf16_round(rotate_chunk(w, c, q)).transpose(1, 0, 2), _pair_sum(heads(a[:, :w.hd])), "Q"),
                (position_rows(kp, table, p, r.pool.ppc), bf16_round(rotate_chunk(w, c, k)).transpose(1, 0, 2),
                 _pair_sum(heads(a[:, w.hd:2 * w.hd])), "K"),
                (position_rows(vp, table, p, r.pool.ppc), bf16_round(v.reshape(w.N, w.heads, w.head_dim)).transpose(1, 0, 2),
                 heads(a[:, 2 * w.hd:]), "V")]
        for got, ref, bound, what in refs:
            d, t, u = _bound_check(got, ref, bound, "slot %d %s" % (s, what))
            diff, total, worst = diff + d, total + t, max(worst, u)
    return diff, total, worst


@pytest.mark.parametrize("name,with_bias", [("tiny", True), ("ragged128", True), ("ragged64", False),
                                            ("edge_s1_h0", True)])
def test_w8a8_project_publish_pages_match_oracle(name, with_bias):
    w = W.WORKLOADS[name]
    say("case", name, "W8A8 projection: Q and pages, bias", with_bias)
    r = RoundRunner(w)
    live = _w8a8_round(r, with_bias=with_bias)
    diff, total, worst = _check_pages(r, live, range(w.S + 1))
    say(name, "elements differing from the oracle: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))


def test_w8a8_slot_subset():
    w = W.WORKLOADS["ragged128"]
    say("case ragged128, W8A8 projection: slots 1..S-1")
    r = RoundRunner(w)
    live = _w8a8_round(r, slot_first=1, nslots=w.S - 1)
    diff, total, worst = _check_pages(r, live, range(1, w.S))
    say("elements differing from the oracle: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))


@pytest.mark.parametrize("name", ["tiny", "ragged128", "edge_s1_h0"])
def test_w8a8_round_parity(name):
    w = W.WORKLOADS[name]
    say("case", name, "W8A8 projection: full round")
    r = RoundRunner(w)
    r.seed_clean()
    live = _w8a8_round(r)
    out = r.attention("fp32")
    ref = oracle_round(w, r.k, live, r.clean_for_round(), storage="bf16")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    mx, rel = err_stats(g, ref)
    say(name, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2


def test_w8a8_full_size_sampled():
    """Wan2.1-1.3B S = 4: W8A8 projection of all five live slots; pages on
    sampled tokens against the oracle's W8A8 projection, attention on sampled
    rows and heads against the oracle over the whole projected context."""
    w = W.WORKLOADS["wan1.3b_s4"]
    say("case wan1.3b_s4, W8A8 projection, full size")
    r = RoundRunner(w)
    r.seed_clean()
    live = _w8a8_round(r)
    out = r.attention("fp32")
    rng = np.random.default_rng(22)
    toks = np.array(sorted(set([0, 1, 255, 256, 4607, 4608, w.N - 1] + list(rng.integers(0, w.N, 40)))))
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    kp, vp = read_pages(r.pool, w)
    table = r.pool.table.cpu().numpy()
    qf = bf16_dev_bits_to_f32(r.q)
    diff = total = 0
    worst = 0.0
    heads = lambda m: m.reshape(len(toks), w.heads, w.head_dim).transpose(1, 0, 2)
    for s in range(w.S + 1):
        c = sch.slot_chunk(s)
        t, y, x = token_grid(c, w.chunk_frames, w.frame_h, w.frame_w)
        q, k, v = (a.reshape(w.N, w.heads, w.head_dim)[toks] for a in live[s])
        a = ACC_REL * r.absum(s, toks)
        qr = bf16_round(rope_3d(q, t[toks], y[toks], x[toks], w.rope_split, w.rope_theta))
        kr = bf16_round(rope_3d(k, t[toks], y[toks], x[toks], w.rope_split, w.rope_theta))
        p = w.T - 1 - s
        for got, ref, bound, what in (
                (qf[s][:, toks], qr.transpose(1, 0, 2), _pair_sum(heads(a[:, :w.hd])), "Q"),
                (position_rows(kp, table, p, r.pool.ppc)[:, toks], kr.transpose(1, 0, 2),
                 _pair_sum(heads(a[:, w.hd:2 * w.hd])), "K"),
                (position_rows(vp, table, p, r.pool.ppc)[:, toks], bf16_round(v).transpose(1, 0, 2),
                 heads(a[:, 2 * w.hd:]), "V")):
            d, tt, u = _bound_check(got, ref, bound, "slot %d %s" % (s, what))
            diff, total, worst = diff + d, total + tt, max(worst, u)
    say("sampled elements differing from the oracle: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))
    rows = np.array(sorted(set([0, 255, 256, 4607, 4608, w.N - 1] + list(rng.integers(0, w.N, 10)))))
    heads = [0, 7]
    ref = oracle_rows(w, r.k, live, r.clean_for_round(), rows, heads=heads)
    g = gpu_rows(out, w, rows, heads=heads)
    mx, rel = err_stats(g, ref)
    say("attention rows", len(rows), "heads", heads, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2
    assert torch.isfinite(out).all().item()


@pytest.mark.parametrize("name,C", [("tiny", 5), ("edge_s1_h0", 5)])
def test_w8a8_whole_video(name, C):
    """Every round of a short video published through the W8A8 projection,
    from the first fill round to the last drain round: the store's projected
    K/V becomes anchor or history, and each occupied slot matches the oracle's
    fill schedule over the positions that hold a chunk."""
    import wavefront_causal_attention_amd as wf
    from _gpu_round import config_of
    w = W.WORKLOADS[name]
    say("case", name, "W8A8 projection, whole video of", C, "chunks")
    pool = wf.Pool(config_of(w, first_round=0, total_chunks=C))
    q = pool.q_buffer()
    wt, b = W.projection_weights(w)
    w8, sw = wf.quantize_rows_fp8(to_dev(wt, "bf16"))
    wc, ws = quantize_rows_fp8(wt)
    bd = to_dev(b, "bf16")
    clean = {}
    for k in range(C + w.S):
        sch = RoundSchedule(w.S, w.A, w.H, k, fill=True, total_chunks=C)
        present = [s for s in range(w.S + 1) if sch.slot_present(s)]
        lo, hi = present[0], present[-1]
        xs = {s: W.draw_hidden(w, k, s) for s in present}
        x8, sx = wf.quantize_rows_fp8(to_dev(np.concatenate([xs[s] for s in present], 0), "bf16"))
        pool.project_publish_w8a8(0, lo, hi - lo + 1, x8, x8.stride(0), sx, w.hd, w8, sw, bd, q_out=q)
        out = pool.out_buffer("fp32")
        out.fill_(float("nan"))
        pool.attention(0, lo, hi - lo + 1, q, out)
        torch.cuda.synchronize()
        live = [None] * (w.S + 1)
        for s in present:
            c8, s8 = quantize_rows_fp8(xs[s])
            live[s] = tuple(split_qkv(project_qkv_w8a8(c8, s8, wc, ws, b), w.hd))
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


def test_w8a8_14b_sampled_pages():
    """14B-class widths (hidden 5120, 40 heads, 15360 projection outputs): the
    quantiser's 16-vectors-per-lane form on every weight row (codes and scales
    bit-exact against the oracle), and W8A8 pages on sampled tokens of every
    live slot within the summation bound."""
    import wavefront_causal_attention_amd as wf
    w = W.WORKLOADS["wan14b_s4"]
    say("case wan14b_s4, W8A8 projection, sampled tokens")
    r = RoundRunner(w)
    wt, b = W.projection_weights(w)
    w8, sw = wf.quantize_rows_fp8(to_dev(wt, "bf16"))
    xs = [W.draw_hidden(w, r.k, s) for s in range(w.S + 1)]
    x8, sx = wf.quantize_rows_fp8(to_dev(np.concatenate(xs, 0), "bf16"))
    r.pool.project_publish_w8a8(0, 0, w.S + 1, x8, x8.stride(0), sx, w.hd, w8, sw, to_dev(b, "bf16"), q_out=r.q)
    torch.cuda.synchronize()
    wc, ws = quantize_rows_fp8(wt)
    assert np.array_equal(w8.cpu().numpy(), wc) and np.array_equal(sw.cpu().numpy(), ws)
    wabs = np.abs(fp8_e4m3_decode(wc) * ws.astype(np.float64)[:, None])
    rng = np.random.default_rng(23)
    toks = np.array(sorted(set([0, 1, 1559, 1560, w.N - 1] + list(rng.integers(0, w.N, 20)))))
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    kp, vp = read_pages(r.pool, w)
    table = r.pool.table.cpu().numpy()
    qf = bf16_dev_bits_to_f32(r.q)
    x8h, sxh = x8.cpu().numpy(), sx.cpu().numpy()
    heads = lambda m: m.reshape(len(toks), w.heads, w.head_dim).transpose(1, 0, 2)
    diff = total = 0
    worst = 0.0
    for s in range(w.S + 1):
        c8, s8 = quantize_rows_fp8(xs[s][toks])
        rows = s * w.N + toks
        assert np.array_equal(x8h[rows], c8) and np.array_equal(sxh[rows], s8)
        q, k, v = split_qkv(project_qkv_w8a8(c8, s8, wc, ws, b), w.hd)
        a = ACC_REL * (np.abs(fp8_e4m3_decode(c8) * s8.astype(np.float64)[:, None]) @ wabs.T)
        t, y, x = token_grid(sch.slot_chunk(s), w.chunk_frames, w.frame_h, w.frame_w)
        rot = lambda m: bf16_round(rope_3d(m.reshape(len(toks), w.heads, w.head_dim), t[toks], y[toks], x[toks],
                                           w.rope_split, w.rope_theta))
        p = w.T - 1 - s
        for got, ref, bound, what in (
                (qf[s][:, toks], rot(q).transpose(1, 0, 2), _pair_sum(heads(a[:, :w.hd])), "Q"),
                (position_rows(kp, table, p, r.pool.ppc)[:, toks], rot(k).transpose(1, 0, 2),
                 _pair_sum(heads(a[:, w.hd:2 * w.hd])), "K"),
                (position_rows(vp, table, p, r.pool.ppc)[:, toks], bf16_round(heads(v)), heads(a[:, 2 * w.hd:]), "V")):
            d, tt, u = _bound_check(got, ref, bound, "slot %d %s" % (s, what))
            diff, total, worst = diff + d, total + tt, max(worst, u)
    say("sampled elements differing from the oracle: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))


@pytest.mark.parametrize("kind", ["bf16", "w8a8"])
def test_projection_with_padded_rows_equals_packed_rows(kind):
    """Hidden-state rows with a padded stride (padding filled with large
    values the kernels must not read) publish exactly what packed rows do."""
    import wavefront_causal_attention_amd as wf
    w = W.WORKLOADS["ragged128"]
    say("case ragged128,", kind, "projection, padded row stride")
    xs = np.concatenate([W.draw_hidden(w, w.steady_round, s) for s in range(w.S + 1)], 0)
    wt, b = W.projection_weights(w)
    wd, bd = to_dev(wt, "bf16"), to_dev(b, "bf16")
    pad = 144                                          # elements (bf16) / codes (e4m3) past each row, 16-byte rows
    xp = np.full((xs.shape[0], w.hd + pad), 3.0e38, dtype=np.float32)
    xp[:, :w.hd] = xs
    outs = []
    for x in (to_dev(xs, "bf16"), to_dev(xp, "bf16")):
        r = RoundRunner(w)
        if kind == "bf16":
            r.pool.project_publish(0, 0, w.S + 1, x, x.stride(0), w.hd, wd, bd, q_out=r.q)
        else:
            w8, sw = wf.quantize_rows_fp8(wd)
            pitch = w.hd + (pad if x.stride(0) > w.hd else 0)
            codes = torch.full((x.shape[0], pitch), 0x7F, dtype=torch.uint8, device="cuda")  # NaN codes in padding
            x8, sx = wf.quantize_rows_fp8(x[:, :w.hd], codes[:, :w.hd])
            r.pool.project_publish_w8a8(0, 0, w.S + 1, x8, x8.stride(0), sx, w.hd, w8, sw, bd, q_out=r.q)
        torch.cuda.synchronize()
        kp, vp = read_pages(r.pool, w)
        outs.append((r.q.clone(), kp, vp, r.pool.table.cpu().numpy(), r.pool.ppc))
    assert torch.equal(outs[0][0], outs[1][0])
    for s in range(w.S + 1):                       # the published positions (anchor and history are not)
        p = w.T - 1 - s
        for i in (1, 2):
            assert np.array_equal(position_rows(outs[0][i], outs[0][3], p, outs[0][4]),
                                  position_rows(outs[1][i], outs[1][3], p, outs[1][4])), (s, i)


@pytest.mark.parametrize("kind,hidden", [("bf16", 256), ("bf16", 640), ("w8a8", 256), ("w8a8", 640)])
def test_projection_hidden_width_other_than_heads_times_dim(kind, hidden):
    """A linear layer whose input width differs from h*d (384 here): Q and the
    pages against the oracle's projection of the same operands, within one
    bf16 ulp plus the summation bound: for bf16 the fp32 one, hidden x 2^-24 x
    sum |x w| for any order of additions; for W8A8 the e4m3 MFMA's."""
    import wavefront_causal_attention_amd as wf
    from oracle import project_qkv
    w = W.WORKLOADS["ragged128"]
    say("case ragged128,", kind, "projection, hidden", hidden)
    rng = np.random.default_rng(1000 + hidden)
    xs = [W.round_to_bf16(rng.standard_normal((w.N, hidden), dtype=np.float32)) for _ in range(w.S + 1)]
    wt = W.round_to_bf16(rng.standard_normal((3 * w.hd, hidden), dtype=np.float32) / np.float32(np.sqrt(hidden)))
    b = W.round_to_bf16(rng.standard_normal(3 * w.hd, dtype=np.float32) * np.float32(0.1))
    r = RoundRunner(w)
    xd, wd, bd = to_dev(np.concatenate(xs, 0), "bf16"), to_dev(wt, "bf16"), to_dev(b, "bf16")
    if kind == "bf16":
        r.pool.project_publish(0, 0, w.S + 1, xd, hidden, hidden, wd, bd, q_out=r.q)
        live = [tuple(split_qkv(project_qkv(x, wt, b), w.hd)) for x in xs]
        wabs = np.abs(wt.astype(np.float64))
        r.absum = lambda s, rows=slice(None): np.abs(xs[s][rows].astype(np.float64)) @ wabs.T
        r.acc_rel = hidden * 2.0 ** -24
    else:
        w8, sw = wf.quantize_rows_fp8(wd)
        x8, sx = wf.quantize_rows_fp8(xd)
        r.pool.project_publish_w8a8(0, 0, w.S + 1, x8, x8.stride(0), sx, hidden, w8, sw, bd, q_out=r.q)
        wc, ws = quantize_rows_fp8(wt)
        q8 = [quantize_rows_fp8(x) for x in xs]
        live = [tuple(split_qkv(project_qkv_w8a8(c, s, wc, ws, b), w.hd)) for c, s in q8]
        wabs = np.abs(fp8_e4m3_decode(wc) * ws.astype(np.float64)[:, None])
        r.absum = lambda s, rows=slice(None): (np.abs(fp8_e4m3_decode(q8[s][0][rows]) *
                                                      q8[s][1][rows].astype(np.float64)[:, None]) @ wabs.T)
    torch.cuda.synchronize()
    diff, total, worst = _check_pages(r, live, range(w.S + 1))
    say("elements differing from the oracle: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))


def test_e4m3_mfma_summation_on_controlled_codes():
    """The tolerance basis of the W8A8 pages, on codes chosen by hand: one
    128-channel stage (two 64-code MFMA k-groups) with unit scales and unit
    V weights, so a V element is the plain sum of its token's codes.
      token 0: 448, -448 and 62 x 2^-9 -> exact 62 x 2^-9 = 0.12109375
      token 1: 448, -448, 448, -448 and 60 x 2^-6 -> exact 0.9375
      token 2: 448 and 63 x 2^-9 (the small ones far below the largest)
      other tokens: random finite codes (Q/K/V weights random finite codes).
    Every published element must lie within one bf16 ulp plus
    ACC_REL * sum |x^ w^| of the exact sum (the bound the other W8A8 tests
    use); the observed values of the cancelling tokens are printed."""
    w = W.WORKLOADS["ragged128"]
    hidden = 128
    say("case ragged128, e4m3 MFMA summation on controlled codes")
    rng = np.random.default_rng(77)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    xs_codes = []
    for s in range(w.S + 1):
        x = rng.choice(finite, size=(w.N, hidden))
        if s == 0:
            x[:3] = 0
            x[0, 0], x[0, 1], x[0, 2:64] = 0x7E, 0xFE, 0x01
            x[1, 0:4], x[1, 4:64] = [0x7E, 0xFE, 0x7E, 0xFE], 0x08
            x[2, 0], x[2, 1:64] = 0x7E, 0x01
        xs_codes.append(x)
    wc = rng.choice(finite, size=(3 * w.hd, hidden))
    wc[2 * w.hd:] = 0x38                                      # V weights: 1.0
    ones = lambda n: np.ones(n, dtype=np.float32)
    r = RoundRunner(w)
    x8 = torch.from_numpy(np.concatenate(xs_codes, 0)).cuda()
    sx = torch.from_numpy(ones((w.S + 1) * w.N)).cuda()
    w8 = torch.from_numpy(wc).cuda()
    sw = torch.from_numpy(ones(3 * w.hd)).cuda()
    r.pool.project_publish_w8a8(0, 0, w.S + 1, x8, x8.stride(0), sx, hidden, w8, sw, None, q_out=r.q)
    torch.cuda.synchronize()
    live = [tuple(split_qkv(project_qkv_w8a8(xs_codes[s], ones(w.N), wc, ones(3 * w.hd), None), w.hd))
            for s in range(w.S + 1)]
    r.live = live
    wabs = np.abs(fp8_e4m3_decode(wc))
    r.absum = lambda s, rows=slice(None): np.abs(fp8_e4m3_decode(xs_codes[s][rows])) @ wabs.T
    diff, total, worst = _check_pages(r, live, range(w.S + 1))
    say("elements differing from the exact sums: %d of %d; worst share of the allowance %.3f" % (diff, total, worst))
    # the cancelling tokens, through slot 0's V pages
    _, vp = read_pages(r.pool, w)
    v0 = position_rows(vp, r.pool.table.cpu().numpy(), w.T - 1, r.pool.ppc)      # [heads, N, d]
    for tok, exact in [(0, 62 * 2.0 ** -9), (1, 60 * 2.0 ** -6), (2, 448 + 63 * 2.0 ** -9)]:
        got = float(v0[0, tok, 0])
        absum = float(np.sum(np.abs(fp8_e4m3_decode(xs_codes[0][tok]))))
        say("token %d: exact %.8f, published %.8f, |error| / sum|x w| = %.3e (allowed %.3e)"
            % (tok, exact, got, abs(got - exact) / absum, ACC_REL))
        assert np.all(v0[:, tok, :] == got)                    # every V channel sums the same codes
        assert abs(got - exact) <= float(_bf16_ulp(np.float64(exact))) + ACC_REL * absum
