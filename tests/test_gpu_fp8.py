"""GPU parity of the fp8-e4m3 QK path against the fp64 oracle (storage "fp8").

Bar: max-abs <= 3e-2 and relative L2 <= 1.5e-2 (fp32 output mode) against the
oracle evaluated on the same quantised Q/K (the quantiser is part of the
method of this path). The quantised pages themselves are compared bit for
bit: chunk means (fp32), block scales and every e4m3 code equal the oracle's,
whose decisions are taken on the same fp64 values.
"""
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import (RoundSchedule, fp8_block_quantize, fp8_e4m3_decode, oracle_round,
                    rotate_chunk)

from _gpu_round import RoundRunner, err_stats, gpu_rows, oracle_rows

pytestmark = pytest.mark.gpu

FP8_MAX_ABS = 3e-2
FP8_REL_L2 = 1.5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import wavefront_causal_attention_amd as wf
    wf.load()
    yield


def _code_distance(a, b):
    """Steps between e4m3 codes of equal sign (0x00 and 0x80 are both zero)."""
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    za, zb = (a & 0x7F) == 0, (b & 0x7F) == 0
    same_sign = ((a >> 7) == (b >> 7)) | za | zb
    mag = np.abs((a & 0x7F) - (b & 0x7F))
    return np.where(za & zb, 0, np.where(same_sign, mag, (a & 0x7F) + (b & 0x7F)))


@pytest.mark.parametrize("name,heads", [("ragged_fp8", None), ("ragged_fp8_64", None), ("tiny_fp8", None),
                                        ("wan1.3b_s4_fp8", [0, 7, 11])])
def test_fp8_publish_codes_scales_and_means(name, heads):
    w = W.WORKLOADS[name]
    say("case", w.name, "fp8 publish")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
    torch.cuda.synchronize()
    pool = r.pool
    g = pool.geometry
    D, pt, ppc, h = w.head_dim, w.page_tokens, pool.ppc, w.heads
    npages = w.T * ppc
    table = pool.table.cpu().numpy()
    kp = pool.pool[g["k_off"]:g["k_off"] + npages * h * pt * D].cpu().numpy()
    kp = kp.reshape(npages, h, D // 16, pt, 16).transpose(0, 1, 3, 2, 4).reshape(npages, h, pt, D)
    ks = pool.pool[g["kscale_off"]:g["kscale_off"] + npages * h * pt * 4].view(torch.float32)
    ks = ks.cpu().numpy().reshape(npages, h, pt)
    km = pool.pool[g["kmean_off"]:g["kmean_off"] + w.T * h * D * 4].view(torch.float32)
    km = km.cpu().numpy().reshape(w.T, h, D)
    sch = RoundSchedule(w.S, w.A, w.H, r.k)
    clean = r.clean_for_round()
    pos_slot = {w.T - 1 - s: s for s in range(w.S + 1)}
    total = diff = 0
    for p in range(w.T):
        c = sch.chunk_at(p)
        kk = r.live[pos_slot[p]][1] if p in pos_slot else clean[c][0]
        kr = rotate_chunk(w, c, kk)                         # [N, h, d] fp64
        pages = table[p * ppc:(p + 1) * ppc]
        grp = pages[0] // ppc
        codes = np.concatenate([kp[pg] for pg in pages], axis=1)        # [h, N, d]
        scales = np.concatenate([ks[pg] for pg in pages], axis=1)       # [h, N]
        for hh in (range(h) if heads is None else heads):
            mu32 = np.mean(kr[:, hh, :], axis=0).astype(np.float32)
            assert np.array_equal(km[grp, hh], mu32), (p, hh)
            ref_codes, ref_scales = fp8_block_quantize(kr[:, hh, :] - mu32.astype(np.float64))
            tok_scale = np.repeat(ref_scales, 64)[:w.N]
            assert np.array_equal(scales[hh], tok_scale), (p, hh)
            dist = _code_distance(codes[hh], ref_codes)
            total += dist.size
            diff += int(np.count_nonzero(dist))
    # queries
    qcodes = r.q.cpu().numpy()                              # [S+1, h, N, d] uint8
    qsc = r.qs.cpu().numpy()
    for s in range(w.S + 1):
        qr = rotate_chunk(w, sch.slot_chunk(s), r.live[s][0])
        for hh in (range(h) if heads is None else heads):
            ref_codes, ref_scales = fp8_block_quantize(qr[:, hh, :])
            assert np.array_equal(qsc[s, hh, :len(ref_scales)], ref_scales), (s, hh)
            dist = _code_distance(qcodes[s, hh], ref_codes)
            total += dist.size
            diff += int(np.count_nonzero(dist))
    say("fp8 codes differing from the oracle's: %d of %d" % (diff, total))
    assert diff == 0


@pytest.mark.parametrize("name", ["ragged_fp8", "ragged_fp8_64", "tiny_fp8"])
def test_fp8_round_parity_full(name):
    w = W.WORKLOADS[name]
    say("case", w.name, "fp8 full round")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="fp8")
    mx, rel = err_stats(g, ref)
    exact = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="exact")
    mxe, rele = err_stats(g, exact)
    say("fp8 vs storage=fp8: max_abs %.3e rel_l2 %.3e | vs exact: max_abs %.3e rel_l2 %.3e"
        % (mx, rel, mxe, rele))
    assert mx <= FP8_MAX_ABS and rel <= FP8_REL_L2


def test_fp8_noisier_slots_poisoned_with_nan():
    w = W.WORKLOADS["ragged_fp8"]
    say("case", w.name, "fp8 nan poison")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    base = r.attention("fp32").cpu().numpy()
    live = list(r.live)
    s = 2
    nan = np.full((w.N, w.hd), np.nan, dtype=np.float32)
    r.publish_live(live=[(nan, nan, nan)] * s + live[s:], slot_first=0, nslots=s)
    out = r.attention("fp32").cpu().numpy()
    assert np.array_equal(out[s:], base[s:])


@pytest.mark.timeout(900)
def test_fp8_full_size_every_output():
    """Every output of the full-size fp8 round (fused QKV input) against the
    oracle on the same quantised Q/K, the oracle on the host's cores."""
    from oracle.parallel import compare_every_output, host_workers
    w = W.WORKLOADS["wan1.3b_s4_fp8"]
    say("case", w.name, "full size, every output;", host_workers(), "oracle workers")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live(live=W.draw_slots(w, r.k, range(w.S + 1)))
    out = r.attention("fp32").cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim)
    assert np.isfinite(out).all()
    mx, rel, worst, n = compare_every_output(out, w, r.k, "fp8", say=say)
    say(w.name, "every output (%d units): max_abs %.3e rel_l2 %.3e worst unit rel_l2 %.3e"
        % (n, mx, rel, worst))
    assert mx <= FP8_MAX_ABS and rel <= FP8_REL_L2 and worst <= FP8_REL_L2


def test_fp8_all_live_mask_round_parity():
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["ragged_fp8"], live_mask="all")
    say("case", w.name, "fp8 all-live mask")
    r = RoundRunner(w)
    r.seed_clean()
    r.publish_live()
    out = r.attention("fp32")
    g = gpu_rows(out, w, np.arange(w.N))
    assert not np.isnan(g).any()
    ref = oracle_round(w, r.k, r.live, r.clean_for_round(), storage="fp8", mask="all")
    mx, rel = err_stats(g, ref)
    say("fp8 all-live vs storage=fp8: max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= FP8_MAX_ABS and rel <= FP8_REL_L2


@pytest.mark.parametrize("name,C", [("ragged_fp8_64", 5), ("tiny_fp8", 5)])
def test_fp8_fill_and_drain_whole_video(name, C):
    """Every round of a short video on the fp8 QK path: per-tile key scales
    and chunk means follow each chunk to whichever position it occupies while
    the pipeline fills and drains."""
    from _gpu_round import run_whole_video
    w = W.WORKLOADS[name]
    say("case", name, "fp8 whole video of", C, "chunks")

    def check(k, out, live, clean, lo, hi):
        ref = oracle_round(w, k, live, clean, storage="fp8", fill=True, total_chunks=C,
                           slots=range(lo, hi + 1))
        o = out.cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim).astype(np.float64)
        assert np.isnan(np.delete(o, list(range(lo, hi + 1)), axis=0)).all()
        mx, rel = err_stats(o[lo:hi + 1], ref)
        say(name, "round", k, "slots", lo, "..", hi, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= FP8_MAX_ABS and rel <= FP8_REL_L2, (k, mx, rel)

    run_whole_video(w, C, check)
