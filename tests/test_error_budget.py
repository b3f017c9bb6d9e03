"""Error budget of the parity bars, on the CPU.

The attention kernel rounds in known places: Q and K are the published bf16
pages (or e4m3 codes), scores accumulate in fp32, P = exp2(scaled score -
scaled row max) is rounded to bf16 before the PV product, the row sum adds the
same rounded P in fp32, and O = (P V) / sum in fp32. A numpy emulation of those
steps, run against the fp64 oracle on the same inputs, shows what the bars
leave room for and why each comparison uses the storage model it does:

* bf16: the emulation is within the bar (max-abs 1e-2, rel-L2 5e-3) against
  the oracle on the same bf16 pages, with a visible error from the bf16 P
  rounding (about 2^-9 / sqrt(3) relative);
* channel outliers in Q and K (the 14B-class workload): rounding the rotated
  Q and K to bf16 alone moves O past the bar against unrounded inputs, so bf16
  parity is judged against the published pages (storage "bf16");
* fp8: e4m3 quantisation alone moves O past the fp8 bar (rel-L2 1.5e-2)
  against unquantised inputs, so fp8 parity is judged against the quantised
  pages (storage "fp8"), where the emulation is well within it.
"""
import dataclasses
import math

import numpy as np

import wf_inputs as W
from oracle import RoundSchedule, bf16_round, oracle_round, rotated_context

BF16_BAR = (1e-2, 5e-3)
FP8_BAR = (3e-2, 1.5e-2)


def _round_inputs(w, k):
    sch = RoundSchedule(w.S, w.A, w.H, k)
    live = [W.draw(w, k, s) for s in range(w.S + 1)]
    clean = {c: W.stored_draw(w, c)[1:] for c in sch.chunk_ids()[:w.A + w.H]}
    return live, clean


def _emulated_kernel(Qs, ctx_k, ctx_v, w):
    """Per slot s and head: the kernel's arithmetic over the legal prefix
    (positions 0 .. T-1-s) of the stored pages Qs [S+1, N, h, d], ctx_* [T, N, h, d]."""
    S1, N, h, d = Qs.shape
    c = np.float32(math.log2(math.e) / math.sqrt(d))
    out = np.zeros(Qs.shape, dtype=np.float64)
    for s in range(S1):
        npos = w.T - s
        for hh in range(h):
            q = Qs[s, :, hh, :].astype(np.float32)
            kk = ctx_k[:npos, :, hh, :].reshape(npos * N, d).astype(np.float32)
            vv = ctx_v[:npos, :, hh, :].reshape(npos * N, d).astype(np.float32)
            sc = q @ kk.T                                            # fp32 scores
            m = sc.max(axis=1, keepdims=True)
            p = np.exp2(sc * c - m * c).astype(np.float32)
            pb = bf16_round(p).astype(np.float32)                    # P as the PV MFMA sees it
            l = pb.sum(axis=1, dtype=np.float32)
            out[s, :, hh, :] = (pb @ vv) / l[:, None]
    return out


def _err(a, b):
    d = a - b
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / np.linalg.norm(b))


def test_bf16_bar_leaves_room_for_the_kernels_rounding():
    w = W.WORKLOADS["ragged128"]
    k = w.steady_round
    live, clean = _round_inputs(w, k)
    Qs, ck, cv, _ = rotated_context(w, k, live, clean, storage="bf16")
    emu = _emulated_kernel(Qs, ck, cv, w)
    ref = oracle_round(w, k, live, clean, storage="bf16")
    mx, rel = _err(emu, ref)
    assert mx <= BF16_BAR[0] / 4 and rel <= BF16_BAR[1] / 2, (mx, rel)
    # the bf16 P rounding is a real error of about 2^-9 / sqrt(3) relative
    assert 0.3 * 2.0 ** -9 / math.sqrt(3) <= rel <= 3 * 2.0 ** -9 / math.sqrt(3), rel


def test_qk_outliers_need_the_published_pages_as_reference():
    w = dataclasses.replace(W.WORKLOADS["ragged128"], outlier_frac=0.02, outlier_scale=20.0)
    assert W.outlier_channels(w).size >= 4
    k = w.steady_round
    live, clean = _round_inputs(w, k)
    Qs, ck, cv, _ = rotated_context(w, k, live, clean, storage="bf16")
    emu = _emulated_kernel(Qs, ck, cv, w)
    on_pages = oracle_round(w, k, live, clean, storage="bf16")
    exact = oracle_round(w, k, live, clean, storage="exact")
    mx_p, rel_p = _err(emu, on_pages)
    mx_x, rel_x = _err(emu, exact)
    assert mx_p <= BF16_BAR[0] and rel_p <= BF16_BAR[1], (mx_p, rel_p)
    assert mx_x > BF16_BAR[0] or rel_x > BF16_BAR[1], (mx_x, rel_x)
    # the rotated-Q/K rounding alone, with exact softmax arithmetic, already does it
    mx_r, rel_r = _err(on_pages, exact)
    assert mx_r > BF16_BAR[0] or rel_r > BF16_BAR[1], (mx_r, rel_r)


def test_fp8_bar_is_judged_against_the_quantised_pages():
    w = W.WORKLOADS["ragged_fp8"]
    k = w.steady_round
    live, clean = _round_inputs(w, k)
    Qs, ck, cv, _ = rotated_context(w, k, live, clean, storage="fp8")
    emu = _emulated_kernel(Qs, ck, cv, w)
    on_codes = oracle_round(w, k, live, clean, storage="fp8")
    exact = oracle_round(w, k, live, clean, storage="exact")
    mx_q, rel_q = _err(on_codes, exact)
    assert rel_q > FP8_BAR[1], rel_q                       # e4m3 quantisation alone
    mx, rel = _err(emu, on_codes)
    assert mx <= FP8_BAR[0] / 4 and rel <= FP8_BAR[1] / 4, (mx, rel)
