"""Pins of the oracle's QKV projection (oracle/projection.py) against brute
force, closed forms and the pages' printed model widths."""
import json
import os

import numpy as np

from oracle import project_qkv, split_qkv
import wf_inputs as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_projection_equals_python_loops():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((6, 5))
    b = rng.standard_normal(6)
    y = project_qkv(x, w, b)
    for n in range(3):
        for o in range(6):
            acc = b[o]
            for c in range(5):
                acc += x[n, c] * w[o, c]
            assert abs(y[n, o] - acc) <= 1e-12


def test_stacked_identities_give_q_k_v_by_closed_form():
    rng = np.random.default_rng(6)
    hd = 8
    x = rng.standard_normal((4, hd))
    eye = np.eye(hd)
    q, k, v = split_qkv(project_qkv(x, np.concatenate([eye, 2 * eye, -eye], 0)), hd)
    assert np.array_equal(q, x) and np.array_equal(k, 2 * x) and np.array_equal(v, -x)


def test_one_hot_rows_select_input_channels_in_output_order():
    hd = 6
    src = np.array([5, 0, 3, 1, 4, 2, 2, 2, 0, 1, 5, 3, 4, 4, 1, 0, 3, 5])   # input channel per output channel
    w = np.zeros((3 * hd, hd))
    w[np.arange(3 * hd), src] = 1.0
    x = np.arange(2 * hd, dtype=np.float64).reshape(2, hd) + 1.0
    y = project_qkv(x, w)
    assert np.array_equal(y, x[:, src])
    q, k, v = split_qkv(y, hd)
    assert np.array_equal(q, x[:, src[:hd]]) and np.array_equal(v, x[:, src[2 * hd:]])


def test_bias_alone_and_linearity():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((9, 3))
    b = rng.standard_normal(9)
    assert np.array_equal(project_qkv(np.zeros((2, 3)), w, b), np.tile(b, (2, 1)))
    x1, x2 = rng.standard_normal((4, 3)), rng.standard_normal((4, 3))
    lhs = project_qkv(2.5 * x1 + x2, w)
    rhs = 2.5 * project_qkv(x1, w) + project_qkv(x2, w)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12


def test_workload_projection_widths_follow_table11():
    """hidden = heads x 128 for the Wan2.1 models (Table 11); the projection
    maps it to 3 x heads x head_dim."""
    t11 = json.load(open(os.path.join(GOLDEN, "table11_shapes.json")))["models"]
    for name, model in (("wan1.3b_s4", "1.3B"), ("wan14b_s4", "14B")):
        w = W.WORKLOADS[name]
        assert w.heads == t11[model]["heads"] and w.hd == t11[model]["hidden"]
        wt, b = W.projection_weights(W.WORKLOADS["tiny"])
        assert wt.shape == (3 * W.WORKLOADS["tiny"].hd, W.WORKLOADS["tiny"].hd) and b.shape == (wt.shape[0],)


# ---- W8A8: per-row e4m3 quantiser and the projection of dequantised operands

from fractions import Fraction

from oracle import FP8_E4M3_MAX, fp8_e4m3_decode, project_qkv_w8a8, quantize_rows_fp8

_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])     # the 254 finite codes
_VALS = fp8_e4m3_decode(_CODES)


def _nearest_code_brute(q):
    """Nearest finite e4m3 value by exhaustive search; ties to the even code;
    beyond +-448 the largest finite value of that sign; zero is code 0."""
    if q == 0:
        return 0
    d = np.abs(_VALS - np.clip(q, -FP8_E4M3_MAX, FP8_E4M3_MAX))
    best = np.flatnonzero(d == d.min())
    best = [c for c in _CODES[best] if (c >> 7) == (1 if q < 0 else 0)] or list(_CODES[best])
    even = [c for c in best if c % 2 == 0]
    return int((even or best)[0])


def _row_data(rng, rows, cols):
    x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    x[1, :] = 0.0                                              # an all-zero row
    x[2, 3] = 1e4 * np.abs(x[2]).max()                         # one outlier: the rest goes subnormal
    return x.astype(np.float32).astype(np.float64)


def test_row_quantiser_codes_are_the_nearest_e4m3_by_exhaustive_search():
    rng = np.random.default_rng(31)
    x = _row_data(rng, 6, 40)
    codes, scales = quantize_rows_fp8(x)
    for r in range(x.shape[0]):
        q = x[r].astype(np.float32) / scales[r]                # the fp32 quotient the reading names
        for c in range(x.shape[1]):
            assert codes[r, c] == _nearest_code_brute(float(q[c])), (r, c, float(q[c]))


def test_row_quantiser_ties_round_to_even_codes():
    # row scale 1 (absmax 448); values exactly halfway between neighbours
    vals = [448.0, 8.5, 9.5, 0.5 * (2 ** -9), 1.5 * (2 ** -9), 1.0625, -1.0625, 240.0 + 8.0]
    codes, scales = quantize_rows_fp8(np.array([vals]))
    assert scales[0] == np.float32(1.0)
    dec = fp8_e4m3_decode(codes[0])
    assert list(dec) == [448.0, 8.0, 10.0, 0.0, 2.0 * 2 ** -9, 1.0, -1.0, 256.0]
    assert all(int(c) % 2 == 0 for c in codes[0][1:])


def test_row_quantiser_scales_absmax_zero_rows_and_row_independence():
    rng = np.random.default_rng(32)
    x = _row_data(rng, 5, 33)
    codes, scales = quantize_rows_fp8(x)
    for r in range(5):
        a = np.float32(np.abs(x[r]).max())
        if a == 0:
            assert scales[r] == 1.0 and not codes[r].any()
            continue
        assert scales[r] == a / np.float32(448.0)
        i = int(np.argmax(np.abs(x[r])))
        assert abs(fp8_e4m3_decode(codes[r, i])) == 448.0      # the absmax element saturates exactly
    # scaling one row by a power of two scales only that row's scale; codes unchanged
    y = x.copy()
    y[3] *= 2.0 ** 11
    c2, s2 = quantize_rows_fp8(y)
    assert np.array_equal(c2, codes)
    assert s2[3] == scales[3] * np.float32(2.0 ** 11)
    assert np.array_equal(np.delete(s2, 3), np.delete(scales, 3))


def test_w8a8_projection_equals_exact_rational_arithmetic():
    rng = np.random.default_rng(33)
    xc = rng.choice(_CODES, (3, 7)).astype(np.uint8)
    wc = rng.choice(_CODES, (5, 7)).astype(np.uint8)
    sx = rng.uniform(1e-3, 1e-1, 3).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, 5).astype(np.float32)
    b = rng.standard_normal(5)
    y = project_qkv_w8a8(xc, sx, wc, sw, b)
    for n in range(3):
        for o in range(5):
            acc = Fraction(float(b[o]))
            mag = abs(Fraction(float(b[o])))
            for c in range(7):
                t = (Fraction(float(fp8_e4m3_decode(xc[n, c]))) * Fraction(float(sx[n])) *
                     Fraction(float(fp8_e4m3_decode(wc[o, c]))) * Fraction(float(sw[o])))
                acc += t
                mag += abs(t)
            assert abs(Fraction(float(y[n, o])) - acc) <= mag * Fraction(1, 2 ** 50), (n, o)


def test_w8a8_projection_within_the_e4m3_error_bound_of_the_unquantised_one():
    """Each dequantised operand is within half an e4m3 step of the input:
    relative 2^-4 for normals, absolute scale * 2^-10 below 2^-6 * scale; the
    product bound follows term by term. A scale applied along the wrong axis,
    a dropped scale or a transposed operand breaks it by orders of magnitude."""
    rng = np.random.default_rng(34)
    x = rng.standard_normal((16, 64)) * np.exp2(rng.integers(-3, 4, (16, 1)))
    w = rng.standard_normal((24, 64)) * np.exp2(rng.integers(-6, 0, (24, 1)))
    x[0, 5] = 40.0                                  # an outlier token row
    b = rng.standard_normal(24)
    xc, sx = quantize_rows_fp8(x)
    wc, sw = quantize_rows_fp8(w)
    yq = project_qkv_w8a8(xc, sx, wc, sw, b)
    y = project_qkv(x, w, b)
    ex = 2.0 ** -4 * np.abs(x) + sx.astype(np.float64)[:, None] * 2.0 ** -10
    ew = 2.0 ** -4 * np.abs(w) + sw.astype(np.float64)[:, None] * 2.0 ** -10
    bound = ex @ np.abs(w).T + np.abs(x) @ ew.T + ex @ ew.T
    assert np.all(np.abs(yq - y) <= bound * (1 + 1e-12) + 1e-12)
    assert np.max(np.abs(yq - y)) > 0                # the quantisation is not a no-op
    # the dequantised operands themselves, element by element
    xd = fp8_e4m3_decode(xc) * sx.astype(np.float64)[:, None]
    assert np.all(np.abs(xd - x) <= ex * (1 + 1e-12))


def test_row_quantiser_decides_codes_on_the_fp32_quotient():
    """The code is decided on the correctly rounded fp32 quotient x / scale.
    These bf16 rows put that quotient next to an e4m3 midpoint, where
    multiplying by the fp32 reciprocal of the scale instead lands one code up."""
    x = np.array([[1.1875, 0.111328125], [2.375, 0.890625], [0.0673828125, -0.050537109375]])
    codes, scales = quantize_rows_fp8(x)
    for r in range(3):
        q = np.float32(x[r, 1]) / scales[r]
        assert codes[r, 1] == _nearest_code_brute(float(q))
        recip = np.float32(x[r, 1]) * (np.float32(1.0) / scales[r])
        assert _nearest_code_brute(float(recip)) == codes[r, 1] + 1
    assert [int(c) for c in codes[:, 1]] == [98, 114, 250]
