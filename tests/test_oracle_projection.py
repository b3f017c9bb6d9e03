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
