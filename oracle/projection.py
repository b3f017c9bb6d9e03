"""QKV projection ahead of RoPE and publish, fp64.

The pages place the publish right after the QKV projection and RoPE (hyper.ai
summary, section "Method", WaveRT paragraph; e-cogni.com.br, "Como
funciona"; aikraft.ru, "Early Publication"), and give the model widths: the
hidden size is heads x 128 and the attention works on heads x 128 channels
(thelatestinai.com listing, Table 11). The projection is a linear layer from
the hidden state to the concatenated [Q | K | V], each heads x head_dim wide:

    qkv[n, o] = sum_c x[n, c] * w[o, c] + b[o]

with w stored [out, in] (3*h*d rows, one per output channel) and b optional.
Q is output channels [0, h*d), K [h*d, 2*h*d), V [2*h*d, 3*h*d), head-major
inside each, which is the layout of a fused [tokens, 3*h*d] projection output.
The pages say nothing of normalisation between the projection and RoPE; none
is applied (the plainest reading).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def project_qkv(x, w, b=None) -> np.ndarray:
    """[tokens, 3*h*d] fp64 = x @ w^T + b for x [tokens, C], w [3*h*d, C], b [3*h*d]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)[None, :]
    return y


def split_qkv(y, hd: int):
    """(q, k, v), each [tokens, h*d], from a [tokens, 3*h*d] projection output."""
    return y[:, :hd], y[:, hd:2 * hd], y[:, 2 * hd:3 * hd]
