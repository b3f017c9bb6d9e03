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

W8A8. The pages name W8A8 quantisation of weights and activations as a local
optimisation of the runtime (e-cogni.com.br, "Como funciona") and measure it
paired with SageAttention (thelatestinai.com listing, Table 6, the Sage+W8A8
rows); they give neither the 8-bit format nor the scale granularity. Reading
taken here: both operands in OCP fp8 e4m3 (the 8-bit format of the quantised
attention path), one scale per row of each operand - per token for the
activations, per output channel for the weights, which are stored [out, in] so
an output channel is a weight row - with scale = absmax / 448, and the
projection is the plain product of the dequantised operands:

    qkv[n, o] = sum_c (sx[n] * x8[n, c]) * (sw[o] * w8[o, c]) + b[o]

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .numerics import FP8_E4M3_MAX, fp8_e4m3_decode, fp8_e4m3_encode


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


def quantize_rows_fp8(x):
    """Per-row e4m3 quantisation of x [rows, cols], read at fp32 (bf16 inputs
    are exact there). Each row gets the fp32 scale fp32(absmax) / 448 (1 for an
    all-zero row); its codes are the e4m3 encoding (nearest, ties to even,
    saturating) of the fp32 quotient x / scale. Returns (codes uint8
    [rows, cols], scales float32 [rows])."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    rows = x32.shape[0]
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.ones(rows, dtype=np.float32)
    for r in range(rows):
        amax = np.max(np.abs(x32[r])) if x32.shape[1] else np.float32(0)
        s = amax / np.float32(FP8_E4M3_MAX) if amax > 0 else np.float32(1.0)
        scales[r] = s
        codes[r] = fp8_e4m3_encode((x32[r] / s).astype(np.float64))
    return codes, scales


def project_qkv_w8a8(x_codes, x_scales, w_codes, w_scales, b=None) -> np.ndarray:
    """[tokens, 3*h*d] fp64 projection of the dequantised operands:
    (sx * x8) @ (sw * w8)^T + b, x8 [tokens, C] with sx [tokens], w8
    [3*h*d, C] with sw [3*h*d]."""
    xd = fp8_e4m3_decode(x_codes) * np.asarray(x_scales, dtype=np.float64)[:, None]
    wd = fp8_e4m3_decode(w_codes) * np.asarray(w_scales, dtype=np.float64)[:, None]
    return project_qkv(xd, wd, b)
