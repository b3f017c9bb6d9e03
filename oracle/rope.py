"""3D rotary position embedding in fp64.

The pages only say that K/V are published after "QKV projection and RoPE"
(hyper.ai summary, section "Method", WaveRT paragraph) and that chunks are 3
latent frames of a Wan2.1 model (aikraft.ru metrics table). They do not define
the embedding, so this oracle takes the plain 3D reading:

  * head_dim d is split into contiguous channel ranges for the time, row and
    column axes, (d_t, d_h, d_w), default d_h = d_w = 2*floor(d/6),
    d_t = d - 2*d_h (44/42/42 at d = 128);
  * within an axis range of width d_a, channel pair (2m, 2m+1) is rotated by the
    angle pos_a * theta^(-2m/d_a), m = 0 .. d_a/2 - 1;
  * token n of a chunk is latent frame n // (H_p*W_p), patch row
    (n // W_p) % H_p and patch column n % W_p; the time position is
    chunk_frames * chunk_id + frame.
"""
from __future__ import annotations

import numpy as np


def rope_split(d: int, split=None) -> tuple:
    if split is not None:
        split = tuple(int(x) for x in split)
        if sum(split) != d or any(x % 2 for x in split):
            raise ValueError("rope split must be even widths summing to head_dim")
        return split
    dh = 2 * (d // 6)
    return (d - 2 * dh, dh, dh)


def token_grid(chunk_id: int, chunk_frames: int, frame_h: int, frame_w: int):
    """(t, y, x) positions of the chunk's tokens, frame-major then row then column."""
    N = chunk_frames * frame_h * frame_w
    n = np.arange(N, dtype=np.int64)
    f = n // (frame_h * frame_w)
    y = (n // frame_w) % frame_h
    x = n % frame_w
    t = chunk_frames * chunk_id + f
    return t, y, x


def rope_3d(v: np.ndarray, t, y, x, split, theta: float) -> np.ndarray:
    """Rotate v[..., N, heads, d] (fp64) by the 3D positions of its N tokens."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    off = 0
    for pos, da in zip((t, y, x), split):
        if da == 0:
            continue
        m = np.arange(da // 2, dtype=np.float64)
        omega = float(theta) ** (-2.0 * m / da)                  # [da/2]
        phi = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]   # [N, da/2]
        c = np.cos(phi)[:, None, :]                              # broadcast over heads
        s = np.sin(phi)[:, None, :]
        ev = v[..., off:off + da:2]
        od = v[..., off + 1:off + da:2]
        out[..., off:off + da:2] = ev * c - od * s
        out[..., off + 1:off + da:2] = ev * s + od * c
        off += da
    return out
