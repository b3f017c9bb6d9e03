"""One wavefront round end to end: schedule -> RoPE -> storage -> attention.

Order of steps follows the WaveRT description (hyper.ai summary, section
"Method"; aikraft.ru "Early Publication"): K/V are published after QKV
projection and RoPE, into ordered attention slots (e-cogni.com.br, "Como
funciona"), and attention then runs over the ordered context.

Storage models of the published Q/K pages:
  "exact" - no rounding (self-checks);
  "bf16"  - post-RoPE Q and K rounded to bfloat16; V rounded to bfloat16
            (the page format; exact for bf16 inputs);
  "fp8"   - post-RoPE Q quantised per 64-token block to e4m3; K has its
            per-(chunk, head) fp32 channel mean removed, is quantised the same
            way, and the mean is added back: K_hat = deq(K8) + mean; V bf16.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, fp8_block_quantize, fp8_e4m3_decode
from .rope import rope_3d, token_grid
from .schedule import RoundSchedule, slot_position
from .attention import round_attention


def rotate_chunk(shape, chunk_id: int, x) -> np.ndarray:
    """Post-RoPE fp64 [N, heads, d] of a chunk's pre-RoPE projection x[N, heads*d]."""
    x = np.asarray(x, dtype=np.float64).reshape(shape.N, shape.heads, shape.head_dim)
    t, y, xx = token_grid(chunk_id, shape.chunk_frames, shape.frame_h, shape.frame_w)
    return rope_3d(x, t, y, xx, shape.rope_split, shape.rope_theta)


def _fp8_q(qr: np.ndarray) -> np.ndarray:
    out = np.empty_like(qr)
    for h in range(qr.shape[1]):
        codes, sc = fp8_block_quantize(qr[:, h, :])
        out[:, h, :] = fp8_e4m3_decode(codes) * np.repeat(sc.astype(np.float64), 64)[:qr.shape[0], None]
    return out


def _fp8_k(kr: np.ndarray) -> np.ndarray:
    out = np.empty_like(kr)
    for h in range(kr.shape[1]):
        mu = np.mean(kr[:, h, :], axis=0).astype(np.float32).astype(np.float64)   # [d]
        codes, sc = fp8_block_quantize(kr[:, h, :] - mu[None, :])
        deq = fp8_e4m3_decode(codes) * np.repeat(sc.astype(np.float64), 64)[:kr.shape[0], None]
        out[:, h, :] = deq + mu[None, :]
    return out


def store(x: np.ndarray, storage: str, kind: str) -> np.ndarray:
    if storage == "exact":
        return x
    if storage == "bf16":
        return bf16_round(x)
    if storage == "fp8":
        return _fp8_q(x) if kind == "q" else _fp8_k(x)
    raise ValueError("unknown storage model " + storage)


def rotated_context(shape, k, live, clean, storage="bf16", sched=None):
    """Post-storage Q of live slots and K/V of every context position.

    live:  sequence over slots s = 0..S of pre-RoPE (q, k, v) [N, heads*d]
           (None for a slot that holds no chunk in a fill or drain round)
    clean: mapping chunk_id -> pre-RoPE (k, v) for the anchor and history chunks
    sched: the round's RoundSchedule (default: a steady-state round k)
    Returns (Qs [S+1, N, heads, d], ctx_k [T, ...], ctx_v [T, ...], chunk_ids);
    positions and slots without a chunk are NaN.
    """
    S, A, H = shape.S, shape.A, shape.H
    sched = RoundSchedule(S, A, H, k) if sched is None else sched
    T = sched.T
    N, h, d = shape.N, shape.heads, shape.head_dim
    ids = sched.chunk_ids()
    pos_of_slot = {slot_position(s, S, A, H): s for s in range(S + 1)}
    ctx_k = np.empty((T, N, h, d))
    ctx_v = np.empty((T, N, h, d))
    for p in range(T):
        c = ids[p]
        if not sched.present(p):
            ctx_k[p] = np.nan
            ctx_v[p] = np.nan
            continue
        if p in pos_of_slot:
            _, kk, vv = live[pos_of_slot[p]]
        else:
            kk, vv = clean[c]
        ctx_k[p] = store(rotate_chunk(shape, c, kk), storage, "k")
        vv = np.asarray(vv, dtype=np.float64).reshape(N, h, d)
        ctx_v[p] = vv if storage == "exact" else bf16_round(vv)     # V pages are bf16
    Qs = np.empty((S + 1, N, h, d))
    for s in range(S + 1):
        if not sched.slot_present(s):
            Qs[s] = np.nan
            continue
        Qs[s] = store(rotate_chunk(shape, sched.slot_chunk(s), live[s][0]), storage, "q")
    return Qs, ctx_k, ctx_v, ids


def oracle_round(shape, k, live, clean, storage="bf16", rows=None, slots=None, mask="wavefront",
                 fill=False, total_chunks=None):
    """O[slots, rows, heads, d] (fp64) of one wavefront round.

    See rotated_context for the inputs; rows/slots restrict what is evaluated;
    mask selects the live-slot visibility (see schedule.live_mask); fill and
    total_chunks admit the rounds that fill and drain the pipeline, where each
    slot reads only the positions that hold a chunk (slots without one are NaN).
    """
    sched = RoundSchedule(shape.S, shape.A, shape.H, k, fill=fill, total_chunks=total_chunks)
    Qs, ctx_k, ctx_v, _ = rotated_context(shape, k, live, clean, storage, sched=sched)
    legal = {s: sched.legal_present(s, mask) for s in range(shape.S + 1)}
    out = round_attention(Qs, ctx_k, ctx_v, shape.S, shape.A, shape.H, rows=rows, slots=slots, kind=mask,
                          legal=legal)
    slots = list(range(shape.S + 1)) if slots is None else list(slots)
    for i, s in enumerate(slots):
        if not sched.slot_present(s):
            out[i] = np.nan
    return out
