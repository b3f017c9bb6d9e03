"""Masked softmax attention over the ordered wavefront context, fp64.

Wave Forcing, hyper.ai summary, section "Method": full attention inside each
chunk, chunk-wise causal attention along time, mask M_WF(s, j) = 1[j >= s] over
the query's own slot and every cleaner one. e-cogni.com.br article, "Como
funciona": the context is anchor | clean history | live store | denoising K/V
and a query slot sees K/V only of itself and of cleaner predecessors.

The result is plain scaled-dot-product attention; the scale is 1/sqrt(d)
(the pages do not state it; this is the standard reading).
"""
from __future__ import annotations

import numpy as np

from .schedule import legal_positions, live_mask, slot_position


def masked_softmax_attention(q, k, v, scale, mask=None, return_p=False):
    """softmax(q k^T * scale, masked to -inf where mask is False) v, all fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sc = (q @ k.T) * scale
    if mask is not None:
        sc = np.where(mask, sc, -np.inf)
    m = np.max(sc, axis=-1, keepdims=True)
    e = np.exp(sc - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    o = p @ v
    return (o, p) if return_p else o


def slot_attention(q, k_ctx, v_ctx, scale, block=512, return_p=False):
    """Unmasked attention of q[M, d] over one slot's gathered legal context."""
    if return_p:
        return masked_softmax_attention(q, k_ctx, v_ctx, scale, return_p=True)
    out = np.empty((q.shape[0], v_ctx.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], block):
        out[r0:r0 + block] = masked_softmax_attention(q[r0:r0 + block], k_ctx, v_ctx, scale)
    return out


def round_attention(Qs, ctx_k, ctx_v, S, A, H, rows=None, slots=None, scale=None, kind="wavefront",
                    legal=None):
    """Per-slot gather formulation.

    Qs:     [S+1, N, heads, d]     post-storage queries of live slots s = 0..S
    ctx_k:  [T, N, heads, d]       post-storage keys by context position
    ctx_v:  [T, N, heads, d]       values by context position
    rows:   optional query row indices (within a chunk) to evaluate
    slots:  optional subset of slots
    legal:  optional mapping slot -> context positions it reads (default: the
            live mask's legal positions)
    Returns O[S+1 (or len(slots)), len(rows) or N, heads, d] in fp64.
    """
    Qs = np.asarray(Qs)
    d = Qs.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    slots = list(range(S + 1)) if slots is None else list(slots)
    rows = np.arange(Qs.shape[1]) if rows is None else np.asarray(rows)
    heads = Qs.shape[2]
    out = np.zeros((len(slots), len(rows), heads, ctx_v.shape[-1]), dtype=np.float64)
    for si, s in enumerate(slots):
        pos = legal[s] if legal is not None else legal_positions(s, S, A, H, kind)
        if not pos:                                    # a slot with no chunk this round
            out[si] = np.nan
            continue
        for h in range(heads):
            kc = np.concatenate([ctx_k[p][:, h, :] for p in pos], axis=0)
            vc = np.concatenate([ctx_v[p][:, h, :] for p in pos], axis=0)
            out[si, :, h, :] = slot_attention(Qs[s][rows, h, :], kc, vc, scale)
    return out


def dense_round_attention(Qs, ctx_k, ctx_v, S, A, H, scale=None, return_p=False, kind="wavefront"):
    """Second formulation: one dense softmax per head over every query row of the
    round against every key of the context, with the live mask (M_WF by
    default) expanded to a token mask. Small inputs only.
    """
    Qs = np.asarray(Qs, dtype=np.float64)
    S1, N, heads, d = Qs.shape
    T = ctx_k.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    M = live_mask(S, kind)
    # chunk-level visibility [query slot, context position]
    vis = np.zeros((S + 1, T), dtype=bool)
    for s in range(S + 1):
        for p in range(T):
            if p < A + H:
                vis[s, p] = True                          # anchor and clean history
            else:
                for j in range(S + 1):
                    if slot_position(j, S, A, H) == p:
                        vis[s, p] = bool(M[s, j])
    tok_mask = np.repeat(np.repeat(vis, N, axis=0), N, axis=1)   # [(S+1)N, T N]
    out = np.zeros((S + 1, N, heads, ctx_v.shape[-1]))
    ps = []
    for h in range(heads):
        q = Qs[:, :, h, :].reshape((S + 1) * N, d)
        k = ctx_k[:, :, h, :].reshape(T * N, d)
        v = ctx_v[:, :, h, :].reshape(T * N, -1)
        o, p = masked_softmax_attention(q, k, v, scale, mask=tok_mask, return_p=True)
        out[:, :, h, :] = o.reshape(S + 1, N, -1)
        ps.append(p)
    return (out, ps, tok_mask) if return_p else out
