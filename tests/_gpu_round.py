"""Helpers for the GPU parity tests: drive a pool through the C ABI with seeded
inputs, and evaluate the oracle on the same inputs (never on GPU results)."""
from __future__ import annotations

import numpy as np
import torch

import wf_inputs as W
import wavefront_causal_attention_amd as wf
from oracle import RoundSchedule, oracle_round


def config_of(w: W.Workload, first_round=None, num_layers=1, total_chunks=0):
    return wf.make_config(S=w.S, anchor_chunks=w.A, history_chunks=w.H, heads=w.heads,
                          head_dim=w.head_dim, chunk_frames=w.chunk_frames, frame_h=w.frame_h,
                          frame_w=w.frame_w, page_tokens=w.page_tokens, in_dtype=w.in_dtype,
                          qk_dtype=w.qk_dtype, rope_split=w.rope_split, rope_theta=w.rope_theta,
                          first_round=first_round, num_layers=num_layers, live_mask=w.live_mask,
                          total_chunks=total_chunks)


def to_dev(x: np.ndarray, in_dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if in_dtype == "bf16" else t
    return t.cuda()


def stack_dev(arrs, in_dtype):
    return to_dev(np.concatenate(arrs, axis=0), in_dtype)


class RoundRunner:
    """A pool plus the seeded data published into it, round by round."""

    def __init__(self, w: W.Workload, k0=None, draw=None, stored=None):
        self.w = w
        self.k0 = w.steady_round if k0 is None else k0
        self.draw = draw or (lambda k, s: W.draw(w, k, s))
        self.stored = stored or (lambda c: W.stored_draw(w, c))
        self.pool = wf.Pool(config_of(w, first_round=self.k0))
        self.q = self.pool.q_buffer()
        self.qs = self.pool.q_scale_buffer()
        self.k = self.k0
        self.live = None
        self.clean = {}

    def seed_clean(self):
        """Publish anchor and history of the current round (slots S+1 .. T-1)."""
        w = self.w
        sch = RoundSchedule(w.S, w.A, w.H, self.k)
        ks, vs = [], []
        for slot in range(w.S + 1, w.T):
            c = sch.chunk_at(w.T - 1 - slot)
            _, kk, vv = self.stored(c)
            self.clean[c] = (kk, vv)
            ks.append(kk)
            vs.append(vv)
        kd, vd = stack_dev(ks, w.in_dtype), stack_dev(vs, w.in_dtype)
        self.pool.publish(0, w.S + 1, w.T - w.S - 1, None, kd, vd, w.hd)
        torch.cuda.synchronize()

    def publish_live(self, live=None, slot_first=0, nslots=None):
        w = self.w
        if live is None:
            live = [self.draw(self.k, s) for s in range(w.S + 1)]
        self.live = live
        nslots = w.S + 1 - slot_first if nslots is None else nslots
        sel = live[slot_first:slot_first + nslots]
        if w.fused_qkv:
            fused = np.concatenate([np.concatenate(x, axis=1) for x in sel], axis=0)
            fd = to_dev(fused, w.in_dtype)
            hd = w.hd
            self.pool.publish(0, slot_first, nslots, fd[:, :hd], fd[:, hd:], fd[:, 2 * hd:], 3 * hd,
                              q_out=self.q, q_scales=self.qs)
            self._keep = fd
        else:
            qd = stack_dev([x[0] for x in sel], w.in_dtype)
            kd = stack_dev([x[1] for x in sel], w.in_dtype)
            vd = stack_dev([x[2] for x in sel], w.in_dtype)
            self.pool.publish(0, slot_first, nslots, qd, kd, vd, w.hd, q_out=self.q, q_scales=self.qs)
            self._keep = (qd, kd, vd)

    def attention(self, out_dtype="fp32", slot_first=0, nslots=None):
        w = self.w
        nslots = w.S + 1 - slot_first if nslots is None else nslots
        out = self.pool.out_buffer(out_dtype)
        out.fill_(float("nan"))
        self.pool.attention(0, slot_first, nslots, self.q, out, q_scales=self.qs)
        torch.cuda.synchronize()
        return out

    def advance(self):
        w = self.w
        sch = RoundSchedule(w.S, w.A, w.H, self.k)
        # the store's chunk becomes history with the K/V it was published with
        c = sch.chunk_at(w.A + w.H)
        self.clean[c] = tuple(self.live[w.S][1:])
        self.pool.advance()
        self.k += 1

    def clean_for_round(self):
        sch = RoundSchedule(self.w.S, self.w.A, self.w.H, self.k)
        return {c: self.clean[c] for c in sch.chunk_ids()[:self.w.A + self.w.H]}


def run_whole_video(w, C, check_round):
    """Drive one pool through every round of a C-chunk video, from the first
    fill round to the last drain round, publishing and attending only the
    slots that hold a chunk; check_round(k, out, live, clean, lo, hi) checks
    each round. Anchor and history are never seeded: they are what the store
    slot published in earlier rounds. Every K/V page, key scale and key mean of
    the pool starts as NaN (all bytes 0xFF: NaN in bf16, e4m3 and fp32), so a
    read of a page no chunk was published to shows up in the outputs."""
    pool = wf.Pool(config_of(w, first_round=0, total_chunks=C))
    g = pool.geometry
    for off, nbytes in ((g["k_off"], g["k_layer_bytes"]), (g["v_off"], g["v_layer_bytes"]),
                        (g["kscale_off"], g["kscale_layer_bytes"]), (g["kmean_off"], g["kmean_layer_bytes"])):
        if nbytes > 0:
            pool.pool[off:off + nbytes].fill_(0xFF)
    torch.cuda.synchronize()
    q, qs = pool.q_buffer(), pool.q_scale_buffer()
    clean = {}
    for k in range(C + w.S):
        sch = RoundSchedule(w.S, w.A, w.H, k, fill=True, total_chunks=C)
        assert pool.chunk_ids() == [-1 if x is None else x for x in sch.present_chunk_ids()]
        present = [s for s in range(w.S + 1) if sch.slot_present(s)]
        lo, hi = present[0], present[-1]
        assert present == list(range(lo, hi + 1))
        live = [W.draw(w, k, s) if s in present else None for s in range(w.S + 1)]
        sel = live[lo:hi + 1]
        if w.fused_qkv:
            fd = stack_dev([np.concatenate(x, axis=1) for x in sel], w.in_dtype)
            pool.publish(0, lo, hi - lo + 1, fd[:, :w.hd], fd[:, w.hd:2 * w.hd], fd[:, 2 * w.hd:], 3 * w.hd,
                         q_out=q, q_scales=qs)
        else:
            pool.publish(0, lo, hi - lo + 1, stack_dev([x[0] for x in sel], w.in_dtype),
                         stack_dev([x[1] for x in sel], w.in_dtype), stack_dev([x[2] for x in sel], w.in_dtype),
                         w.hd, q_out=q, q_scales=qs)
        out = pool.out_buffer("fp32")
        out.fill_(float("nan"))
        pool.attention(0, lo, hi - lo + 1, q, out, q_scales=qs)
        torch.cuda.synchronize()
        check_round(k, out, live, {c: clean[c] for c in sch.present_chunk_ids()[:w.A + w.H] if c is not None},
                    lo, hi)
        if w.S in present:                       # the store's chunk becomes anchor or history
            clean[sch.slot_chunk(w.S)] = tuple(live[w.S][1:])
        if k < C - 1 + w.S:
            pool.advance()


def head_subset(w: W.Workload, heads):
    """Workload restricted to some heads (attention is independent per head)."""
    import dataclasses
    return dataclasses.replace(w, heads=len(heads))


def take_heads(x: np.ndarray, w: W.Workload, heads):
    d = w.head_dim
    return np.concatenate([x[:, h * d:(h + 1) * d] for h in heads], axis=1)


def oracle_rows(w, k, live, clean, rows, heads=None, storage=None, slots=None):
    """Oracle O[slots, rows, heads, d] on the same seeded inputs."""
    storage = storage or w.qk_dtype
    if heads is not None:
        ws = head_subset(w, heads)
        live = [tuple(take_heads(a, w, heads) for a in x) for x in live]
        clean = {c: tuple(take_heads(a, w, heads) for a in kv) for c, kv in clean.items()}
        w = ws
    return oracle_round(w, k, live, clean, storage=storage, rows=rows, slots=slots, mask=w.live_mask)


def gpu_rows(out: torch.Tensor, w: W.Workload, rows, heads=None, slots=None):
    o = out.float().cpu().numpy().reshape(w.S + 1, w.N, w.heads, w.head_dim)
    o = o[:, rows]
    if heads is not None:
        o = o[:, :, heads]
    if slots is not None:
        o = o[slots]
    return o.astype(np.float64)


def err_stats(gpu: np.ndarray, ref: np.ndarray):
    diff = gpu - ref
    return float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / np.linalg.norm(ref))


def bf16_dev_bits_to_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor (any int16 view) -> float32 numpy of the same values."""
    return (t.view(torch.int16).cpu().numpy().astype(np.int32).astype(np.uint32) << 16).view(np.float32)


def read_pages(pool, w: W.Workload, layer=0):
    """K and V pages of one layer as float32 [page, head, token, d]."""
    g = pool.geometry
    npages = w.T * pool.ppc
    D, pt = w.head_dim, w.page_tokens
    n = npages * w.heads * pt * D * 2
    ko = g["k_off"] + layer * g["k_layer_bytes"]
    vo = g["v_off"] + layer * g["v_layer_bytes"]
    kp = pool.pool[ko:ko + n].view(torch.int16).view(npages, w.heads, D // 8, pt, 8).permute(0, 1, 3, 2, 4)
    vp = pool.pool[vo:vo + n].view(torch.int16).view(npages, w.heads, pt // 8, D, 8).permute(0, 1, 2, 4, 3)
    return (bf16_dev_bits_to_f32(kp.reshape(npages, w.heads, pt, D).contiguous()),
            bf16_dev_bits_to_f32(vp.reshape(npages, w.heads, pt, D).contiguous()))


def position_rows(pages: np.ndarray, table, p: int, ppc: int) -> np.ndarray:
    """[heads, N, d] of context position p from pages [page, head, token, d]."""
    return np.concatenate([pages[table[p * ppc + i]] for i in range(ppc)], axis=1)


# fp32 accumulation of `hidden` bf16 products of size ~1/sqrt(hidden) leaves
# an absolute error near 2^-24 * sqrt(hidden); where the exact value is that
# small (cancellation), one bf16 ulp of it is finer than the fp32 result, so
# elements are compared in ulps above this floor and absolutely below it.
ABS_FLOOR = 2.0 ** -14


def bf16_ulps(a, b):
    """bf16 ulps between got and ref, 0 where they differ by less than ABS_FLOOR."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    ia = (a.view(np.uint32) >> 16).astype(np.int64)
    ib = (b.view(np.uint32) >> 16).astype(np.int64)
    u = np.abs(ia - ib)
    return np.where(np.abs(a.astype(np.float64) - b.astype(np.float64)) < ABS_FLOOR, 0, u)


def worst_ulp(got, ref):
    u = bf16_ulps(got, ref)
    i = np.unravel_index(int(np.argmax(u)), u.shape)
    return "worst %d ulp at %s: got %r ref %r" % (int(u[i]), i, float(got[i]), float(ref[i]))
