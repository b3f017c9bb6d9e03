"""Wavefront schedule model: which chunk sits at which context position.

Wave Forcing, hyper.ai summary, section "Method": the wavefront updates chunk i
at stage s in round k = i + s; attention is chunk-causal with the mask
M_WF(s, j) = 1[j >= s] over the query's own slot and all cleaner ones.
thelatestinai.com listing, Table 3: s indexes denoising stages 0 <= s < S and
the store occupies stage s = S. e-cogni.com.br article, "Como funciona": each
layer's context is anchor (initial chunk) | bounded clean history | live store |
denoising K/V.

Context positions are numbered cleanest first:
    [anchor_0 .. anchor_{A-1} | hist_0 (oldest) .. hist_{H-1} | store | slot S-1 .. slot 0]
"""
from __future__ import annotations

from collections import deque

import numpy as np


def live_mask(S: int, kind: str = "wavefront") -> np.ndarray:
    """Visibility among the S+1 live slots (store included), indexed [query s][key j].

    "wavefront": M_WF(s, j) = 1[j >= s] (hyper.ai summary, "Method").
    "all": every live slot sees every live slot, the bidirectional live K/V of
    Rolling Forcing that the pages contrast Wave Forcing with (thelatestinai.com
    listing, Table 9; e-cogni.com.br, "Como funciona").
    """
    if kind not in ("wavefront", "all"):
        raise ValueError("unknown live mask %r" % kind)
    M = np.zeros((S + 1, S + 1), dtype=np.int64)
    for s in range(S + 1):
        for j in range(S + 1):
            M[s, j] = 1 if (kind == "all" or j >= s) else 0
    return M


def slot_position(s: int, S: int, A: int, H: int) -> int:
    """Context position of live slot s (s = S is the store)."""
    if not 0 <= s <= S:
        raise ValueError("slot out of range")
    if s == S:
        return A + H
    return A + H + 1 + (S - 1 - s)


def legal_positions(s: int, S: int, A: int, H: int, kind: str = "wavefront") -> list:
    """Context positions query slot s may read, in context order.

    Anchor and clean history are cleaner than every live slot and are read by
    all of them; among live slots the live mask (M_WF by default) decides.
    """
    M = live_mask(S, kind)
    out = list(range(A)) + list(range(A, A + H))
    live = [j for j in range(S, -1, -1) if M[s, j]]          # store first, then S-1 .. 0
    out += [slot_position(j, S, A, H) for j in live]
    return sorted(out)


class RoundSchedule:
    """Chunk ids of every context position in round k.

    By default only steady-state rounds are modelled (the schedule raises for k
    below the first full round). With fill=True the schedule also covers the
    rounds that fill the pipeline, and with total_chunks = C the rounds that
    drain it after the last chunk (rounds run from 0 to C-1+S). In those rounds
    some positions hold no chunk (present() is False) and are left out of every
    legal context. The pages mention the fill and its latency (thelatestinai.com
    listing, Figure 1 caption) without detail; the reading here: chunk i enters
    slot 0 in round i and moves one stage per round (k = i + s), is stored in
    round i + S, and from then on is clean: anchor chunk a (a < A) sits at
    anchor position a, every later chunk enters the history ring, which keeps
    the H most recently stored non-anchor chunks.
    """

    def __init__(self, S: int, A: int, H: int, k: int, fill: bool = False, total_chunks=None):
        if k < 0 or (not fill and k < S + H + A):
            raise ValueError("round %d is a fill round; first full round is %d" % (k, S + H + A))
        if total_chunks is not None and k > total_chunks - 1 + S:
            raise ValueError("round %d is past the last round %d" % (k, total_chunks - 1 + S))
        self.S, self.A, self.H, self.k = S, A, H, k
        self.C = total_chunks
        self.T = A + H + S + 1

    def chunk_at(self, p: int) -> int:
        S, A, H, k = self.S, self.A, self.H, self.k
        if p < A:
            return p                                   # anchor: the initial chunk(s)
        if p < A + H:
            return k - S - H + (p - A)                 # history, oldest first
        if p == A + H:
            return k - S                               # store = stage S
        s = S - 1 - (p - A - H - 1)
        return k - s                                   # live slot s holds chunk i = k - s

    def present(self, p: int) -> bool:
        """Whether position p holds a chunk in this round."""
        c = self.chunk_at(p)
        last = self.C - 1 if self.C is not None else None
        if p < self.A:
            return self.k >= c + self.S + 1 and (last is None or c <= last)   # stored already
        if p < self.A + self.H:
            return c >= self.A and (last is None or c <= last)               # non-anchor, stored
        return c >= 0 and (last is None or c <= last)                       # live: store and slots

    def chunk_ids(self) -> list:
        return [self.chunk_at(p) for p in range(self.T)]

    def present_chunk_ids(self) -> list:
        """Chunk id per position, None where the position is empty."""
        return [self.chunk_at(p) if self.present(p) else None for p in range(self.T)]

    def slot_present(self, s: int) -> bool:
        return self.present(slot_position(s, self.S, self.A, self.H))

    def legal_present(self, s: int, kind: str = "wavefront") -> list:
        """Positions query slot s reads in this round: its legal ones that hold a chunk."""
        return [p for p in legal_positions(s, self.S, self.A, self.H, kind) if self.present(p)]

    def slot_chunk(self, s: int) -> int:
        return self.chunk_at(slot_position(s, self.S, self.A, self.H))


class GroupRing:
    """Physical-page-group bookkeeping written as a plain rotation.

    The H+S+1 non-anchor positions hold one page group each. When a round ends
    every chunk moves one position cleaner without being copied: the store's
    group becomes the newest history, and the group that held the oldest
    history is handed to slot 0 (the noisiest), which is re-published next
    round. Anchor groups never move.
    """

    def __init__(self, S: int, A: int, H: int):
        self.A = A
        self.ring = deque(range(A, A + H + S + 1))

    def advance(self):
        self.ring.rotate(-1)

    def groups(self) -> list:
        return list(range(self.A)) + list(self.ring)
