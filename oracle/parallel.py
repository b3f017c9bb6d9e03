"""The oracle of one round spread over the host's cores.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the full-size parity
tests and the benchmark's CPU-baseline leg use it to evaluate every output of
a full-size round in reasonable time.

Work is split into (slot, heads) units, since attention is independent per
query slot and per head (hyper.ai summary, section "Method": the mask acts
between slots, every head alike). Each unit runs in a spawned worker process
that regenerates the round's seeded inputs itself (wf_inputs: live slots drawn
with draw(), anchor and history with stored_draw()), so no GPU state or GPU
result ever reaches the oracle, and calls oracle_round on that unit's slot and
heads with single-threaded BLAS. The oracle's arithmetic is unchanged: this
module only decides which slot and heads each call evaluates.

The workers import only numpy, threadpoolctl, wf_inputs and this package.
"""
from __future__ import annotations

import dataclasses
import functools
import multiprocessing as mp
import os

import numpy as np


def host_workers(limit: int = 16) -> int:
    """Worker processes: the CPUs this process may run on, at most `limit`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


@functools.lru_cache(maxsize=1)
def _round_inputs(w, k):
    import wf_inputs as W
    from .schedule import RoundSchedule
    sch = RoundSchedule(w.S, w.A, w.H, k)
    live = [W.draw(w, k, s) for s in range(w.S + 1)]
    clean = {c: W.stored_draw(w, c)[1:] for c in sch.chunk_ids()[:w.A + w.H]}
    return live, clean


def _unit(args):
    w, k, slot, heads, rows, storage = args
    from .round import oracle_round
    live, clean = _round_inputs(w, k)
    d = w.head_dim

    def take(x):
        return np.ascontiguousarray(np.concatenate([x[:, h * d:(h + 1) * d] for h in heads], axis=1))

    wh = dataclasses.replace(w, heads=len(heads))
    live_h = [tuple(take(a) for a in x) for x in live]
    clean_h = {c: tuple(take(a) for a in kv) for c, kv in clean.items()}
    o = oracle_round(wh, k, live_h, clean_h, storage=storage, rows=rows, slots=[slot], mask=w.live_mask)
    return slot, tuple(heads), o[0]


def oracle_units(w, k, units, storage, rows=None, workers=None):
    """Yield (slot, heads, O[rows, len(heads), d]) for every (slot, heads)
    unit of round k of workload w, as the workers finish them. A worker that
    dies raises BrokenProcessPool here instead of being replaced."""
    from concurrent.futures import ProcessPoolExecutor, as_completed
    tasks = [(w, k, s, tuple(h), rows, storage) for s, h in units]
    with ProcessPoolExecutor(max_workers=workers or host_workers(), mp_context=mp.get_context("spawn"),
                             initializer=_init_worker) as ex:
        futs = [ex.submit(_unit, t) for t in tasks]
        for f in as_completed(futs):
            yield f.result()


def compare_every_output(out: np.ndarray, w, k, storage, rows=None, heads_per_unit=1, say=print):
    """Compare a GPU round output out[S+1, N, heads, d] (fp32 output mode) with
    the oracle on every slot and head (rows: all, or the given rows).

    Returns (max_abs, rel_l2 over the whole round, worst per-unit rel_l2,
    units); the location of the largest difference, (slot, head, row,
    channel, got, oracle), is printed with the last progress line."""
    units = [(s, tuple(range(h0, min(h0 + heads_per_unit, w.heads))))
             for s in range(w.S + 1) for h0 in range(0, w.heads, heads_per_unit)]
    rsel = slice(None) if rows is None else np.asarray(rows)
    rids = np.arange(w.N) if rows is None else np.asarray(rows)
    mx, se, sr, worst, where = 0.0, 0.0, 0.0, 0.0, None
    for i, (s, hs, ref) in enumerate(oracle_units(w, k, units, storage, rows=rows)):
        g = out[s][rsel][:, list(hs), :].astype(np.float64)
        assert g.shape == ref.shape, (g.shape, ref.shape)
        diff = g - ref
        e, r = float(np.sum(diff * diff)), float(np.sum(ref * ref))
        j = np.unravel_index(int(np.argmax(np.abs(diff))), diff.shape)
        if abs(diff[j]) > mx:
            mx = float(abs(diff[j]))
            where = (s, hs[j[1]], int(rids[j[0]]), int(j[2]), float(g[j]), float(ref[j]))
        se += e
        sr += r
        worst = max(worst, (e / r) ** 0.5)
        if (i + 1) % 10 == 0 or i + 1 == len(units):
            say("  oracle units %d/%d: max_abs %.3e worst unit rel_l2 %.3e" % (i + 1, len(units), mx, worst))
    say("  largest difference at slot %d head %d row %d channel %d: got %.6g oracle %.6g" % where)
    return mx, (se / sr) ** 0.5, worst, len(units)
