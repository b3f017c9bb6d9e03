"""CPU check of the multi-process oracle runner used by the full-size GPU
parity tests: split into (slot, heads) units, it computes what one serial
oracle_round call does on the same seeded inputs."""
import numpy as np
import pytest

import wf_inputs as W
from oracle import RoundSchedule, oracle_round

from oracle.parallel import compare_every_output, oracle_units


def _serial(w, k, storage):
    sch = RoundSchedule(w.S, w.A, w.H, k)
    live = [W.draw(w, k, s) for s in range(w.S + 1)]
    clean = {c: W.stored_draw(w, c)[1:] for c in sch.chunk_ids()[:w.A + w.H]}
    return oracle_round(w, k, live, clean, storage=storage)


@pytest.mark.parametrize("name,storage", [("ragged128", "bf16"), ("ragged_fp8", "fp8"), ("tiny", "bf16")])
def test_pooled_oracle_equals_serial_oracle(name, storage):
    w = W.WORKLOADS[name]
    k = w.steady_round
    ref = _serial(w, k, storage)                       # [S+1, N, heads, d]
    units = [(s, (h,)) for s in range(w.S + 1) for h in range(w.heads)]
    seen = set()
    for s, hs, o in oracle_units(w, k, units, storage, workers=3):
        assert np.allclose(o, ref[s][:, list(hs), :], rtol=0, atol=1e-12)
        seen.add((s, hs))
    assert seen == set(units)
    # the comparison helper on the serial result itself, and on a planted error
    out = ref.astype(np.float32)
    mx, rel, worst, n = compare_every_output(out, w, k, storage, heads_per_unit=2, say=lambda *a: None)
    assert n == (w.S + 1) * ((w.heads + 1) // 2) and mx < 1e-5 and worst < 1e-6
    out[w.S, 5, w.heads - 1, 3] += 0.5
    mx, rel, worst, n = compare_every_output(out, w, k, storage, say=lambda *a: None)
    assert abs(mx - 0.5) < 1e-5 and worst > 1e-3


def test_pooled_oracle_rows_subset():
    w = W.WORKLOADS["ragged128"]
    k = w.steady_round
    rows = np.array([0, 7, 255, 256, w.N - 1])
    ref = _serial(w, k, "bf16")[:, rows]
    for s, hs, o in oracle_units(w, k, [(1, (0, 2)), (3, (1,))], "bf16", rows=rows, workers=2):
        assert np.allclose(o, ref[s][:, list(hs), :], rtol=0, atol=1e-12)
