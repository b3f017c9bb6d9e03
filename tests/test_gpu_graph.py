"""HIP-graph capture and replay of a whole round, through the C ABI.

A round's launches (publish or the fused projection, attention, the advance)
are captured once; the pool's device round counter drives the page-table
rotation and the live slots' RoPE time offsets, so replaying the same graph in
later rounds computes those rounds. Each replay (fresh inputs copied into the
captured input buffers first, the output reset eagerly in between) must equal
the same round run eagerly on a twin pool bit for bit, and meet the parity bar
against the oracle; after the replays the host state (wf_round_replayed) and
the device agree, so eager rounds continue on the same pool.
"""
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W
from oracle import oracle_round, project_qkv, project_qkv_w8a8, quantize_rows_fp8, split_qkv

from _gpu_round import RoundRunner, err_stats, gpu_rows, to_dev

pytestmark = pytest.mark.gpu

BAR = {"bf16": (1e-2, 5e-3), "fp8": (3e-2, 1.5e-2)}
REPLAYS = 4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import wavefront_causal_attention_amd as wf
    wf.load()
    yield


class _Path:
    """One way of publishing a round: from projection outputs, or through the
    fused projection (bf16 or W8A8), with static device input buffers."""

    def __init__(self, w, kind):
        import wavefront_causal_attention_amd as wf
        self.w, self.kind = w, kind
        S1, N, hd = w.S + 1, w.N, w.hd
        dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
        if kind == "publish":
            self.buf = torch.empty((S1 * N, 3 * hd), dtype=dt, device="cuda")
        else:
            self.buf = torch.zeros((S1 * N, hd), dtype=torch.bfloat16, device="cuda")
            self.wt, self.b = W.projection_weights(w)
            self.wd, self.bd = to_dev(self.wt, "bf16"), to_dev(self.b, "bf16")
            if kind == "w8a8":
                self.w8, self.sw = wf.quantize_rows_fp8(self.wd)
                self.x8, self.sx = wf.quantize_rows_fp8(self.buf)
                self.wc, self.ws = quantize_rows_fp8(self.wt)

    def set_round(self, k):
        """Copy round k's inputs into the static buffers; returns the fp64
        (q, k, v) of every live slot as the oracle sees them."""
        w = self.w
        if self.kind == "publish":
            live = [W.draw(w, k, s) for s in range(w.S + 1)]
            host = np.concatenate([np.concatenate(x, axis=1) for x in live], axis=0)
        else:
            xs = [W.draw_hidden(w, k, s) for s in range(w.S + 1)]
            host = np.concatenate(xs, axis=0)
            if self.kind == "project":
                live = [tuple(split_qkv(project_qkv(x, self.wt, self.b), w.hd)) for x in xs]
            else:
                q8 = [quantize_rows_fp8(x) for x in xs]
                live = [tuple(split_qkv(project_qkv_w8a8(c, s, self.wc, self.ws, self.b), w.hd)) for c, s in q8]
        self.buf.copy_(torch.from_numpy(np.ascontiguousarray(host, dtype=np.float32)).to(self.buf.dtype))
        return live

    def publish(self, r: RoundRunner):
        import wavefront_causal_attention_amd as wf
        w, hd = self.w, self.w.hd
        if self.kind == "publish":
            b = self.buf
            r.pool.publish(0, 0, w.S + 1, b[:, :hd], b[:, hd:2 * hd], b[:, 2 * hd:], 3 * hd, q_out=r.q,
                           q_scales=r.qs)
        elif self.kind == "project":
            r.pool.project_publish(0, 0, w.S + 1, self.buf, hd, hd, self.wd, self.bd, q_out=r.q)
        else:
            wf.quantize_rows_fp8(self.buf, self.x8, self.sx)
            r.pool.project_publish_w8a8(0, 0, w.S + 1, self.x8, self.x8.stride(0), self.sx, hd, self.w8, self.sw,
                                        self.bd, q_out=r.q)


@pytest.mark.parametrize("name,kind", [("ragged128", "publish"), ("edge_s1_h0", "publish"),
                                       ("ragged_fp8", "publish"), ("ragged128", "project"),
                                       ("ragged128", "w8a8")])
def test_graph_replays_equal_eager_rounds(name, kind):
    w = W.WORKLOADS[name]
    say("case", name, kind, "graph capture +", REPLAYS, "replays")
    eager, graph = RoundRunner(w), RoundRunner(w)
    eager.seed_clean()
    graph.seed_clean()
    pe, pg = _Path(w, kind), _Path(w, kind)
    out_e, out_g = eager.pool.out_buffer("fp32"), graph.pool.out_buffer("fp32")

    pg.set_round(graph.k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pg.publish(graph)
        graph.pool.attention(0, 0, w.S + 1, graph.q, out_g, q_scales=graph.qs)
        graph.pool.advance()
    torch.cuda.synchronize()
    k0 = graph.k
    assert graph.pool.round_index() == k0              # the captured advance did not move the host

    mx_bar, rel_bar = BAR[w.qk_dtype]
    for r in range(REPLAYS):
        k = k0 + r
        live = pg.set_round(k)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        graph.pool.round_replayed()
        torch.cuda.synchronize()
        # the same round, eagerly, on the twin pool
        pe.set_round(k)
        pe.publish(eager)
        eager.live = live
        out_e.fill_(float("nan"))
        eager.pool.attention(0, 0, w.S + 1, eager.q, out_e, q_scales=eager.qs)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay of round %d differs from the eager round" % k
        ref = oracle_round(w, k, live, eager.clean_for_round(), storage=w.qk_dtype)
        mx, rel = err_stats(gpu_rows(out_g, w, np.arange(w.N)), ref)
        say(name, kind, "replayed round", k, "max_abs %.3e rel_l2 %.3e" % (mx, rel))
        assert mx <= mx_bar and rel <= rel_bar
        eager.advance()
        assert graph.pool.round_index() == eager.pool.round_index() == k + 1
        assert graph.pool.page_table_host() == eager.pool.page_table_host()
        assert torch.equal(graph.pool.table, eager.pool.table)    # the device tables agree too

    # eager rounds continue on the replayed pool
    k = k0 + REPLAYS
    live = pg.set_round(k)
    pg.publish(graph)
    out_g.fill_(float("nan"))
    graph.pool.attention(0, 0, w.S + 1, graph.q, out_g, q_scales=graph.qs)
    torch.cuda.synchronize()
    ref = oracle_round(w, k, live, eager.clean_for_round(), storage=w.qk_dtype)
    mx, rel = err_stats(gpu_rows(out_g, w, np.arange(w.N)), ref)
    say(name, kind, "eager round", k, "after the replays: max_abs %.3e rel_l2 %.3e" % (mx, rel))
    assert mx <= mx_bar and rel <= rel_bar


def test_graph_replays_two_layers():
    """One captured round of a two-layer pool (both layers' publish and
    attention, one advance): each replay equals the same rounds run eagerly on
    a twin pool, in both layers, and leaves the same shared page table."""
    import wavefront_causal_attention_amd as wf
    from _gpu_round import config_of, stack_dev
    w = W.WORKLOADS["ragged128"]
    say("case ragged128, two layers, graph capture +", REPLAYS, "replays")
    pools = [wf.Pool(config_of(w, first_round=w.steady_round, num_layers=2)) for _ in range(2)]
    ids = pools[0].chunk_ids()
    for pool in pools:                                  # seed anchor and history of both layers
        for layer in range(2):
            cl = [W.stored_draw(w, ids[w.T - 1 - slot] + 1000 * layer) for slot in range(w.S + 1, w.T)]
            pool.publish(layer, w.S + 1, w.T - w.S - 1, None, stack_dev([x[1] for x in cl], w.in_dtype),
                         stack_dev([x[2] for x in cl], w.in_dtype), w.hd)
    bufs = [[torch.empty((w.S + 1) * w.N, 3 * w.hd, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
            for _ in range(2)]
    qs = [pool.q_buffer() for pool in pools]
    outs = [[pool.out_buffer("fp32") for _ in range(2)] for pool in pools]

    def set_round(i, k):
        for layer in range(2):
            live = [W.draw(w, k + 1000 * layer, s) for s in range(w.S + 1)]
            host = np.concatenate([np.concatenate(x, axis=1) for x in live], axis=0)
            bufs[i][layer].copy_(torch.from_numpy(host).to(torch.bfloat16))

    def round_launches(i):
        hd = w.hd
        for layer in range(2):
            b = bufs[i][layer]
            pools[i].publish(layer, 0, w.S + 1, b[:, :hd], b[:, hd:2 * hd], b[:, 2 * hd:], 3 * hd, q_out=qs[i])
            pools[i].attention(layer, 0, w.S + 1, qs[i], outs[i][layer])
        pools[i].advance()

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_launches(1)
    k0 = w.steady_round
    for r in range(REPLAYS):
        set_round(0, k0 + r)
        set_round(1, k0 + r)
        for o in outs[1]:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        pools[1].round_replayed()
        round_launches(0)
        torch.cuda.synchronize()
        for layer in range(2):
            assert not torch.isnan(outs[1][layer]).any()
            assert torch.equal(outs[1][layer], outs[0][layer]), (r, layer)
        assert pools[1].round_index() == pools[0].round_index() == k0 + r + 1
        assert torch.equal(pools[1].table, pools[0].table)
        for layer in range(2):
            assert pools[1].ready_mask(layer) == pools[0].ready_mask(layer)
    say("two layers: %d replays equal to the eager rounds" % REPLAYS)


def test_capture_of_a_fill_round_is_refused():
    """Only steady rounds can be replayed, so an advance captured in a round
    that fills the pipeline is refused on the host before anything is
    enqueued, and the pool's state is left as it was."""
    import wavefront_causal_attention_amd as wf
    from _gpu_round import config_of, stack_dev
    w = W.WORKLOADS["tiny"]
    say("case tiny, capture in fill round 0")
    pool = wf.Pool(config_of(w, first_round=0))
    q = pool.q_buffer()
    live = W.draw(w, 0, 0)
    qd, kd, vd = (stack_dev([x], w.in_dtype) for x in live)
    table0 = pool.table.clone()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(wf.WfError) as e:
        with torch.cuda.graph(g):
            pool.publish(0, 0, 1, qd, kd, vd, w.hd, q_out=q)   # round 0: only slot 0 holds a chunk
            pool.advance()
    assert e.value.status == wf.WF_E_INVALID_ARG
    assert "steady" in str(e.value)
    torch.cuda.synchronize()
    assert pool.round_index() == 0
    assert torch.equal(pool.table, table0)
    # the pool still runs eagerly
    pool.publish(0, 0, 1, qd, kd, vd, w.hd, q_out=q)
    pool.advance()
    torch.cuda.synchronize()
    assert pool.round_index() == 1


def test_replay_bookkeeping_without_a_capture_is_refused():
    """A device pool from which no advance was captured has no replay to
    follow: the host state must not move away from the device's."""
    import wavefront_causal_attention_amd as wf
    from _gpu_round import config_of
    w = W.WORKLOADS["tiny"]
    pool = wf.Pool(config_of(w))
    k = pool.round_index()
    with pytest.raises(wf.WfError) as e:
        pool.round_replayed()
    assert e.value.status == wf.WF_E_INVALID_ARG and "captured" in str(e.value)
    assert pool.round_index() == k
