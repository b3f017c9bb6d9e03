"""wf_kv_publish_noalloc against wf_kv_publish, through the C ABI.

Twin pools of one configuration receive the same inputs, one through each
entry point. The published pages (K, V, fp8 scales and chunk means) and Q must
be equal bit for bit, and so must the attention over them, on two calls in a
row: every live slot, then a smaller call (two slots, fresh values), which
reuses the static scratch the first call left behind.
"""
import sys

import numpy as np
import pytest
import torch

import wf_inputs as W

from _gpu_round import RoundRunner, stack_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import wavefront_causal_attention_amd as wf
    wf.load()
    yield


def _published_bytes(r):
    """K pages, V pages, fp8 scales and means of layer 0, and Q (+ scales)."""
    w, pool = r.w, r.pool
    g = pool.geometry
    npages = w.T * pool.ppc
    elems = npages * w.heads * w.page_tokens * w.head_dim
    fp8 = w.qk_dtype == "fp8"
    parts = [pool.pool[g["k_off"]:g["k_off"] + elems * (1 if fp8 else 2)],
             pool.pool[g["v_off"]:g["v_off"] + elems * 2]]
    if fp8:
        parts.append(pool.pool[g["kscale_off"]:g["kscale_off"] + npages * w.heads * w.page_tokens * 4])
        parts.append(pool.pool[g["kmean_off"]:g["kmean_off"] + w.T * w.heads * w.head_dim * 4])
    out = [p.cpu().numpy().copy() for p in parts]
    out.append(r.q.view(torch.uint8).cpu().numpy().copy())
    if r.qs is not None:
        out.append(r.qs.cpu().numpy().view(np.uint8).copy())
    return out


def _publish(r, live, slot_first, nslots, noalloc):
    w = r.w
    sel = live[slot_first:slot_first + nslots]
    if w.fused_qkv:
        fd = stack_dev([np.concatenate(x, axis=1) for x in sel], w.in_dtype)
        r.pool.publish(0, slot_first, nslots, fd[:, :w.hd], fd[:, w.hd:2 * w.hd], fd[:, 2 * w.hd:], 3 * w.hd,
                       q_out=r.q, q_scales=r.qs, noalloc=noalloc)
        keep = fd
    else:
        qd, kd, vd = (stack_dev([x[i] for x in sel], w.in_dtype) for i in range(3))
        r.pool.publish(0, slot_first, nslots, qd, kd, vd, w.hd, q_out=r.q, q_scales=r.qs, noalloc=noalloc)
        keep = (qd, kd, vd)
    torch.cuda.synchronize()
    return keep


@pytest.mark.parametrize("name", ["wan1.3b_s4_fp8", "ragged_fp8", "tiny_fp8", "ragged128"])
def test_noalloc_publish_equals_publish_on_two_calls(name):
    w = W.WORKLOADS[name]
    say("case", name, "wf_kv_publish_noalloc vs wf_kv_publish")
    ref, got = RoundRunner(w), RoundRunner(w)
    ref.seed_clean()
    got.seed_clean()
    live = W.draw_slots(w, ref.k, range(w.S + 1))
    # call 1: every live slot
    _publish(ref, live, 0, w.S + 1, noalloc=False)
    _publish(got, live, 0, w.S + 1, noalloc=True)
    for i, (a, b) in enumerate(zip(_published_bytes(ref), _published_bytes(got))):
        assert np.array_equal(a, b), ("call 1", i)
    oa, ob = ref.attention("fp32"), got.attention("fp32")
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    # call 2, smaller: two slots with fresh values
    live2 = [tuple(np.ascontiguousarray(a[::-1]) for a in x) for x in W.draw_slots(w, ref.k + 100, range(w.S + 1))]
    live2 = [tuple(W.round_to_bf16(a) if w.in_dtype == "bf16" else a for a in x) for x in live2]
    first, n = (1, 2) if w.S >= 2 else (0, 1)
    _publish(ref, live2, first, n, noalloc=False)
    _publish(got, live2, first, n, noalloc=True)
    for i, (a, b) in enumerate(zip(_published_bytes(ref), _published_bytes(got))):
        assert np.array_equal(a, b), ("call 2", i)
    oa, ob = ref.attention("fp32"), got.attention("fp32")
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    say(name, "two calls: pages, Q and attention bit-identical")
