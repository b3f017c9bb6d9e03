"""Benchmark: one wavefront round per step on one MI355X.

A step is the whole hot path over one round of synthetic Wan2.1-shaped input:
fused 3D-RoPE + K/V publish of all S+1 slots, wavefront attention of all S+1
query slots over the paged context, and the round advance (page-table
rotation). Inputs are resident in HBM before timing starts.

Prints one JSON line. `value` is mask-aware attention TFLOP/s over the whole
step (publish + attention + advance); rounds/s, per-kernel times, the
attention roofline and an fp64-oracle CPU baseline ride along. With
--layers L a step is one model round: every layer publishes and attends over
its own pages (one pool, one page table), then one advance.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "wavefront-round attention TFLOP/s + rounds/sec, 1 MI355X, Wan2.1-1.3B S=4 shape"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E
# the attention kernel and the host code that orders its work (the order
# decides which K/V reads hit L2, so it changes the traffic)
ATTN_SOURCES = [os.path.join(ROOT, "wavefront_causal_attention_amd", "csrc", f)
                for f in ("wf_attention.hip", "wf_internal.h", "wf_api.cpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_file(workload: str, fp8: bool) -> str:
    """The committed counter summary of this workload's attention kernel."""
    return os.path.join(ROOT, "profiles", f"attn_{'fp8' if fp8 else 'bf16'}_{workload}_traffic.txt")


def measured_traffic(workload: str, fp8: bool):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None if there is none or the kernel source changed
    since the counters were taken."""
    path = traffic_file(workload, fp8)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan1.3b_s4")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step in a HIP graph and time its replays (the pool's device round "
                         "counter advances each replay)")
    ap.add_argument("--live-mask", default="wavefront", choices=["wavefront", "all"],
                    help="all: every live slot reads every live slot (no tile skipped), for "
                         "measuring what the wavefront mask saves")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers sharing one pool and page table; a step is then one model round "
                         "(publish + attention of every layer, one advance)")
    ap.add_argument("--project", nargs="?", const="bf16", default=None, choices=["bf16", "w8a8"],
                    help="publish through the fused QKV projection (hidden states -> RoPE'd Q/K/V pages) "
                         "instead of from a projection output; also times hipBLASLt addmm + publish. "
                         "w8a8: the hidden states are quantised to e4m3 per token each step and the "
                         "projection runs on e4m3 operands (weight quantised once, per output channel)")
    ap.add_argument("--repeats", type=int, default=3,
                    help="blocks of --steps steps timed in all (the first is the headline); median and "
                         "min-max over the blocks are reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows per (slot, head) in the CPU baseline; 0: the whole round")
    ap.add_argument("--cpu-workers", type=int, default=16, help="oracle worker processes (at most)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the wavefront round is built and timed on a single "
              "MI355X; multi-GPU runs are not supported (requested %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import wf_inputs as W
    import wavefront_causal_attention_amd as wf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wf.load()
    w = W.WORKLOADS[args.workload]
    if args.live_mask != w.live_mask:
        import dataclasses
        w = dataclasses.replace(w, live_mask=args.live_mask)
    dev = torch.device("cuda:0")
    k0 = w.steady_round
    cfg = wf.make_config(S=w.S, anchor_chunks=w.A, history_chunks=w.H, heads=w.heads,
                         head_dim=w.head_dim, chunk_frames=w.chunk_frames, frame_h=w.frame_h,
                         frame_w=w.frame_w, page_tokens=w.page_tokens, in_dtype=w.in_dtype,
                         qk_dtype=w.qk_dtype, rope_split=w.rope_split, rope_theta=w.rope_theta,
                         first_round=k0, live_mask=w.live_mask, num_layers=args.layers)
    pool = wf.Pool(cfg, device=dev)
    L = args.layers
    tdt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32

    def to_dev(arrs):
        return torch.from_numpy(np.concatenate(arrs, 0)).to(tdt).to(dev)

    # seed anchor + history with the K/V their store rounds published
    ids = pool.chunk_ids()
    cl = [W.stored_draw(w, ids[w.T - 1 - slot]) for slot in range(w.S + 1, w.T)]
    kc, vc = to_dev([x[1] for x in cl]), to_dev([x[2] for x in cl])
    for layer in range(L):
        pool.publish(layer, w.S + 1, w.T - w.S - 1, None, kc, vc, w.hd)
    del cl
    # live slots: one seeded round of projected Q/K/V, resident for every step
    live = W.draw_slots(w, k0, range(w.S + 1))
    if w.fused_qkv:
        fused = to_dev([np.concatenate(x, 1) for x in live])
        qd, kd, vd, stride = fused[:, :w.hd], fused[:, w.hd:2 * w.hd], fused[:, 2 * w.hd:], 3 * w.hd
    else:
        qd, kd, vd = to_dev([x[0] for x in live]), to_dev([x[1] for x in live]), to_dev([x[2] for x in live])
        stride = w.hd
    del live
    q = pool.q_buffer()
    qs = pool.q_scale_buffer()
    out = pool.out_buffer(args.out_dtype)
    if args.project:
        assert w.qk_dtype == "bf16", "the fused projection publishes bf16 pages"
        xh = to_dev([W.draw_hidden(w, k0, s) for s in range(w.S + 1)]).to(torch.bfloat16)
        wt_np, b_np = W.projection_weights(w)
        wproj = torch.from_numpy(wt_np).to(torch.bfloat16).to(dev)            # [3hd, hidden]
        bproj = torch.from_numpy(b_np).to(torch.bfloat16).to(dev)
        if args.project == "w8a8":
            w8, sw8 = wf.quantize_rows_fp8(wproj)                              # once, like a checkpoint
            x8, sx8 = wf.quantize_rows_fp8(xh)                                 # buffers reused every step
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    # every layer publishes the same resident projection output into its own
    # pages and attends over them: the work per layer is the real one
    def step(ev=None, stream=stream):
        for layer in range(L):
            if ev is not None and layer == 0:
                ev[0].record(stream)
            if args.project == "w8a8":
                wf.quantize_rows_fp8(xh, x8, sx8, stream=stream)
                pool.project_publish_w8a8(layer, 0, w.S + 1, x8, x8.stride(0), sx8, w.hd, w8, sw8, bproj,
                                          q_out=q, stream=stream)
            elif args.project:
                pool.project_publish(layer, 0, w.S + 1, xh, w.hd, w.hd, wproj, bproj, q_out=q, stream=stream)
            else:
                pool.publish(layer, 0, w.S + 1, qd, kd, vd, stride, q_out=q, q_scales=qs, stream=stream)
            if ev is not None and layer == 0:
                ev[1].record(stream)
            pool.attention(layer, 0, w.S + 1, q, out, q_scales=qs, stream=stream)
            if ev is not None and layer == 0:
                ev[2].record(stream)
        if ev is not None:
            ev[3].record(stream)
        pool.advance(stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # further blocks of K steps, for the median and spread over repeats (the
    # first block above is the headline)
    blocks = [{"ms_per_step": wall * 1e3 / K, "attention_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
               "publish_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))}]
    for _ in range(max(0, args.repeats - 1)):
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for i in range(K):
            step(rev[i])
        torch.cuda.synchronize()
        blocks.append({"ms_per_step": (time.perf_counter() - tb) * 1e3 / K,
                       "attention_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in rev])),
                       "publish_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in rev]))})

    # one GPU's share of the round: the noisiest slot alone (it reads the
    # whole context, the critical consumer of the round), K launches
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    pool.publish(0, 0, w.S + 1, qd, kd, vd, stride, q_out=q, q_scales=qs, stream=stream)   # this round's slots
    torch.cuda.synchronize()
    cev[0].record(stream)
    for i in range(K):
        pool.attention(0, 0, 1, q, out, q_scales=qs, stream=stream)
        cev[i + 1].record(stream)
    torch.cuda.synchronize()
    slot0_ms = [cev[i].elapsed_time(cev[i + 1]) for i in range(K)]

    # the matrix-core rate this GPU sustains under MFMA load at its current
    # clock (wf_mfma_calibrate: the attention step's MFMA mix, operands in
    # registers, one 8-wave workgroup per CU), timed right after the attention
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    csteps = 4096
    cal_out = torch.empty(ncu * 512, dtype=torch.float32, device=dev)
    wf.wf_mfma_calibrate(ncu, csteps, cal_out, stream=stream)
    cal_ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    cal_ev[0].record(stream)
    for i in range(5):
        wf.wf_mfma_calibrate(ncu, csteps, cal_out, stream=stream)
        cal_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    cal_ms = [cal_ev[i].elapsed_time(cal_ev[i + 1]) for i in range(5)]
    cal_flops = float(ncu) * 8 * csteps * 32 * 32768

    graph = None
    if args.graph:
        # the same step captured once and replayed; each replay is one more round
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(stream=torch.cuda.current_stream())
        for _ in range(args.warmup):
            g.replay()
            pool.round_replayed()
        torch.cuda.synchronize()
        # alternate blocks of K replays and K eager steps, so that clock drift
        # over the run does not favour either
        blocks = {"graph": [], "eager": []}
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for b in range(6):
            mode = "graph" if b % 2 == 0 else "eager"
            ge[0].record(stream)
            for _ in range(K):
                if mode == "graph":
                    g.replay()
                    pool.round_replayed()
                else:
                    step()
            ge[1].record(stream)
            torch.cuda.synchronize()
            blocks[mode].append(ge[0].elapsed_time(ge[1]) / K)
        graph = {"replay_stream_ms_per_step": round(float(np.median(blocks["graph"])), 4),
                 "eager_stream_ms_per_step": round(float(np.median(blocks["eager"])), 4),
                 "blocks": "3 x %d replays alternated with 3 x %d eager steps, medians" % (K, K)}

    pub_ms = [e[0].elapsed_time(e[1]) for e in evs]          # layer 0's kernels
    att_ms = [e[1].elapsed_time(e[2]) for e in evs]
    adv_ms = [e[3].elapsed_time(e[4]) for e in evs]
    gpu_ms = [e[0].elapsed_time(e[4]) for e in evs]           # whole step on the stream
    ms_step = wall * 1e3 / K
    F = w.attention_flops() * L
    att_avg = float(np.mean(att_ms))
    pub_avg = float(np.mean(pub_ms))
    n_el = (w.S + 1) * w.N * w.hd
    in_bytes = 3 * n_el * (2 if w.in_dtype == "bf16" else 4)
    qk_bytes = 1 if w.qk_dtype == "fp8" else 2
    pub_bytes = in_bytes + 2 * n_el * qk_bytes + 2 * n_el            # read QKV; write Q, K, V
    attn_tflops = w.attention_flops() / (att_avg * 1e-3) / 1e12
    # the counters were taken with the workload's own mask and bf16 output
    same_launch = args.live_mask == W.WORKLOADS[args.workload].live_mask and args.out_dtype == "bf16"
    traffic = measured_traffic(args.workload, w.qk_dtype == "fp8") if same_launch else None

    proj = None
    if args.project:
        # the same projection unfused: hipBLASLt addmm to a [tokens, 3hd] bf16
        # output, then the publish kernel reads it back; and each part alone
        wT = wproj.t().contiguous()                                   # [hidden, 3hd]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        parts = {"addmm": [], "publish": [], "bf16_fused": [], "quantize": [], "w8a8": []}
        for i in range(K + 2):
            ev[0].record(stream)
            y = torch.addmm(bproj, xh, wT)
            ev[1].record(stream)
            pool.publish(0, 0, w.S + 1, y[:, :w.hd], y[:, w.hd:2 * w.hd], y[:, 2 * w.hd:], 3 * w.hd,
                         q_out=q, stream=stream)
            ev[2].record(stream)
            pool.project_publish(0, 0, w.S + 1, xh, w.hd, w.hd, wproj, bproj, q_out=q, stream=stream)
            ev[3].record(stream)
            if args.project == "w8a8":
                wf.quantize_rows_fp8(xh, x8, sx8, stream=stream)
                ev[4].record(stream)
                pool.project_publish_w8a8(0, 0, w.S + 1, x8, x8.stride(0), sx8, w.hd, w8, sw8, bproj,
                                          q_out=q, stream=stream)
                ev[5].record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                parts["addmm"].append(ev[0].elapsed_time(ev[1]))
                parts["publish"].append(ev[1].elapsed_time(ev[2]))
                parts["bf16_fused"].append(ev[2].elapsed_time(ev[3]))
                if args.project == "w8a8":
                    parts["quantize"].append(ev[3].elapsed_time(ev[4]))
                    parts["w8a8"].append(ev[4].elapsed_time(ev[5]))
        avg = {k: float(np.mean(v)) for k, v in parts.items() if v}
        pf = 2.0 * (w.S + 1) * w.N * 3 * w.hd * w.hd
        fused_ms = float(np.mean(pub_ms))
        if args.project == "w8a8":
            tf = pf / (avg["w8a8"] * 1e-3) / 1e12
            qbytes = (w.S + 1) * w.N * w.hd * 3 + (w.S + 1) * w.N * 4     # read bf16, write codes + scales
            proj = {"mode": "w8a8",
                    "step_ms": round(fused_ms, 4),
                    "quantize_ms": round(avg["quantize"], 4),
                    "quantize_gbps": round(qbytes / (avg["quantize"] * 1e-3) / 1e9, 1),
                    "w8a8_projection_ms": round(avg["w8a8"], 4),
                    "w8a8_tflops": round(tf, 1),
                    "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
                    "flops": pf,
                    "bf16_fused_ms": round(avg["bf16_fused"], 4),
                    "unfused_addmm_ms": round(avg["addmm"], 4),
                    "unfused_publish_ms": round(avg["publish"], 4),
                    "unfused_ms": round(avg["addmm"] + avg["publish"], 4)}
        else:
            proj = {"fused_ms": round(fused_ms, 4),
                    "fused_tflops": round(pf / (fused_ms * 1e-3) / 1e12, 1),
                    "roofline": {"bound": "mfma", "achieved": round(pf / (fused_ms * 1e-3) / 1e12, 1),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(pf / (fused_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
                    "flops": pf,
                    "unfused_addmm_ms": round(avg["addmm"], 4),
                    "unfused_publish_ms": round(avg["publish"], 4),
                    "unfused_ms": round(avg["addmm"] + avg["publish"], 4)}

    # A device-to-device memcpy (torch copy_, the runtime's copy kernel) moving
    # as many bytes as the publish (half read, half written), timed in the same
    # session beside the publish's own rate. Not a ceiling: a streaming copy
    # kernel with non-temporal loads moves the same bytes faster.
    ncopy = pub_bytes // 2
    csrc = torch.empty(ncopy, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    torch.cuda.synchronize()
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        for _ in range(3):
            cdst.copy_(csrc)
        kev[0].record(stream)
        for _ in range(20):
            cdst.copy_(csrc)
        kev[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * ncopy / (kev[0].elapsed_time(kev[1]) / 20 * 1e-3) / 1e9
    # the library's streaming copy of the same bytes (wf_stream_copy_calibrate:
    # non-temporal 16-byte loads, nothing else): the HBM rate attainable for
    # this read/write mix, the publish kernels' same-session ceiling
    nstream = ncopy // 16 * 16
    for _ in range(3):
        wf.wf_stream_copy_calibrate(csrc, cdst, nstream, stream=stream)
    kev[0].record(stream)
    for _ in range(20):
        wf.wf_stream_copy_calibrate(csrc, cdst, nstream, stream=stream)
    kev[1].record(stream)
    torch.cuda.synchronize()
    stream_gbps = 2 * nstream / (kev[0].elapsed_time(kev[1]) / 20 * 1e-3) / 1e9
    del csrc, cdst

    if args.calibrate_copy_mib > 0:
        nb = args.calibrate_copy_mib * (1 << 20)
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    # bf16: the dense bf16 MFMA peak. fp8: half the flops (QK^T) run on fp8
    # MFMAs and half (PV) on bf16, so the bound is F / (F/2 / 5000 + F/2 / 2500)
    attn_peak = (PEAK_BF16_TFLOPS if w.qk_dtype == "bf16"
                 else 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS))
    res = {
        "metric": METRIC,
        "value": round(F * K / wall / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.qk_dtype == "bf16" else "fp8-qk/bf16-pv",
        "data": "synthetic: seeded N(0,1) Q/K/V, bf16, steady-state round",
        "config": {"workload": w.name, "S": w.S, "anchor_chunks": w.A, "history_chunks": w.H,
                   "chunk_tokens": w.N, "chunk_shape": [w.chunk_frames, w.frame_h, w.frame_w],
                   "heads": w.heads, "head_dim": w.head_dim, "page_tokens": w.page_tokens,
                   "mask_aware_flops_per_round": F, "out_dtype": args.out_dtype,
                   "live_mask": w.live_mask, "layers": L},
        "rounds_per_sec": round(1e3 / ms_step, 3),
        "attention_ms": round(att_avg, 4),
        "attention_ms_minmax": [round(min(att_ms), 4), round(max(att_ms), 4)],
        "attention_ms_median": round(float(np.median(att_ms)), 4),
        "stream_ms_per_step": round(float(np.mean(gpu_ms)), 4),
        # stream time not spent in the step's kernels (launch gaps), one layer only
        "launch_gap_ms": (round(float(np.mean(gpu_ms)) - att_avg - pub_avg - float(np.mean(adv_ms)), 4)
                          if L == 1 else None),
        "publish_ms": round(pub_avg, 4),
        "advance_ms": round(float(np.mean(adv_ms)), 4),
        "attention_tflops": round(attn_tflops, 2),
        "publish_gbps": round(pub_bytes / (pub_avg * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": round(attn_peak, 1),
                     "unit": "TFLOP/s", "frac": round(attn_tflops / attn_peak, 4),
                     "traffic": traffic},
        "publish_roofline": {"bound": "hbm", "achieved": round(pub_bytes / (pub_avg * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": round(pub_bytes / (pub_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                             "algorithmic_bytes": pub_bytes,
                             "d2d_memcpy_gbps": round(copy_gbps, 1),
                             "frac_of_d2d_memcpy": round(pub_bytes / (pub_avg * 1e-3) / 1e9 / copy_gbps, 4),
                             "stream_copy_gbps": round(stream_gbps, 1),
                             "frac_of_stream_copy": round(pub_bytes / (pub_avg * 1e-3) / 1e9 / stream_gbps, 4)},
    }
    def _spread(key):
        v = [b[key] for b in blocks]
        return {"median": round(float(np.median(v)), 4), "min": round(min(v), 4), "max": round(max(v), 4),
                "blocks": [round(x, 4) for x in v]}
    res["repeats"] = {"blocks": len(blocks), "steps_per_block": K, "ms_per_step": _spread("ms_per_step"),
                      "attention_ms": _spread("attention_ms"), "publish_ms": _spread("publish_ms")}
    f0 = 4.0 * w.N * w.N * w.head_dim * w.heads * w.T         # slot 0 reads all T chunks under either mask
    s0 = float(np.mean(slot0_ms))
    res["critical_slot"] = {"slot": 0, "key_chunks": w.T, "attention_ms": round(s0, 4),
                            "attention_ms_minmax": [round(min(slot0_ms), 4), round(max(slot0_ms), 4)],
                            "flops": f0, "tflops": round(f0 / (s0 * 1e-3) / 1e12, 2),
                            "launches": K}
    cal_tflops = cal_flops / (float(np.median(cal_ms)) * 1e-3) / 1e12
    res["mfma_ceiling"] = {"tflops": round(cal_tflops, 1), "frac_of_peak": round(cal_tflops / PEAK_BF16_TFLOPS, 4),
                           # the ceiling is that of bf16 MFMAs: compared with bf16 attention only
                           "attention_frac_of_ceiling": (round(attn_tflops / cal_tflops, 4)
                                                         if w.qk_dtype == "bf16" else None),
                           "ms": round(float(np.median(cal_ms)), 4), "cus": ncu,
                           "what": "wf_mfma_calibrate: the attention step's 32 bf16 MFMAs per wave, operands in "
                                   "registers, one 8-wave workgroup per CU, 4096 steps, median of 5 launches"}
    if graph is not None:
        res["graph"] = graph
    if proj is not None:
        res["projection"] = proj
        res["config"]["publish"] = ("per-token e4m3 quantisation + W8A8 fused QKV projection + RoPE + publish"
                                    if args.project == "w8a8" else "fused QKV projection + RoPE + publish")
        del res["publish_roofline"]
        del res["publish_gbps"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_rows, args.cpu_workers)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, rows_per_slot_head, max_workers):
    """The fp64 oracle on the same round, timed on the host's cores.

    The oracle as it stands evaluates every (slot, head) unit of the round
    (every query row, or `rows_per_slot_head` rows spread over the chunk),
    each unit in a worker process with single-threaded BLAS, one worker per
    core up to `max_workers`; each worker draws the round's seeded inputs
    once and rotates the context chunks of its heads. FLOPs are the
    mask-aware QK^T + PV FLOPs of the evaluated rows."""
    import numpy as np
    from oracle.parallel import host_workers, oracle_units
    workers = host_workers(max_workers)
    k = w.steady_round
    rows = None if rows_per_slot_head <= 0 else np.linspace(0, w.N - 1, rows_per_slot_head).astype(np.int64)
    nrows = w.N if rows is None else len(rows)
    units = [(s, (h,)) for s in range(w.S + 1) for h in range(w.heads)]
    storage = "fp8" if w.qk_dtype == "fp8" else "bf16"        # the published page format
    t0 = time.perf_counter()
    for _ in oracle_units(w, k, units, storage, rows=rows, workers=workers):
        pass
    dt = time.perf_counter() - t0
    pairs = w.key_chunk_pairs()
    flops = 4.0 * nrows * w.N * w.head_dim * w.heads * pairs
    what = "the whole round" if rows is None else "%d query rows per (slot, head)" % nrows
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers),
            "kind": "oracle",
            "sample": "%s round k=%d, %s: all %d slots x %d heads over the full legal context, "
                      "RoPE and %s storage of the context chunks included; fp64 numpy, %d worker "
                      "processes x 1 BLAS thread; %.1f s"
                      % (w.name, k, what, w.S + 1, w.heads, storage, workers, dt)}


if __name__ == "__main__":
    main()
