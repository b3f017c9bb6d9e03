"""Seeded synthetic inputs for wavefront-round attention.

This module is shared by the tests, the benchmark and the smoke check. It holds
only workload shapes and random draws: no RoPE, no schedule, no attention and
no quantisation. Both the fp64 oracle and the HIP path consume what it returns.

Workloads follow the Wave Forcing pages: Wan2.1 model widths (p5 Table 11),
3 latent frames per chunk at 832x480 (p3 metrics table; p4 limitations), and
the pages' own system runs use dummy DiT weights (p5 Fig. 7 caption, Table 4
caption), so activations are drawn i.i.d. N(0, 1).

Draw key: every (workload seed, round, slot) triple owns an independent PCG64
stream, from which q, k and v are drawn in that order. A chunk that a round
publishes from the store slot (slot S) becomes clean history later; its K/V are
therefore re-drawn with the key (seed, round it was stored in, S).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    S: int                 # denoising slots; the store is slot S
    A: int                 # anchor chunks
    H: int                 # clean-history ring chunks
    heads: int
    head_dim: int
    chunk_frames: int      # latent frames per chunk
    frame_h: int           # patch rows per latent frame
    frame_w: int           # patch columns per latent frame
    page_tokens: int       # tokens per K/V page (divides the chunk)
    in_dtype: str          # "fp32" | "bf16": dtype of the projected Q/K/V
    qk_dtype: str          # "bf16" | "fp8": published Q/K format
    rope_split: tuple      # (d_t, d_h, d_w)
    rope_theta: float
    seed: int
    outlier_frac: float = 0.0     # fraction of the h*d channels scaled in Q and K
    outlier_scale: float = 1.0
    fused_qkv: bool = False       # input is one [tokens, 3*h*d] projection output
    layer_rounds: int = 1         # consecutive rounds of one layer's pool
    live_mask: str = "wavefront"  # "wavefront" (M_WF) or "all" (every live slot sees every live slot)
    description: str = ""

    @property
    def N(self) -> int:
        return self.chunk_frames * self.frame_h * self.frame_w

    @property
    def T(self) -> int:
        """Ordered context positions: anchor | history | store | slots S-1..0."""
        return self.A + self.H + self.S + 1

    @property
    def hd(self) -> int:
        return self.heads * self.head_dim

    @property
    def steady_round(self) -> int:
        """First round whose history ring is full of chunks other than the anchor."""
        return self.S + self.H + self.A

    def key_chunk_pairs(self) -> int:
        """Legal (query chunk, key chunk) pairs in one round (all slots)."""
        if self.live_mask == "all":
            return (self.S + 1) * self.T
        return (self.S + 1) * (self.A + self.H) + (self.S + 1) * (self.S + 2) // 2

    def attention_flops(self) -> float:
        """Mask-aware FLOPs of one round: QK^T plus PV, one multiply-add = 2."""
        return 4.0 * self.N * self.N * self.head_dim * self.heads * self.key_chunk_pairs()


def _split(d: int) -> tuple:
    dh = 2 * (d // 6)
    return (d - 2 * dh, dh, dh)


WORKLOADS = {
    # Tiny CPU-checkable round: S=2 + store, one 8x8 latent frame per chunk.
    "tiny": Workload("tiny", S=2, A=1, H=2, heads=2, head_dim=64, chunk_frames=1,
                     frame_h=8, frame_w=8, page_tokens=64, in_dtype="fp32", qk_dtype="bf16",
                     rope_split=_split(64), rope_theta=1e4, seed=1,
                     description="S=2+store, chunk 64 tokens (1x8x8), A=1, H=2, 2 heads x 64, fp32"),
    # Wan2.1-1.3B, 4-step WF: chunk = 3 latent frames x 30x52 patches.
    "wan1.3b_s4": Workload("wan1.3b_s4", S=4, A=1, H=2, heads=12, head_dim=128, chunk_frames=3,
                           frame_h=30, frame_w=52, page_tokens=1560, in_dtype="bf16",
                           qk_dtype="bf16", rope_split=(44, 42, 42), rope_theta=1e4, seed=2,
                           description="Wan2.1-1.3B S=4+store, chunk 4680 (3x30x52), 12x128, A=1 H=2, bf16"),
    # Wan2.1-1.3B, 5-step WF, 30 consecutive layer-rounds with rotation.
    "wan1.3b_s5_30": Workload("wan1.3b_s5_30", S=5, A=1, H=2, heads=12, head_dim=128,
                              chunk_frames=3, frame_h=30, frame_w=52, page_tokens=1560,
                              in_dtype="bf16", qk_dtype="bf16", rope_split=(44, 42, 42),
                              rope_theta=1e4, seed=3, layer_rounds=30,
                              description="Wan2.1-1.3B S=5+store, 30 consecutive layer-rounds"),
    # 14B-class: 40 heads, history ring 3, 1% outlier channels x20 in Q and K.
    "wan14b_s4": Workload("wan14b_s4", S=4, A=1, H=3, heads=40, head_dim=128, chunk_frames=3,
                          frame_h=30, frame_w=52, page_tokens=1560, in_dtype="bf16",
                          qk_dtype="bf16", rope_split=(44, 42, 42), rope_theta=1e4, seed=4,
                          outlier_frac=0.01, outlier_scale=20.0,
                          description="14B-class S=4+store, chunk 4680, 40x128, H=3, Q/K outliers"),
    # Quantised QK path from a fused bf16 QKV projection output.
    "wan1.3b_s4_fp8": Workload("wan1.3b_s4_fp8", S=4, A=1, H=2, heads=12, head_dim=128,
                               chunk_frames=3, frame_h=30, frame_w=52, page_tokens=1560,
                               in_dtype="bf16", qk_dtype="fp8", rope_split=(44, 42, 42),
                               rope_theta=1e4, seed=5, fused_qkv=True,
                               description="Wan2.1-1.3B S=4 round, Q/K fp8 e4m3, fused QKV input"),
    # Mid-size parity shapes: several tiles, ragged query and key tails, pages
    # that key tiles straddle.
    "ragged128": Workload("ragged128", S=3, A=1, H=2, heads=3, head_dim=128, chunk_frames=2,
                          frame_h=12, frame_w=13, page_tokens=104, in_dtype="bf16",
                          qk_dtype="bf16", rope_split=(44, 42, 42), rope_theta=1e4, seed=11,
                          description="S=3, chunk 312 (2x12x13), page 104, 3x128, bf16"),
    "ragged64": Workload("ragged64", S=3, A=1, H=1, heads=2, head_dim=64, chunk_frames=3,
                         frame_h=6, frame_w=12, page_tokens=72, in_dtype="bf16", qk_dtype="bf16",
                         rope_split=_split(64), rope_theta=1e4, seed=12,
                         description="S=3, chunk 216 (3x6x12), page 72, 2x64, bf16"),
    # Degenerate schedule: one denoising slot, two anchor chunks, no history;
    # 24-token pages, so 64-key tiles straddle pages and chunks.
    "edge_s1_h0": Workload("edge_s1_h0", S=1, A=2, H=0, heads=2, head_dim=64, chunk_frames=1,
                           frame_h=8, frame_w=9, page_tokens=24, in_dtype="bf16", qk_dtype="bf16",
                           rope_split=_split(64), rope_theta=1e4, seed=14,
                           description="S=1, A=2, H=0, chunk 72 (1x8x9), page 24, 2x64, bf16"),
    # Largest schedule the library takes: T = A+H+S+1 = 64 context positions
    # (every bit of the readiness mask) and T x pages-per-chunk = 1024 pages
    # (the attention kernel's LDS page table, full), 8192-key contexts.
    "max64": Workload("max64", S=30, A=1, H=32, heads=2, head_dim=64, chunk_frames=2,
                      frame_h=8, frame_w=8, page_tokens=8, in_dtype="bf16", qk_dtype="bf16",
                      rope_split=_split(64), rope_theta=1e4, seed=17,
                      description="S=30, A=1, H=32: T=64, chunk 128 (2x8x8), page 8 (1024 pages), 2x64"),
    # The most query slots the library takes: S = 62 (slots 32..62 use the
    # work-list entry's high slot bits), T = 64, one 8x8 frame per chunk.
    "slots62": Workload("slots62", S=62, A=1, H=0, heads=2, head_dim=64, chunk_frames=1,
                        frame_h=8, frame_w=8, page_tokens=64, in_dtype="bf16", qk_dtype="bf16",
                        rope_split=_split(64), rope_theta=1e4, seed=18,
                        description="S=62, A=1, H=0: T=64, 63 query slots, chunk 64 (1x8x8), 2x64"),
    # fp8 QK with chunks shorter than one 64-key tile.
    "tiny_fp8": Workload("tiny_fp8", S=2, A=1, H=1, heads=2, head_dim=64, chunk_frames=1,
                         frame_h=6, frame_w=8, page_tokens=24, in_dtype="bf16", qk_dtype="fp8",
                         rope_split=_split(64), rope_theta=1e4, seed=16,
                         description="fp8 QK, chunk 48 (1x6x8), page 24, 2x64, separate inputs"),
    # fp8 QK at head_dim 64 from separate Q/K/V inputs.
    "ragged_fp8_64": Workload("ragged_fp8_64", S=2, A=1, H=1, heads=2, head_dim=64, chunk_frames=2,
                              frame_h=6, frame_w=10, page_tokens=40, in_dtype="bf16", qk_dtype="fp8",
                              rope_split=_split(64), rope_theta=1e4, seed=15,
                              description="fp8 QK, chunk 120 (2x6x10), page 40, 2x64, separate inputs"),
    "ragged_fp8": Workload("ragged_fp8", S=3, A=1, H=2, heads=3, head_dim=128, chunk_frames=2,
                           frame_h=12, frame_w=13, page_tokens=104, in_dtype="bf16",
                           qk_dtype="fp8", rope_split=(44, 42, 42), rope_theta=1e4, seed=13,
                           fused_qkv=True,
                           description="fp8 QK, chunk 312 (2x12x13), 3x128, fused QKV"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("round_to_bf16 expects finite values")
    u = x.view(np.uint32) if x.flags.c_contiguous else np.ascontiguousarray(x).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                                           # finite inputs cannot overflow
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def outlier_channels(w: Workload) -> np.ndarray:
    """The fixed set of h*d channel indices scaled in Q and K (empty if none)."""
    n = int(round(w.outlier_frac * w.hd))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0x6F75])))
    return np.sort(rng.choice(w.hd, size=n, replace=False))


def draw(w: Workload, round_index: int, slot: int):
    """Pre-RoPE q, k, v of one chunk as float32 [N, heads*head_dim].

    Values are bf16-exact when the workload's input dtype is bf16.
    """
    ss = np.random.SeedSequence([w.seed, int(round_index), int(slot)])
    rng = np.random.Generator(np.random.PCG64(ss))
    shape = (w.N, w.hd)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    ch = outlier_channels(w)
    if ch.size:
        q[:, ch] *= np.float32(w.outlier_scale)
        k[:, ch] *= np.float32(w.outlier_scale)
    if w.in_dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def draw_hidden(w: Workload, round_index: int, slot: int) -> np.ndarray:
    """Hidden states entering the QKV projection for one chunk: float32
    [N, hidden] (hidden = heads * head_dim, the Wan2.1 widths), N(0, 1),
    bf16-exact. Own stream per (seed, round, slot), apart from draw()'s."""
    ss = np.random.SeedSequence([w.seed, 0x68696464, int(round_index), int(slot)])
    rng = np.random.Generator(np.random.PCG64(ss))
    return round_to_bf16(rng.standard_normal((w.N, w.hd), dtype=np.float32))


def projection_weights(w: Workload, layer: int = 0):
    """Random-init QKV projection of one layer: weight float32 [3*h*d, hidden]
    ([out, in]) ~ N(0, 1/hidden), bias float32 [3*h*d] ~ N(0, 0.1^2), both
    bf16-exact, so the projected Q/K/V are about N(0, 1)."""
    ss = np.random.SeedSequence([w.seed, 0x77716b76, int(layer)])
    rng = np.random.Generator(np.random.PCG64(ss))
    wt = rng.standard_normal((3 * w.hd, w.hd), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.hd))
    b = rng.standard_normal(3 * w.hd, dtype=np.float32) * np.float32(0.1)
    return round_to_bf16(wt), round_to_bf16(b)


def stored_draw(w: Workload, chunk_id: int):
    """K/V of a clean chunk as published by the store slot (round chunk_id + S)."""
    return draw(w, chunk_id + w.S, w.S)


def draw_slots(w: Workload, round_index: int, slots, threads: int = 8):
    """draw() for several slots of one round, drawn concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    slots = list(slots)
    with ThreadPoolExecutor(max(1, min(threads, len(slots)))) as ex:
        return list(ex.map(lambda s: draw(w, round_index, s), slots))
