"""fp64 CPU oracle for one wavefront round of chunk-wise causal attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library or its Python binding may
import, call or link anything under this package; only the tests, the smoke
check and the benchmark's CPU-baseline leg do. The oracle shares no code with
the HIP path: it has its own schedule model, RoPE, rounding emulation and
attention, written from the method's definition, slowly and plainly.

Sources (the Wave Forcing pages, arXiv 2611.00859):
  * hyper.ai summary, section "Method": rounds k = i + s, full attention within
    a chunk, chunk-causal attention in time, mask M_WF(s, j) = 1[j >= s].
  * e-cogni.com.br article, section "Como funciona": the ordered per-layer
    context anchor | bounded clean history | live store | denoising K/V; a
    query slot reads itself and cleaner predecessors only.
  * thelatestinai.com listing, Table 3 (notation: stage s, store = stage S,
    rank S is Store) and Figure 1 (S=4 wavefront, one chunk per round).
  * hyper.ai summary, section "Method" (WaveRT paragraph): K/V are published
    after QKV projection and RoPE.
  * thelatestinai.com listing, Table 11: model widths (hidden = heads x 128),
    the shape of the QKV projection that precedes RoPE.
  * e-cogni.com.br article, section "Como funciona", and thelatestinai.com
    listing, Table 6: W8A8 (8-bit weights and activations) in the projections.

Where the pages are silent the oracle takes these readings: softmax scale
1/sqrt(d); adjacent-pair 3D RoPE on contiguous t|h|w channel ranges with
per-axis frequencies theta^(-2m/d_a); token order frame, row, column; absolute
latent-frame position chunk_frames * chunk_id + frame; published Q/K stored as
bf16 (or fp8 e4m3 with per-64-token-block absmax scales and a per-chunk K mean).

Parity status: every function here is pinned by a CPU test against the pages'
closed forms, invariants, brute force or a library routine. The fp8 storage
model (per-64-token block scales restarting at each chunk, the per-chunk K mean
removed and added back) is pinned by properties of that definition: the
half-step error bound per block, exact reconstruction at each block's absmax
and of a chunk constant along tokens, a short last block with its own scale,
power-of-two equivariance, and blocks restarting at every chunk of a built
context; its encoder is pinned to torch's float8_e4m3fn cast. What the pages
do not fix is the choice of that scheme (they only name an fp8 payload with
scales). Likewise the W8A8 format (e4m3, one scale per token and per output
channel) is a reading: its quantiser is pinned to brute-force nearest rounding
and its projection to exact rational arithmetic, but the choice of format and
granularity is not fixed by the pages.
"""
from .schedule import (RoundSchedule, live_mask, legal_positions, GroupRing,
                       slot_position)
from .rope import rope_split, token_grid, rope_3d
from .numerics import (bf16_round, fp8_e4m3_encode, fp8_e4m3_decode,
                       fp8_block_quantize, FP8_E4M3_MAX)
from .attention import (masked_softmax_attention, slot_attention, round_attention,
                        dense_round_attention)
from .round import oracle_round, rotate_chunk, rotated_context
from .projection import project_qkv, project_qkv_w8a8, quantize_rows_fp8, split_qkv

__all__ = [
    "RoundSchedule", "live_mask", "legal_positions", "GroupRing", "slot_position",
    "rope_split", "token_grid", "rope_3d",
    "bf16_round", "fp8_e4m3_encode", "fp8_e4m3_decode", "fp8_block_quantize",
    "FP8_E4M3_MAX",
    "masked_softmax_attention", "slot_attention", "round_attention",
    "dense_round_attention",
    "oracle_round", "rotate_chunk", "rotated_context",
    "project_qkv", "split_qkv", "quantize_rows_fp8", "project_qkv_w8a8",
]
