"""MI355X (gfx950) wavefront-round attention: paged K/V pool, fused 3D-RoPE
publish and chunk-causal flash attention behind a C ABI (libwf.so).

Python side: `_lib` is the ctypes binding (same names as include/wf.h);
`Pool` owns torch-allocated device memory for one pool and forwards to it.
All computation runs in the HIP kernels of libwf.so; there is no fallback.
"""
from __future__ import annotations

from ._lib import (WF_DTYPE_BF16, WF_DTYPE_FP32, WF_DTYPE_FP8_E4M3, WF_E_HIP, WF_E_INVALID_ARG,
                   WF_E_NOT_READY, WF_E_SHAPE, WF_MASK_ALL_LIVE, WF_MASK_WAVEFRONT, WF_OK, WfError,
                   load, wf_attention_round, wf_attention_work_list, wf_config,
                   wf_geometry, wf_kv_publish, wf_page_table_host, wf_pool_bytes, wf_pool_create,
                   wf_qkv_project_publish, wf_qkv_project_publish_w8a8, wf_quantize_rows_fp8,
                   wf_pool_create_host_model, wf_pool_destroy, wf_ready_mask, wf_round_advance,
                   wf_round_index, wf_round_replayed, wf_schedule_chunk_ids, wf_mfma_calibrate,
                   wf_stream_copy_calibrate)

_DT = {"bf16": WF_DTYPE_BF16, "fp32": WF_DTYPE_FP32, "fp8": WF_DTYPE_FP8_E4M3}


def make_config(S, anchor_chunks, history_chunks, heads, head_dim, chunk_frames, frame_h, frame_w,
                page_tokens, in_dtype="bf16", qk_dtype="bf16", rope_split=None, rope_theta=1e4,
                first_round=None, num_layers=1, live_mask="wavefront", total_chunks=0) -> wf_config:
    """live_mask: "wavefront" (M_WF, the default) or "all" (every live slot sees
    every live slot; no tile is skipped). first_round below S+H+A starts in the
    rounds that fill the pipeline; total_chunks > 0 ends the video (its last S
    rounds drain the pipeline)."""
    c = wf_config()
    c.S, c.anchor_chunks, c.history_chunks = S, anchor_chunks, history_chunks
    c.heads, c.head_dim, c.num_layers = heads, head_dim, num_layers
    c.chunk_frames, c.frame_h, c.frame_w, c.page_tokens = chunk_frames, frame_h, frame_w, page_tokens
    c.in_dtype, c.qk_dtype = _DT[in_dtype], _DT[qk_dtype]
    if rope_split is None:
        dh = 2 * (head_dim // 6)
        rope_split = (head_dim - 2 * dh, dh, dh)
    c.rope_split[0], c.rope_split[1], c.rope_split[2] = rope_split
    c.rope_theta = float(rope_theta)
    c.first_round = S + history_chunks + anchor_chunks if first_round is None else first_round
    c.live_mask = {"wavefront": WF_MASK_WAVEFRONT, "all": WF_MASK_ALL_LIVE}[live_mask]
    c.total_chunks = int(total_chunks)
    return c


class Pool:
    """One K/V slot pool with its page table, in torch-allocated device memory."""

    def __init__(self, cfg: wf_config, device="cuda"):
        import torch
        self.cfg = cfg
        self.pool_bytes, self.table_bytes = wf_pool_bytes(cfg)
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=device)
        self.table = torch.empty(self.table_bytes // 4, dtype=torch.int32, device=device)
        self.handle = wf_pool_create(cfg, self.pool, self.pool_bytes, self.table, self.table_bytes)
        g = wf_geometry(self.handle)
        self.N, self.T, self.ppc = g["N"], g["T"], g["ppc"]
        self.geometry = g

    def close(self):
        if self.handle:
            wf_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def q_buffer(self):
        import torch
        c = self.cfg
        dt = torch.uint8 if c.qk_dtype == WF_DTYPE_FP8_E4M3 else torch.bfloat16
        return torch.empty((c.S + 1, c.heads, self.N, c.head_dim), dtype=dt, device=self.pool.device)

    def q_scale_buffer(self):
        import torch
        c = self.cfg
        if c.qk_dtype != WF_DTYPE_FP8_E4M3:
            return None
        return torch.empty((c.S + 1, c.heads, (self.N + 63) // 64), dtype=torch.float32,
                           device=self.pool.device)

    def out_buffer(self, dtype="fp32"):
        import torch
        c = self.cfg
        dt = torch.float32 if dtype == "fp32" else torch.bfloat16
        return torch.empty((c.S + 1, self.N, c.heads * c.head_dim), dtype=dt, device=self.pool.device)

    def publish(self, layer, slot_first, nslots, q, k, v, row_stride, q_out=None, q_scales=None,
                chunk_t0=None, stream=None, noalloc=False):
        """noalloc: through wf_kv_publish_noalloc (scratch from the library's
        static per-GPU array, not the pool)."""
        wf_kv_publish(self.handle, layer, slot_first, nslots, q, k, v, row_stride, chunk_t0,
                      q_out, q_scales, stream, noalloc)

    def project_publish(self, layer, slot_first, nslots, x, x_row_stride, hidden, w, bias=None, q_out=None,
                        chunk_t0=None, stream=None):
        wf_qkv_project_publish(self.handle, layer, slot_first, nslots, x, x_row_stride, hidden, w, bias,
                               chunk_t0, q_out, stream)

    def project_publish_w8a8(self, layer, slot_first, nslots, x8, x_row_stride, x_scales, hidden, w8, w_scales,
                             bias=None, q_out=None, chunk_t0=None, stream=None):
        wf_qkv_project_publish_w8a8(self.handle, layer, slot_first, nslots, x8, x_row_stride, x_scales, hidden,
                                    w8, w_scales, bias, chunk_t0, q_out, stream)

    def attention(self, layer, slot_first, nslots, q, out, q_scales=None, stream=None):
        import torch
        od = WF_DTYPE_FP32 if out.dtype == torch.float32 else WF_DTYPE_BF16
        wf_attention_round(self.handle, layer, slot_first, nslots, q, q_scales, out, od, stream)

    def advance(self, stream=None):
        wf_round_advance(self.handle, stream)

    def round_replayed(self):
        """Host bookkeeping after one replay of a captured round."""
        wf_round_replayed(self.handle)

    def round_index(self):
        return wf_round_index(self.handle)

    def chunk_ids(self):
        return wf_schedule_chunk_ids(self.handle, self.T)

    def page_table_host(self):
        return wf_page_table_host(self.handle, self.T * self.ppc)

    def ready_mask(self, layer=0):
        return wf_ready_mask(self.handle, layer)


def quantize_rows_fp8(x, codes=None, scales=None, stream=None):
    """Per-row e4m3 codes and fp32 scales of a 2-D bf16 device tensor (rows
    16-byte aligned), for the W8A8 projection. Returns (codes uint8 [rows,
    cols] with 16-byte row pitch, scales float32 [rows])."""
    import torch
    rows, cols = x.shape
    if codes is None:
        pitch = (cols + 15) // 16 * 16
        codes = torch.empty((rows, pitch), dtype=torch.uint8, device=x.device)[:, :cols]
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    wf_quantize_rows_fp8(x, rows, cols, x.stride(0), codes, codes.stride(0), scales, stream)
    return codes, scales
