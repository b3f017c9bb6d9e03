"""The matrix-core calibration kernel (wf_mfma_calibrate) does the MFMA work
it claims: the sum of its per-lane checksums over a wave equals, within fp32
accumulation error, the exact sum of every product its MFMAs accumulate,
computed on the host from the same operand values.

The sum of all elements of a product A B is sum_k colsum(A)[k] * rowsum(B)[k],
whatever the accumulator layout, so only the operand layout is used: lane l of
a v_mfma_f32_32x32x16_bf16 operand holds row (or column) l % 32 and the eight
k values 8 * (l // 32) + 0..7 (the layout the attention kernel's parity
tests already exercise). The checksum depends on every MFMA of every step, so
a kernel that skipped work (or a compiler that removed it) fails here.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, as float64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _lane_values(seed: np.ndarray) -> np.ndarray:
    """[lanes] seeds -> [lanes, 8] bf16 operand values in (-1, 1), never zero:
    the kernel's integer hash, h = (seed + i) * 2654435761 mod 2^32, h ^= h >> 15,
    value ((h & 0xFFFF) + 1/2) / 32768 - 1."""
    i = np.arange(8, dtype=np.uint64)
    h = ((seed.astype(np.uint64)[:, None] + i[None, :]) * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(15)
    f = (((h & np.uint64(0xFFFF)).astype(np.float64) + 0.5) / 32768.0 - 1.0).astype(np.float32)
    return _bf16(f)


def _wave_sum(a: np.ndarray, b: np.ndarray):
    """Sum of all elements of A B (and of |A| |B|) for one wave's fragments
    a, b [64, 8]: k = 8 * (lane // 32) + e."""
    ca = np.stack([a[:32].sum(0), a[32:].sum(0)]).reshape(16)
    cb = np.stack([b[:32].sum(0), b[32:].sum(0)]).reshape(16)
    aa = np.stack([np.abs(a[:32]).sum(0), np.abs(a[32:]).sum(0)]).reshape(16)
    ab = np.stack([np.abs(b[:32]).sum(0), np.abs(b[32:]).sum(0)]).reshape(16)
    return float(ca @ cb), float(aa @ ab)


def _expected(blocks: int, steps: int):
    """Per wave: exact total of the checksums and the sum of |products|."""
    out = []
    for blk in range(blocks):
        for w in range(8):
            ids = np.arange(64, dtype=np.uint64) + np.uint64(blk * 512 + w * 64)
            a = [_lane_values(ids * 64 + 16 * i) for i in range(4)]
            b = [_lane_values(ids * 64 + 16 * i + 8) for i in range(4)]
            tot = mag = 0.0
            # per step: 8 MFMAs a[k&3] b[(k+1)&3] and 8 a[(k+2)&3] b[k&3]
            # (score blocks), 16 a[d] b[g] (output blocks)
            for k in range(8):
                for ia, ib in ((k & 3, (k + 1) & 3), ((k + 2) & 3, k & 3)):
                    t, m = _wave_sum(a[ia], b[ib])
                    tot += t
                    mag += m
            for g in range(4):
                for d in range(4):
                    t, m = _wave_sum(a[d], b[g])
                    tot += t
                    mag += m
            out.append((steps * tot, steps * mag))
    return out


@pytest.mark.parametrize("blocks,steps", [(2, 3), (3, 17)])
def test_mfma_calibrate_checksum_equals_host_sum_of_products(blocks, steps):
    import wavefront_causal_attention_amd as wf
    from wavefront_causal_attention_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    wf.load()
    say("case mfma calibration blocks", blocks, "steps", steps)
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    _lib.wf_mfma_calibrate(blocks, steps, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    again = torch.full_like(out, float("nan"))
    _lib.wf_mfma_calibrate(blocks, steps, again)
    torch.cuda.synchronize()
    assert torch.equal(out, again)                   # deterministic
    exp = _expected(blocks, steps)
    worst = 0.0
    for wv, (tot, mag) in enumerate(exp):
        s = float(got[wv * 64:(wv + 1) * 64].sum())
        err = abs(s - tot) / mag
        worst = max(worst, err)
        # bf16 products summed in fp32 by the MFMAs and 96 accumulators per
        # lane summed in fp32: measured about 1e-8 of sum |products| (errors of
        # random sign), bar 2^-20; a dropped MFMA chain moves the total by a
        # third and a dropped step by 1/steps of it, 1e-4 of sum |products|
        assert err <= 2.0 ** -20, (wv, s, tot, mag)
    say("waves", len(exp), "worst |checksum - exact| / sum|products| = %.2e" % worst)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 215654400])
def test_stream_copy_calibrate_copies_exactly_the_bytes_asked(nbytes):
    """The streaming copy (the publish roofline's same-session HBM rate) moves
    exactly nbytes: the destination equals the source and the guard bytes
    after it are untouched."""
    from wavefront_causal_attention_amd import _lib
    say("case stream copy", nbytes, "bytes")
    guard = 4096
    g = torch.Generator(device="cpu").manual_seed(nbytes % 9973)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    _lib.wf_stream_copy_calibrate(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
