"""The algorithmic byte and flop counts that bench.py divides by measured
times (CPU only). They are checked against closed forms written out here:
a wrong term would misstate every GB/s and roofline fraction the bench
reports.

Per fused forward launch over T active tokens: x read (2 T h_in bytes), y
read and written (4 T h_out), each used adapter's A_i and B_i read once
(2 r_i (h_in + h_out)); flops 2 (h_in + h_out) per token and rank column.
"""
import numpy as np
import pytest

import bench


def _segs(lens, adapters):
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return starts, np.asarray(adapters, np.int32)


def test_decode_step_bytes_closed_form():
    """The decode step (256 tokens, 8 adapters of rank 32; q and o 2560 ->
    2560, gate_up 2560 -> 19456) moves 45 613 056 algorithmic bytes, so one
    launch averages 15 204 352."""
    starts, adap = _segs([32] * 8, range(8))
    ranks = np.full(8, 32)
    total = 0
    for h_out in (2560, 2560, 19456):
        b, f = bench.fwd_work(2560, h_out, ranks, starts, adap)
        assert b == 2 * 256 * 2560 + 4 * 256 * h_out + 2 * 8 * 32 * (2560 + h_out)
        assert f == 2 * (2560 + h_out) * 256 * 32
        total += b
    assert total == 45_613_056
    assert total // 3 == 15_204_352


def test_skipped_and_inactive_segments_move_nothing():
    """Tokens of segments without an adapter (-1) or of a rank-0 adapter, and
    adapters no token uses, add neither bytes nor flops."""
    ranks = np.array([8, 0, 16, 4])
    starts, adap = _segs([5, 7, 0, 3, 9], [0, 1, 2, -1, 2])
    b, f = bench.fwd_work(64, 32, ranks, starts, adap)
    T = 5 + 9  # adapter 0 (5 tokens), adapter 2 (9 tokens, its empty segment adds none)
    w = 8 * (64 + 32) + 16 * (64 + 32)
    assert b == 2 * T * 64 + 4 * T * 32 + 2 * w
    assert f == 2 * (64 + 32) * (5 * 8 + 9 * 16)
    bu, _ = bench.fwd_work(64, 32, ranks, starts, adap, save_u=True)
    assert bu - b == 4 * (5 * 8 + 9 * 16)


def test_shrink_expand_and_backward_closed_forms():
    ranks = np.array([16, 32])
    starts, adap = _segs([40, 24], [1, 0])
    tok_r = 40 * 32 + 24 * 16
    bs, fs = bench.shrink_work(128, ranks, starts, adap)
    assert bs == 2 * 64 * 128 + 2 * (16 + 32) * 128 + 4 * tok_r and fs == 2 * 128 * tok_r
    be, fe = bench.expand_work(96, ranks, starts, adap)
    assert be == 4 * tok_r + 2 * (16 + 32) * 96 + 4 * 64 * 96 and fe == 2 * 96 * tok_r
    bb, fb = bench.bwd_work(128, 96, ranks, starts, adap)
    w = (16 + 32) * (128 + 96)
    # dy and x read, dx read and written, u read, weights read, fp32 dA/dB written
    assert bb == 2 * 64 * 96 + 2 * 64 * 128 + 4 * 64 * 128 + 4 * tok_r + 2 * w + 4 * w
    assert fb == 4 * (128 + 96) * tok_r


@pytest.mark.parametrize("h_in,h_out", [(4096, 4096), (4096, 14336)])
def test_bytes_per_flop_bound(h_in, h_out):
    """The roofline argument: a token's x and y rows carry 2 h_in + 4 h_out
    bytes for 2 r (h_in + h_out) flops, so the fused forward's arithmetic
    intensity stays below r flops per byte (at most 2r/3 for square
    projections): HBM, not MFMA, bounds it at LoRA ranks."""
    r = 16
    starts, adap = _segs([1024] * 8, range(8))
    b, f = bench.fwd_work(h_in, h_out, np.full(8, r), starts, adap)
    per_token = 2 * r * (h_in + h_out) / (2 * h_in + 4 * h_out)
    assert f / b < per_token <= r
