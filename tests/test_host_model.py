"""Pins for the work model the bench prices against (CPU only): the chunk
FLOP and on-chip byte counts printed on the pages (tests/golden)."""

import os

import pytest

from chunkwise_linear_attention_amd import perfmodel as pm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [l.split("#", 1)[0].split() for l in f if l.split("#", 1)[0].strip()]


def test_chunk_model_matches_pages():
    for row in _rows("chunk_model.txt"):
        kind, vals = row[0], list(map(int, row[1:]))
        if kind == "flop_ratio":
            big, small, dk, dv, want = vals
            T = 4096
            ratio = pm.sequence_flops(T, big, dk, dv) / pm.sequence_flops(T, small, dk, dv)
            assert round(ratio) == want
        elif kind == "balance":
            dk, dv, want = vals
            assert int(pm.balance_chunk(dk, dv)) == want
        elif kind == "bytes_inputs_bf16":
            Tc, d, kb = vals
            assert pm.onchip_bytes(Tc, d)["inputs_bf16"] == kb * 1024
        elif kind == "bytes_scores_f32":
            Tc, kb = vals
            assert pm.onchip_bytes(Tc, 128)["scores_f32"] == kb * 1024
        elif kind == "bytes_state_f32":
            d, kb = vals
            assert pm.onchip_bytes(64, d)["state_f32"] == kb * 1024
        else:
            raise AssertionError(kind)


def test_per_unit_counts():
    # forward chunk FLOPs per token-head times tokens equals the per-chunk model
    for dk, dv in ((64, 64), (128, 64), (128, 128)):
        per_tok = pm.chunk_flops_per_token_head(64, dk, dv, "fwd")
        assert per_tok * 64 == pm.chunk_flops(64, dk, dv)
    assert pm.chunk_bytes_per_token_head(128, 128, "fwd") == 4 * 128 + 4 * 128 + 4
    assert pm.chunk_bytes_per_token_head(128, 128, "bwd") == 8 * 128 + 6 * 128 + 8
    assert pm.scan_bytes_per_elem() == 32
    # the large diagonal-scan workload: 17.18 GB, 2.148 ms at 8 TB/s
    n = 8 * 16384 * 4096
    assert pm.roofline_seconds(32 * n) == pytest.approx(2.147e-3, rel=1e-3)
