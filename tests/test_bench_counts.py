"""The benchmark's work counts and contract, on the CPU.

The rates bench.py reports divide a count of visible (query, key) pairs by a
measured time.  These tests pin those counts to the oracle's own visibility
mask, counted element by element on small shares: the zigzag share of every
ring rank ([USP review] section 三, Algorithm 2; [CP vs Ulysses] Figure 2,
every rank the same causal work), packed samples under the whole-stream split
and under the per-sample split ([ByteScale notes], motivation).  They also
check the single-GPU refusal and the source-hash key of the traffic record.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attention as oa  # noqa: E402
from oracle import index as ix  # noqa: E402


def mask_pairs(q_pos, k_pos, cu=None):
    """Visible pairs by the oracle's mask, every (query, key) element counted."""
    seg = None if cu is None else ix.segment_start(cu, q_pos)
    return int(oa._visible(np.asarray(q_pos), np.asarray(k_pos), True, seg).sum())


@pytest.mark.parametrize("S,rd", [(8, 1), (24, 2), (48, 3), (64, 4), (96, 4), (128, 8)])
def test_share_walk_flops_count_visible_pairs(S, rd):
    c = S // (2 * rd)
    D, heads, B = 64, 3, 2
    half, exact = bench.share_walk_flops(D, heads, B, rd, c)
    keys = np.arange(S)
    for r in range(rd):
        pairs = mask_pairs(ix.zigzag_share_positions(S, rd, r), keys)
        assert exact == 4.0 * D * heads * B * pairs, (r, pairs)
        # the half-diagonal convention drops half of each of the two diagonal cells' diagonals
        assert half == 4.0 * D * heads * B * (pairs - c)


def test_all_ranks_half_diagonal_is_the_sum_over_ranks():
    """The all-ranks launches (the 8K MHA workload) count 2 B H S^2 D flops:
    the ranks' half-diagonal counts summed, S^2 / 2 pairs per head."""
    S, rd, D, H, B = 96, 4, 32, 2, 1
    total = sum(bench.share_walk_flops(D, H, B, rd, S // (2 * rd))[0] for _ in range(rd))
    assert total == 2.0 * B * H * S * S * D


def _random_cu(rng, S, n, multiple=1):
    cuts = np.sort(rng.choice(np.arange(1, S // multiple), size=n - 1, replace=False)) * multiple
    return np.concatenate([[0], cuts, [S]]).astype(np.int64)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_pairs_match_the_mask(seed):
    rng = np.random.default_rng(seed)
    S, rd = 128, 4
    cu = _random_cu(rng, S, 5)
    keys = np.arange(S)
    for r in range(rd):
        pos = ix.zigzag_share_positions(S, rd, r)
        assert bench.packed_pairs(cu, pos) == mask_pairs(pos, keys, cu)
    # a single sample is the unpacked causal count
    pos = ix.zigzag_share_positions(S, rd, 1)
    assert bench.packed_pairs(np.array([0, S]), pos) == mask_pairs(pos, keys)


@pytest.mark.parametrize("seed,rd", [(3, 2), (4, 4), (5, 3)])
def test_per_sample_pairs_match_the_mask_on_every_rank(seed, rd):
    rng = np.random.default_rng(seed)
    S = 2 * rd * 24
    cu = _random_cu(rng, S, 4, multiple=2 * rd)
    keys = np.arange(S)
    want = bench.per_sample_pairs(cu, rd)
    for r in range(rd):
        pos = ix.zigzag_per_sample_positions(cu, rd, r)
        assert mask_pairs(pos, keys, cu) == want, r


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "single MI355X" in p.stderr
    assert p.stdout == ""


def test_traffic_record_is_keyed_by_the_walk_source(monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["kernel_source_sha256_16"])
    assert bench.measured_traffic() == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic() is None
