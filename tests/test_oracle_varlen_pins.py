"""Pins of the per-sample zigzag split (Algorithm 2 applied to every packed
sample on its own) against what the pages and counting fix.

* with one sample it is Algorithm 2's split of the whole sequence;
* the ranks' shares partition the positions, each share sorted;
* the causal work is exactly equal on every rank (the pairing argument of
  [CP vs Ulysses] Figure 2, sample by sample), with its closed form;
* USP with this split merges to one-shot attention of the packed samples;
* lengths that do not divide by 2*rd are rejected.
A mutation test plants a wrong chunk partner and shows the balance pin fails.
"""
import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import index as ix
from oracle import usp as ou

CASES = [  # cu_seqlens, rd
    ([0, 64], 4),
    ([0, 16, 24, 64, 96], 2),
    ([0, 8, 16, 40, 48, 128], 4),
    ([0, 48, 96, 240], 3),
    ([0, 32, 64], 1),
]


def check_balance(cu, rd):
    """Visible (query, key) pairs of every rank, which must all be equal; and
    their closed form sum_n [(2 rd - 1) m_n^2 + m_n (m_n + 1)], m_n = s_n / (2 rd)."""
    S = cu[-1]
    keys = np.arange(S)
    loads = []
    for r in range(rd):
        q = ix.zigzag_per_sample_positions(cu, rd, r)
        loads.append(ix.visible_pairs(q, keys, ix.segment_start(cu, q)))
    m = np.diff(cu) // (2 * rd)
    closed = int(((2 * rd - 1) * m * m + m * (m + 1)).sum())
    return loads, closed


@pytest.mark.parametrize("cu,rd", CASES)
def test_v1_balance_exact(cu, rd):
    loads, closed = check_balance(cu, rd)
    assert all(x == closed for x in loads), (loads, closed)


@pytest.mark.parametrize("cu,rd", CASES)
def test_v2_shares_partition_the_sequence(cu, rd):
    S = cu[-1]
    shares = [ix.zigzag_per_sample_positions(cu, rd, r) for r in range(rd)]
    for sh in shares:
        assert len(sh) == S // rd and np.all(np.diff(sh) > 0)
    assert np.array_equal(np.sort(np.concatenate(shares)), np.arange(S))


@pytest.mark.parametrize("S,rd,ud", [(64, 4, 2), (96, 3, 1), (48, 2, 3)])
def test_v3_one_sample_is_algorithm_2(S, rd, ud):
    for r in range(rd):
        for u in range(ud):
            assert np.array_equal(ix.zigzag_per_sample_local_positions([0, S], rd, ud, r, u),
                                  ix.zigzag_local_positions(S, rd, ud, r, u))


def test_v4_stream_zigzag_is_not_balanced_on_the_same_samples():
    """The reading the per-sample split replaces: the same samples cut as one
    stream give unequal causal work (the imbalance the split removes)."""
    cu, rd = [0, 8, 16, 40, 48, 128], 4
    S = cu[-1]
    keys = np.arange(S)
    stream = [ix.visible_pairs(q, keys, ix.segment_start(cu, q))
              for q in (ix.zigzag_share_positions(S, rd, r) for r in range(rd))]
    assert len(set(stream)) > 1
    loads, _ = check_balance(cu, rd)
    assert max(stream) > max(loads)


@pytest.mark.parametrize("cu,rd,ud", [([0, 16, 24, 64, 96], 2, 2), ([0, 48, 96, 240], 3, 1),
                                      ([0, 8, 16, 40, 48, 128], 4, 2)])
def test_v5_usp_with_the_split_equals_one_shot(cu, rd, ud):
    rng = np.random.default_rng(77)
    S, H, Hkv, D = cu[-1], 4, 2, 8
    q, k, v = (rng.standard_normal((1, S, h, D)) for h in (H, Hkv, Hkv))
    scale = 1 / math.sqrt(D)
    o1, l1 = ou.usp_attention(q, k, v, rd, ud, scale, True, cu, per_sample=True)
    o2, l2 = oa.attention_full(q, k, v, scale, True, cu)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_v6_rejects_lengths_that_do_not_divide():
    with pytest.raises(ValueError):
        ix.zigzag_per_sample_positions([0, 12, 32], 4, 0)


def _wrong_partner(cu_seqlens, rd, ring_rank):
    """Chunks r and rd + r of every sample (the sequential partner)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    parts = []
    for n in range(len(cu) - 1):
        chunks = np.split(np.arange(cu[n], cu[n + 1]), 2 * rd)
        parts += [chunks[ring_rank], chunks[rd + ring_rank]]
    return np.concatenate(parts)


def test_v7_mutant_wrong_partner_fails_the_balance_pin(monkeypatch):
    monkeypatch.setattr(ix, "zigzag_per_sample_positions", _wrong_partner)
    loads, closed = check_balance([0, 8, 16, 40, 48, 128], 4)
    assert any(x != closed for x in loads)
