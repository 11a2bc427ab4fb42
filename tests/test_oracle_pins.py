"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check is a plain function returning the worst error (or raising), so the
mutation tests at the bottom can plant a mistake in the oracle and show that
some pin catches it.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import comm
from oracle import index as ix
from oracle import merge as om
from oracle import usp as ou
from tests.conftest import golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, S, H, Hkv, D, seed):
    return _rand((B, S, H, D), seed), _rand((B, S, Hkv, D), seed + 1), _rand((B, S, Hkv, D), seed + 2)


def _err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isneginf(a) & np.isneginf(b)
    if np.any(np.isneginf(a) != np.isneginf(b)):
        return math.inf
    d = np.abs(np.where(both_inf, 0.0, a - np.where(both_inf, 0.0, b)))
    return float(d.max()) if d.size else 0.0


# --------------------------------------------------------------------------
# P1: brute force on tiny shapes (+ a library cross-check)
# --------------------------------------------------------------------------

BRUTE_CASES = [
    # B, S, H, Hkv, D, causal, cu_seqlens
    (1, 1, 1, 1, 4, True, None),
    (1, 7, 2, 1, 3, True, None),
    (2, 12, 4, 2, 8, True, None),
    (1, 16, 4, 1, 5, True, None),
    (1, 10, 2, 2, 4, False, None),
    (1, 16, 2, 1, 4, True, [0, 3, 4, 11, 16]),
    (2, 9, 4, 4, 2, True, [0, 9]),
]


def check_bruteforce(case, seed=11):
    B, S, H, Hkv, D, causal, cu = case
    q, k, v = _qkv(B, S, H, Hkv, D, seed)
    scale = 1.0 / math.sqrt(D)
    o1, l1 = oa.attention_full(q, k, v, scale, causal, cu)
    o2, l2 = oa.attention_bruteforce(q, k, v, scale, causal, cu)
    return max(_err(o1, o2), _err(l1, l2))


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_p1_bruteforce(case):
    assert check_bruteforce(case) <= 1e-13


def check_sdpa(B, S, H, Hkv, D, causal, cu, seed=5):
    """fp64 PyTorch scaled_dot_product_attention with KV heads repeated in
    contiguous groups; the lse comes from a separate logsumexp of the masked
    logits."""
    q, k, v = _qkv(B, S, H, Hkv, D, seed)
    scale = 1.0 / math.sqrt(D)
    o, lse = oa.attention_full(q, k, v, scale, causal, cu)
    G = H // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    mask = torch.ones(S, S, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask)
    if cu is not None:
        seg = torch.zeros(S, dtype=torch.long)
        for n in range(len(cu) - 1):
            seg[cu[n]:cu[n + 1]] = n
        mask &= seg[:, None] == seg[None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    logits = (tq @ tk.transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)     # (B, H, S)
    return max(_err(o, ref.permute(0, 2, 1, 3).numpy()),
               _err(lse, ref_lse.permute(1, 0, 2).numpy()))


@pytest.mark.parametrize("shape", [(1, 64, 4, 2, 16, True, None), (2, 40, 8, 8, 8, True, None),
                                   (1, 48, 4, 1, 8, False, None), (1, 96, 4, 2, 16, True, [0, 17, 60, 96])])
def test_p1_library_crosscheck(shape):
    assert check_sdpa(*shape) <= 1e-12


# --------------------------------------------------------------------------
# P2: closed forms
# --------------------------------------------------------------------------

def check_zero_queries(S=37, H=2, Hkv=1, D=6, cu=None):
    """Q = 0: every visible key has logit 0, so weights are uniform:
    lse_i = ln(#visible) and o_i = mean of the visible values."""
    _, k, v = _qkv(1, S, H, Hkv, D, 3)
    q = np.zeros((1, S, H, D))
    o, lse = oa.attention_full(q, k, v, 0.7, True, cu)
    start = np.zeros(S, dtype=np.int64) if cu is None else ix.segment_start(cu, np.arange(S))
    n = np.arange(S) - start + 1
    csum = np.concatenate([np.zeros((1, Hkv, D)), np.cumsum(v[0], axis=0)])
    mean = (csum[np.arange(S) + 1] - csum[start]) / n[:, None, None]
    worst = 0.0
    for h in range(H):
        worst = max(worst, _err(lse[h, 0], np.log(n)), _err(o[0, :, h], mean[:, h // (H // Hkv)]))
    return worst


def test_p2_zero_queries():
    assert check_zero_queries() <= 1e-13


def test_p2_zero_queries_packed():
    assert check_zero_queries(S=40, cu=[0, 5, 6, 23, 40]) <= 1e-13


def check_single_token():
    q, k, v = _qkv(1, 1, 2, 2, 5, 9)
    o, lse = oa.attention_full(q, k, v, 0.3)
    return max(_err(o, v), _err(lse[:, 0, 0], 0.3 * np.einsum("hd,hd->h", q[0, 0], k[0, 0])))


def test_p2_single_token():
    assert check_single_token() <= 1e-15


def check_dominant_key(S=10, j=3):
    """One key with a huge logit takes all the weight for every row that sees it."""
    D = 4
    q = np.zeros((1, S, 1, D)); q[..., 0] = 1.0
    k = np.zeros((1, S, 1, D)); k[0, j, 0, 0] = 2000.0
    v = _rand((1, S, 1, D), 4)
    o, lse = oa.attention_full(q, k, v, 0.5)
    rows = np.arange(j, S)
    return max(_err(o[0, rows, 0], np.broadcast_to(v[0, j, 0], (len(rows), D))),
               _err(lse[0, 0, rows], 1000.0))


def test_p2_dominant_key():
    assert check_dominant_key() <= 1e-12


def check_identical_keys(S=21, D=3):
    """All keys equal: uniform weights, lse_i = s + ln(i+1) with s the common logit."""
    q = _rand((1, S, 1, D), 6)
    kk = _rand((D,), 7)
    k = np.broadcast_to(kk, (1, S, 1, D)).copy()
    v = _rand((1, S, 1, D), 8)
    o, lse = oa.attention_full(q, k, v, 0.4)
    s = 0.4 * (q[0, :, 0] @ kk)
    mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
    return max(_err(o[0, :, 0], mean), _err(lse[0, 0], s + np.log(np.arange(1, S + 1))))


def test_p2_identical_keys():
    assert check_identical_keys() <= 1e-13


def test_p2_empty_rows_of_a_partial():
    """Queries that see no key of a block get (0, -inf)."""
    q, k, v = _qkv(1, 4, 1, 1, 3, 1)
    o, lse = oa.masked_attention(q, k, v, 1.0, q_pos=[0, 1, 2, 3], k_pos=[10, 11, 12, 13])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# P3: the LSE merge reproduces one-shot attention
# --------------------------------------------------------------------------

def check_merge_identity(S=48, rd=4, H=4, Hkv=2, D=8, cu=None, orders=True):
    """Ring partials of every rank, merged in ring order (and in other orders),
    equal the one-shot rows."""
    q, k, v = _qkv(1, S, H, Hkv, D, 21)
    scale = 0.37
    full_o, full_lse = oa.attention_full(q, k, v, scale, True, cu)
    pos = [ix.zigzag_share_positions(S, rd, r) for r in range(rd)]
    kb = [k[:, p] for p in pos]
    vb = [v[:, p] for p in pos]
    worst = 0.0
    for r in range(rd):
        o, lse, parts = ou.ring_attention_rank(q[:, pos[r]], pos[r], kb, vb, pos, r, scale, True, cu,
                                               return_partials=True)
        worst = max(worst, _err(o, full_o[:, pos[r]]), _err(lse, full_lse[:, :, pos[r]]))
        if orders:
            for perm in itertools.islice(itertools.permutations(range(rd)), 6):
                o2, l2 = om.lse_merge_many([parts[i] for i in perm])
                worst = max(worst, _err(np.transpose(o2, (1, 2, 0, 3)), o), _err(l2, lse))
    return worst


def test_p3_merge_equals_one_shot():
    assert check_merge_identity() <= 1e-12


def test_p3_merge_equals_one_shot_packed():
    assert check_merge_identity(S=64, rd=4, cu=[0, 9, 10, 41, 64]) <= 1e-12


def test_p3_merge_two_single_keys():
    """Two one-key partials merge to the two-key softmax computed directly."""
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal(2) * 3
    v1, v2 = rng.standard_normal((2, 5))
    o, lse = om.lse_merge(v1[None], np.array([a]), v2[None], np.array([b]))
    p1 = 1.0 / (1.0 + math.exp(b - a))
    assert _err(o[0], p1 * v1 + (1 - p1) * v2) <= 1e-15
    assert abs(lse[0] - math.log(math.exp(a) + math.exp(b))) <= 1e-14


def test_p3_empty_partial_is_identity():
    rng = np.random.default_rng(3)
    o1 = rng.standard_normal((6, 4)); l1 = rng.standard_normal(6)
    z = np.zeros((6, 4)); ninf = np.full(6, -np.inf)
    for o, lse in (om.lse_merge(o1, l1, z, ninf), om.lse_merge(z, ninf, o1, l1)):
        assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    o, lse = om.lse_merge(z, ninf, z, ninf)
    assert np.all(o == 0) and np.all(np.isneginf(lse)) and not np.any(np.isnan(o))


def test_p3_merge_large_lse_no_overflow():
    o, lse = om.lse_merge(np.ones((1, 2)), np.array([1000.0]), 2 * np.ones((1, 2)), np.array([1000.0]))
    assert abs(lse[0] - (1000.0 + math.log(2))) <= 1e-12 and _err(o, 1.5 * np.ones((1, 2))) <= 1e-12


# --------------------------------------------------------------------------
# P4: causal loads (golden fixture from the pages)
# --------------------------------------------------------------------------

def check_loads():
    g = golden("causal_loads_cp4.txt")
    cp = 4
    seq = [ix.sequential_rank_units(i, cp) for i in range(cp)]
    assert seq == [float(x) for x in g["sequential_units"]]
    assert max(seq) / (sum(seq) / cp) == float(g["sequential_max_over_mean"][0])
    assert seq[-1] / seq[0] == float(g["sequential_last_over_first"][0])
    assert [ix.chunk_owner(c, cp) for c in range(2 * cp)] == [int(x) for x in g["zigzag_chunk_owner"]]
    chunk_units = [sum(ix._WEIGHT[ix.tile_class(a, b)] for b in range(2 * cp)) for a in range(2 * cp)]
    assert chunk_units == [float(x) for x in g["zigzag_chunk_units"]]
    assert [ix.zigzag_rank_units(r, cp) for r in range(cp)] == [float(x) for x in g["zigzag_rank_units"]]
    return True


def test_p4_loads_match_pages():
    assert check_loads()


@pytest.mark.parametrize("cp", [1, 2, 4, 8, 16])
def test_p4_every_step_costs_two_units(cp):
    for r in range(cp):
        for t in range(cp):
            assert ix.step_units(r, t, cp) == 2.0
    assert sum(ix.zigzag_rank_units(r, cp) for r in range(cp)) == (2 * cp) ** 2 / 2


def test_p4_exact_pair_counts():
    """Token-exact visible pairs per zigzag rank agree with the unit count up to
    the half-diagonal convention: each rank sees 2*cp*c^2 + c pairs exactly."""
    S, cp = 256, 4
    c = S // (2 * cp)
    for r in range(cp):
        p = ix.zigzag_share_positions(S, cp, r)
        assert ix.visible_pairs(p, np.arange(S)) == 2 * cp * c * c + c


# --------------------------------------------------------------------------
# P5: zigzag assignment (Algorithm 2)
# --------------------------------------------------------------------------

def check_zigzag(S=48, rd=3, ud=2):
    c = S // (2 * rd)
    seen = np.concatenate([ix.zigzag_local_positions(S, rd, ud, r, u) for r in range(rd) for u in range(ud)])
    assert np.array_equal(np.sort(seen), np.arange(S))                 # bijection
    for r in range(rd):
        share = np.concatenate([np.arange(r * c, (r + 1) * c),
                                np.arange((2 * rd - 1 - r) * c, (2 * rd - r) * c)])
        assert np.array_equal(ix.zigzag_share_positions(S, rd, r), share)
        parts = [ix.zigzag_local_positions(S, rd, ud, r, u) for u in range(ud)]
        assert np.array_equal(np.concatenate(parts), share)             # the ud parts of the share, in order
        assert all(len(p) == 2 * c // ud for p in parts)
    x = _rand((2, S, 3, 4), 1)
    assert np.array_equal(ix.zigzag_scatter_all(ix.zigzag_extract_all(x, rd, ud), S), x)
    return True


@pytest.mark.parametrize("S,rd,ud", [(48, 3, 2), (64, 4, 1), (256, 4, 2), (32, 1, 4), (96, 2, 3)])
def test_p5_zigzag(S, rd, ud):
    assert check_zigzag(S, rd, ud)


def test_p5_zigzag_cp4_table():
    g = golden("causal_loads_cp4.txt")
    owner = [int(x) for x in g["zigzag_chunk_owner"]]
    S, cp = 64, 4
    c = S // 8
    for r in range(cp):
        chunks = sorted(set(ix.zigzag_share_positions(S, cp, r) // c))
        assert chunks == [i for i, o in enumerate(owner) if o == r]


def test_p5_rejects_uneven():
    with pytest.raises(ValueError):
        ix.zigzag_local_positions(50, 4, 1, 0, 0)


# --------------------------------------------------------------------------
# P6: ring schedule (golden fixture from Figure 1)
# --------------------------------------------------------------------------

def check_schedule():
    g = golden("ring_schedule_cp4.txt")
    for t in range(4):
        row = g[f"step{t + 1}"]
        for gpu in range(4):
            assert row[gpu] == f"Q{gpu}.KV{ix.ring_kv_block(gpu, t, 4)}", (t, gpu)
    return True


def test_p6_schedule():
    assert check_schedule()


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_p6_every_rank_sees_every_block_once(cp):
    for r in range(cp):
        assert sorted(ix.ring_kv_block(r, t, cp) for t in range(cp)) == list(range(cp))
    for t in range(cp):                     # at each step the blocks form a permutation
        assert sorted(ix.ring_kv_block(r, t, cp) for r in range(cp)) == list(range(cp))


# --------------------------------------------------------------------------
# P7: Ulysses layout and the degenerate cases of USP
# --------------------------------------------------------------------------

def check_ulysses(N=4, bs=2, L=24, hc=8, hd=3):
    shards = [_rand((bs, L // N, hc, hd), 30 + u) for u in range(N)]
    heads = [ix.ulysses_fwd(shards, u) for u in range(N)]
    assert all(h.shape == (hc // N, bs, L, hd) for h in heads)
    for u in range(N):
        assert np.array_equal(ix.ulysses_inv(heads, u), shards[u])
    # element map written out: Y_u[h', b, u'*(L/N) + t, :] = X_u'[b, t, u*(hc/N) + h', :]
    u, up, hp, b, t = N - 1, 1, hc // N - 1, bs - 1, 2
    assert np.array_equal(heads[u][hp, b, up * (L // N) + t], shards[up][b, t, u * (hc // N) + hp])
    return True


def test_p7_ulysses_roundtrip():
    assert check_ulysses()


def test_p7_ulysses_n1_is_transpose():
    x = _rand((2, 10, 4, 3), 1)
    assert np.array_equal(ix.ulysses_fwd([x], 0), np.transpose(x, (2, 0, 1, 3)))


def test_p7_gather_reproduces_the_share():
    S, rd, ud = 64, 2, 4
    x = _rand((1, S, 8, 2), 2)
    for r in range(rd):
        shards = [ix.zigzag_extract(x, rd, ud, r, u) for u in range(ud)]
        gathered = np.concatenate([ou.ulysses_to_seq_major(ix.ulysses_fwd(shards, u)) for u in range(ud)],
                                  axis=2)
        assert np.array_equal(gathered, x[:, ix.zigzag_share_positions(S, rd, r)])


def check_degenerate(N, H=4, Hkv=2, S=32, D=4, cu=None):
    """USP with (ud, rd) = (N, 1), (1, N), (2, N/2) all equal one-shot attention."""
    q, k, v = _qkv(1, S, H, Hkv, D, 40)
    scale = 0.5
    o_ref, l_ref = oa.attention_full(q, k, v, scale, True, cu)
    worst = 0.0
    grids = {(N, 1), (1, N)} | ({(2, N // 2)} if N >= 4 else set())
    for ud, rd in grids:
        if H % ud or Hkv % ud:
            continue
        o, lse = ou.usp_attention(q, k, v, rd, ud, scale, True, cu)
        worst = max(worst, _err(o, o_ref), _err(lse, l_ref))
    return worst


@pytest.mark.parametrize("N", [2, 4])
def test_p7_degenerate_cases(N):
    assert check_degenerate(N, H=8, Hkv=4) <= 1e-12


def test_p7_degenerate_gqa_ud2():
    assert check_degenerate(2, H=4, Hkv=2) <= 1e-12


def test_p7_packed_usp():
    assert check_degenerate(4, H=8, Hkv=4, S=64, cu=[0, 7, 30, 31, 64]) <= 1e-12


# --------------------------------------------------------------------------
# P8: communication volume (golden fixture from the worked table)
# --------------------------------------------------------------------------

def check_comm():
    g = golden("comm_volume.txt")
    s, h, cp = int(g["s"][0]), int(g["h"][0]), int(g["cp"][0])
    got = {"ring_mha": comm.mib(comm.ring_elements(s, h, cp)),
           "ulysses_mha": comm.mib(comm.ulysses_elements(s, h, h, cp)),
           "ring_gqa8": comm.mib(comm.ring_elements(s, h // 4, cp)),
           "ulysses_gqa8": comm.mib(comm.ulysses_elements(s, h, h // 4, cp))}
    for key, val in got.items():
        assert val == float(g[key][0]), (key, val)
    return True


def test_p8_comm_volume():
    assert check_comm()


# --------------------------------------------------------------------------
# Mutation checks: a plausible mistake planted in the oracle fails some pin.
# --------------------------------------------------------------------------

def _fails(fn, *args, tol=1e-12):
    try:
        r = fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return r is not True and r > tol


def _strict_visible(q_pos, k_pos, causal, q_seg_start):
    vis = np.ones((len(q_pos), len(k_pos)), dtype=bool)
    if causal:
        vis &= k_pos[None, :] < q_pos[:, None]          # diagonal excluded
    return vis


_orig_merge = om.lse_merge


def _swapped_weight_merge(o1, lse1, o2, lse2):
    """Each partial weighted by the other's factor."""
    o_a, lse = _orig_merge(o1, lse1, np.zeros_like(o2), lse2)
    o_b, _ = _orig_merge(np.zeros_like(o1), lse1, o2, lse2)
    w1 = np.exp(np.asarray(lse1) - lse)[..., None]
    w2 = np.exp(np.asarray(lse2) - lse)[..., None]
    return (o_a / np.where(w1 == 0, 1, w1)) * w2 + (o_b / np.where(w2 == 0, 1, w2)) * w1, lse


MUTANTS = {
    "diagonal_excluded": (oa, "_visible", _strict_visible, [(check_zero_queries,), (check_merge_identity,)]),
    "ring_direction": (ix, "ring_kv_block", lambda r, t, cp: (r + t) % cp, [(check_schedule,)]),
    "diagonal_full_weight": (ix, "_WEIGHT", {ix.FULL: 1.0, ix.DIAGONAL: 1.0, ix.SKIP: 0.0}, [(check_loads,)]),
    "zigzag_wrong_partner": (ix, "zigzag_chunks", lambda r, rd: (r, rd + r), [(check_loads,)]),
    "interleaved_gqa": (oa, "masked_attention", None, [(check_degenerate, 2, 4, 2)]),
    "merge_weights_swapped": (om, "lse_merge", _swapped_weight_merge, [(check_merge_identity,)]),
    "ulysses_reversed_gather": (ix, "ulysses_fwd", None, [(check_ulysses,), (check_degenerate, 2, 4, 2)]),
}


def _interleaved_gqa(q, k, v, scale, q_pos=None, k_pos=None, causal=True, q_seg_start=None, row_block=256):
    """Query head h reads KV head h mod Hkv instead of floor(h / G)."""
    H, Hkv = q.shape[2], k.shape[2]
    idx = np.arange(H) % Hkv
    k2 = np.asarray(k)[:, :, idx]
    v2 = np.asarray(v)[:, :, idx]
    return _orig_masked(q, k2, v2, scale, q_pos, k_pos, causal, q_seg_start, row_block)


_orig_masked = oa.masked_attention
_orig_ulysses_fwd = ix.ulysses_fwd


def _reversed_ulysses_fwd(shards, u):
    return _orig_ulysses_fwd(list(reversed(shards)), u)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    mod, attr, repl, checks = MUTANTS[name]
    if name == "interleaved_gqa":
        repl = _interleaved_gqa
        monkeypatch.setattr(ou, "masked_attention", repl)
    if name == "ulysses_reversed_gather":
        repl = _reversed_ulysses_fwd
    monkeypatch.setattr(mod, attr, repl)
    caught = [_fails(fn, *args) for fn, *args in checks]
    assert any(caught), f"mutant {name} survived every pin"


def test_unmutated_checks_pass():
    assert check_zero_queries() <= 1e-12
    assert check_merge_identity() <= 1e-12
    assert check_schedule() and check_loads() and check_ulysses() and check_comm()
    assert check_degenerate(2, 4, 2) <= 1e-12
