"""Pins of the backward oracle against mathematics it does not share code with.

* B1 central finite differences of the forward oracle's loss sum(o * dO);
* B2 torch autograd (float64, CPU) of a plain masked softmax written with
  torch operations -- an independent derivation of the same derivative;
* B3 the ring decomposition: the step contributions of every rank add up to
  the gradients of the whole sequence;
* B4 closed forms and invariants (constant values, zero upstream gradient,
  single visible key, the sum of dK over the keys, the row-term identity).

Each check returns the worst error, so the mutation tests at the bottom can
plant a mistake in the oracle and show that some pin catches it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import backward as ob
from oracle import index as ix
from oracle import usp as ou

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(B, S, H, Hkv, D, seed):
    return (_rand((B, S, H, D), seed), _rand((B, S, Hkv, D), seed + 1), _rand((B, S, Hkv, D), seed + 2),
            _rand((B, S, H, D), seed + 3))


def _maxerr(a, b):
    return max(float(np.max(np.abs(np.asarray(x) - np.asarray(y)))) if np.size(x) else 0.0 for x, y in zip(a, b))


# --------------------------------------------------------------------------
# B1: finite differences of the forward oracle
# --------------------------------------------------------------------------

FD_CASES = [
    # B, S, H, Hkv, D, causal, cu_seqlens
    (1, 5, 2, 1, 3, True, None),
    (1, 6, 2, 2, 2, False, None),
    (2, 4, 4, 2, 2, True, None),
    (1, 7, 2, 1, 2, True, [0, 2, 3, 7]),
]


def check_finite_differences(case, seed=21, h=1e-6):
    B, S, H, Hkv, D, causal, cu = case
    q, k, v, do = _case(B, S, H, Hkv, D, seed)
    scale = 0.7

    def loss(q_, k_, v_):
        o, _ = oa.attention_full(q_, k_, v_, scale, causal, cu)
        return float((o * do).sum())

    grads = ob.attention_backward_full(q, k, v, do, scale, causal, cu)
    worst = 0.0
    for which, g in enumerate(grads):
        args = [q, k, v]
        x = args[which]
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            worst = max(worst, abs(fd - g[idx]))
    return worst


@pytest.mark.parametrize("case", FD_CASES)
def test_b1_finite_differences(case):
    assert check_finite_differences(case) < 1e-7


# --------------------------------------------------------------------------
# B2: torch autograd of a plain masked softmax
# --------------------------------------------------------------------------

def _torch_grads(q, k, v, do, scale, causal, cu):
    B, S, H, D = q.shape
    G = H // k.shape[2]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(G, dim=2)
    vv = tv.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kk) * scale
    pos = torch.arange(S)
    mask = torch.ones(S, S, dtype=torch.bool)
    if causal:
        mask &= pos[None, :] <= pos[:, None]
    if cu is not None:
        seg = torch.bucketize(pos, torch.tensor(cu[1:]), right=True)
        mask &= seg[None, :] == seg[:, None]
    s = s.masked_fill(~mask, -math.inf)
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


AUTOGRAD_CASES = [
    (2, 40, 4, 2, 8, True, None),
    (1, 33, 6, 1, 16, True, None),
    (1, 24, 2, 2, 8, False, None),
    (1, 50, 4, 2, 8, True, [0, 13, 14, 40, 50]),
]


def check_autograd(case, seed=31):
    B, S, H, Hkv, D, causal, cu = case
    q, k, v, do = _case(B, S, H, Hkv, D, seed)
    scale = 1.0 / math.sqrt(D)
    return _maxerr(ob.attention_backward_full(q, k, v, do, scale, causal, cu),
                   _torch_grads(q, k, v, do, scale, causal, cu))


@pytest.mark.parametrize("case", AUTOGRAD_CASES)
def test_b2_autograd(case):
    assert check_autograd(case) < 1e-10


# --------------------------------------------------------------------------
# B3: the ring decomposition adds up to the whole-sequence gradients
# --------------------------------------------------------------------------

def check_ring_decomposition(B, S, H, Hkv, D, rd, cu=None, seed=41):
    q, k, v, do = _case(B, S, H, Hkv, D, seed)
    scale = 1.0 / math.sqrt(D)
    o, lse = oa.attention_full(q, k, v, scale, True, cu)
    delta = ob.delta_rows(o, do)
    pos = [ix.zigzag_share_positions(S, rd, r) for r in range(rd)]
    kb = [k[:, p] for p in pos]
    vb = [v[:, p] for p in pos]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(rd):
        gq, gk, gv = ob.ring_backward_rank(q[:, pos[r]], pos[r], kb, vb, pos, do[:, pos[r]],
                                           lse[:, :, pos[r]], delta[:, :, pos[r]], r, scale, True, cu)
        dq[:, pos[r]] = gq
        for j in range(rd):
            dk[:, pos[j]] += gk[j]
            dv[:, pos[j]] += gv[j]
    return _maxerr((dq, dk, dv), ob.attention_backward_full(q, k, v, do, scale, True, cu))


@pytest.mark.parametrize("B,S,H,Hkv,D,rd,cu", [
    (1, 48, 4, 2, 8, 4, None),
    (2, 36, 2, 1, 4, 3, None),
    (1, 64, 2, 2, 4, 2, [0, 5, 6, 30, 64]),
    (1, 16, 2, 1, 4, 1, None),
])
def test_b3_ring_decomposition(B, S, H, Hkv, D, rd, cu):
    assert check_ring_decomposition(B, S, H, Hkv, D, rd, cu) < 1e-11


def test_b3_usp_lse_feeds_ring_backward():
    """The lse that the forward oracle's ring produces (merged per rank) is
    the one the backward steps take: rebuilding P from it gives rows that sum
    to one over the cp blocks."""
    B, S, H, Hkv, D, rd = 1, 32, 2, 1, 4, 4
    q, k, v, _ = _case(B, S, H, Hkv, D, 51)
    scale = 0.5
    pos = [ix.zigzag_share_positions(S, rd, r) for r in range(rd)]
    for r in range(rd):
        _, lse = ou.ring_attention_rank(q[:, pos[r]], pos[r], [k[:, p] for p in pos], [v[:, p] for p in pos],
                                        pos, r, scale)
        total = np.zeros((H, B, len(pos[r])))
        for j in range(rd):
            s = np.einsum("bihd,bjhd->hbij", q[:, pos[r]], np.repeat(k[:, pos[j]], H // Hkv, axis=2)) * scale
            vis = pos[j][None, :] <= pos[r][:, None]
            total += np.where(vis, np.exp(s - lse[..., None]), 0.0).sum(-1)
        assert np.max(np.abs(total - 1.0)) < 1e-12


# --------------------------------------------------------------------------
# B4: closed forms and invariants
# --------------------------------------------------------------------------

def check_constant_values(seed=61):
    """Equal value rows make o independent of q and k: dq = dk = 0, and dV of a
    key is the P-weighted sum of the upstream rows."""
    B, S, H, Hkv, D = 1, 20, 2, 1, 4
    q, k, _, do = _case(B, S, H, Hkv, D, seed)
    v = np.broadcast_to(_rand((1, 1, Hkv, D), seed + 9), (B, S, Hkv, D)).copy()
    dq, dk, dv = ob.attention_backward_full(q, k, v, do, 0.9)
    # sum over keys of dV equals the sum over rows and heads of dO (P rows sum to 1)
    tot = do.reshape(B, S, Hkv, H // Hkv, D).sum(axis=(1, 3))
    return max(float(np.abs(dq).max()), float(np.abs(dk).max()), float(np.abs(dv.sum(axis=1) - tot).max()))


def test_b4_constant_values():
    assert check_constant_values() < 1e-12


def test_b4_zero_upstream():
    q, k, v, _ = _case(1, 12, 2, 1, 4, 71)
    for g in ob.attention_backward_full(q, k, v, np.zeros_like(q), 0.5):
        assert np.all(g == 0)


def check_single_key_row(seed=81):
    """Row 0 of a causal sequence sees only key 0: P = 1, so its dq is zero and
    its share of dV[0] is dO[0]."""
    q, k, v, do = _case(1, 9, 2, 2, 3, seed)
    dq, _, dv = ob.attention_backward_full(q, k, v, do, 0.8)
    q1 = q.copy()
    q1[:, 1:] = 0.0
    do1 = do.copy()
    do1[:, 1:] = 0.0                      # only row 0 sends gradient
    _, _, dv1 = ob.attention_backward_full(q1, k, v, do1, 0.8)
    return max(float(np.abs(dq[:, 0]).max()), float(np.abs(dv1[:, 0] - do[:, 0]).max()),
               float(np.abs(dv1[:, 1:]).max()))


def test_b4_single_key_row():
    assert check_single_key_row() < 1e-12


def check_dk_sums_to_zero(seed=91):
    """Adding a constant to every logit of a row leaves the softmax unchanged,
    so each row of dS sums to zero and dK summed over the keys vanishes."""
    B, S, H, Hkv, D = 2, 30, 4, 2, 5
    q, k, v, do = _case(B, S, H, Hkv, D, seed)
    _, dk, _ = ob.attention_backward_full(q, k, v, do, 0.6, True, [0, 11, 30])
    return float(np.abs(dk.sum(axis=1)).max())


def test_b4_dk_sums_to_zero():
    assert check_dk_sums_to_zero() < 1e-11


def test_b4_row_term_identity():
    """rowsum(P * dP) from the probabilities equals rowsum(dO * o)."""
    q, k, v, do = _case(1, 25, 2, 1, 6, 95)
    scale = 0.4
    o, _ = oa.attention_full(q, k, v, scale)
    d1 = ob.delta_rows(o, do)
    s = np.einsum("bihd,bjhd->hbij", q, np.repeat(k, 2, axis=2)) * scale
    s = np.where(np.tril(np.ones((25, 25), bool)), s, -np.inf)
    P = np.exp(s - s.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    dP = np.einsum("bihd,bjhd->hbij", do, np.repeat(v, 2, axis=2))
    assert np.max(np.abs((P * dP).sum(-1) - d1)) < 1e-12


# --------------------------------------------------------------------------
# Mutation tests: a planted mistake must fail some pin
# --------------------------------------------------------------------------

_orig_head_grads = ob._head_grads
_orig_step = ob.ring_step_backward


def _no_row_term(P, q_h, k_h, v_h, do_h, row_term, scale):
    return _orig_head_grads(P, q_h, k_h, v_h, do_h, np.zeros_like(row_term), scale)


def _unscaled_dk(P, q_h, k_h, v_h, do_h, row_term, scale):
    gq, gk, gv = _orig_head_grads(P, q_h, k_h, v_h, do_h, row_term, scale)
    return gq, gk / scale, gv


def _dv_from_dp(P, q_h, k_h, v_h, do_h, row_term, scale):
    gq, gk, _ = _orig_head_grads(P, q_h, k_h, v_h, do_h, row_term, scale)
    dS = P * (do_h @ v_h.T - row_term[:, None])
    return gq, gk, dS.T @ do_h


def _row_term_sign(P, q_h, k_h, v_h, do_h, row_term, scale):
    return _orig_head_grads(P, q_h, k_h, v_h, do_h, -row_term, scale)


def _step_local_lse(q, k_blk, v_blk, do, lse, delta, scale, q_pos, k_pos, causal=True, q_seg_start=None):
    """Each step normalises by its own block's lse instead of the global one."""
    _, lse_j = oa.masked_attention(q, k_blk, v_blk, scale, q_pos, k_pos, causal, q_seg_start)
    return _orig_step(q, k_blk, v_blk, do, lse_j, delta, scale, q_pos, k_pos, causal, q_seg_start)


def _step_wrong_block(q, k_blk, v_blk, do, lse, delta, scale, q_pos, k_pos, causal=True, q_seg_start=None):
    """Keys evaluated at the query positions (positions of the wrong block)."""
    return _orig_step(q, k_blk, v_blk, do, lse, delta, scale, q_pos, q_pos, causal, q_seg_start)


FD0, AG0 = FD_CASES[0], AUTOGRAD_CASES[0]
MUTANTS = {
    "no_row_term": ("_head_grads", _no_row_term, [(check_finite_differences, FD0), (check_autograd, AG0)]),
    "row_term_sign": ("_head_grads", _row_term_sign, [(check_finite_differences, FD0), (check_dk_sums_to_zero,)]),
    "unscaled_dk": ("_head_grads", _unscaled_dk, [(check_autograd, AG0)]),
    "dv_from_dS": ("_head_grads", _dv_from_dp, [(check_constant_values,), (check_single_key_row,)]),
    "step_local_lse": ("ring_step_backward", _step_local_lse, [(check_ring_decomposition, 1, 48, 4, 2, 8, 4)]),
    "step_wrong_positions": ("ring_step_backward", _step_wrong_block,
                             [(check_ring_decomposition, 1, 48, 4, 2, 8, 4)]),
}


def _fails(fn, *args, tol=1e-7):
    try:
        r = fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return r > tol


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutants_are_caught(name, monkeypatch):
    attr, repl, checks = MUTANTS[name]
    monkeypatch.setattr(ob, attr, repl)
    assert any(_fails(fn, *args) for fn, *args in checks), f"mutant {name} survived every pin"


def test_backward_unmutated_checks_pass():
    assert check_finite_differences(FD0) < 1e-7 and check_autograd(AG0) < 1e-10
    assert check_constant_values() < 1e-12 and check_single_key_row() < 1e-12
    assert check_dk_sums_to_zero() < 1e-11
    assert check_ring_decomposition(1, 48, 4, 2, 8, 4) < 1e-11
