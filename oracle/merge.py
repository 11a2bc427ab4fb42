"""LSE merge of two partial attention results, in float64.

Test infrastructure only (see the package docstring).

[CP vs Ulysses], concepts section (online-softmax merge): each KV block gives
a partial output o_j and log-sum-exp lse_j; two partials combine as
lse = log(e^lse1 + e^lse2) and o = e^(lse1 - lse) o1 + e^(lse2 - lse) o2.

The pages never mention a row with no visible key.  Reading used here: such a
partial is (o = 0, lse = -inf) and is the identity of the merge; two empty
partials merge to (0, -inf).  The log is evaluated in the shifted form
M + log(e^(lse1-M) + e^(lse2-M)), M = max(lse1, lse2), which is the same real
number without overflow.
"""
import numpy as np


def lse_merge(o1, lse1, o2, lse2):
    """Merge partials row by row.

    o1, o2: (..., D); lse1, lse2: (...) with the leading shapes equal.
    Returns (o, lse) as new float64 arrays.
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    l1 = np.asarray(lse1, dtype=np.float64)
    l2 = np.asarray(lse2, dtype=np.float64)
    e1 = np.isneginf(l1)
    e2 = np.isneginf(l2)
    both = e1 & e2
    M = np.where(both, 0.0, np.maximum(l1, l2))
    w1 = np.where(e1, 0.0, np.exp(np.where(e1, 0.0, l1 - M)))
    w2 = np.where(e2, 0.0, np.exp(np.where(e2, 0.0, l2 - M)))
    lse = np.where(both, -np.inf, M + np.log(np.where(both, 1.0, w1 + w2)))
    a1 = np.where(e1, 0.0, np.exp(np.where(e1 | both, 0.0, l1 - np.where(both, 0.0, lse))))
    a2 = np.where(e2, 0.0, np.exp(np.where(e2 | both, 0.0, l2 - np.where(both, 0.0, lse))))
    o = a1[..., None] * o1 + a2[..., None] * o2
    return o, lse


def lse_merge_many(partials):
    """Merge a list of (o, lse) partials left to right (ring order)."""
    o, lse = partials[0]
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    for o_j, lse_j in partials[1:]:
        o, lse = lse_merge(o, lse, o_j, lse_j)
    return o, lse
