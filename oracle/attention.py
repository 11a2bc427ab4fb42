"""Masked softmax attention by its definition, in float64.

Test infrastructure only (see the package docstring).

The method reaches exactly the result of attending to the whole sequence at
once ([CP vs Ulysses], concepts section, online-softmax merge: the merged
result equals one pass over the full sequence).  So the oracle is that plain
definition, softmax(scale * Q K^T) V with the causal mask, written out per
query row, plus the log-sum-exp of the scaled logits.

Conventions (readings listed with the design notes):

* Query head h reads KV head floor(h / G), G = H / Hkv: contiguous groups, the
  only mapping under which Ulysses can split query and KV heads in contiguous
  blocks ([USP review] section 三, AllToAll4D).
* A key is visible from a query iff its global position is <= the query's
  (the token itself included) and, for packed samples, both lie in the same
  sample.
* lse is the natural-log log-sum-exp of the scaled logits over the visible
  keys; a row with no visible key has o = 0 and lse = -inf.
"""
import math

import numpy as np


def _visible(q_pos, k_pos, causal, q_seg_start):
    """Boolean (Sq, Sk) visibility matrix from global positions."""
    vis = np.ones((len(q_pos), len(k_pos)), dtype=bool)
    if causal:
        vis &= k_pos[None, :] <= q_pos[:, None]
    if q_seg_start is not None:
        # same sample  <=>  key at or after the query's sample start (the key is
        # never past the query's sample end when it is also at or before it).
        vis &= k_pos[None, :] >= q_seg_start[:, None]
        if not causal:
            raise ValueError("packed samples are defined here with the causal mask only")
    return vis


def masked_attention(q, k, v, scale, q_pos=None, k_pos=None, causal=True, q_seg_start=None,
                     row_block=256):
    """Softmax attention of queries ``q`` against keys/values ``k``, ``v``.

    q: (B, Sq, H, D); k, v: (B, Sk, Hkv, D), any float dtype (computed in
    float64).  ``q_pos`` / ``k_pos``: global positions of the rows (default
    0..S-1).  ``q_seg_start``: for packed samples, the first global position
    of each query's sample.

    Returns o: (B, Sq, H, D) float64 and lse: (H, B, Sq) float64.  Rows with no
    visible key give o = 0, lse = -inf (so the function also serves as one ring
    step's partial result).

    Rows are processed ``row_block`` at a time to bound memory; inside a block
    the logits are one matrix product and the softmax is exact per row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if H % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hkv
    q_pos = np.arange(Sq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(Sk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    if q_seg_start is not None:
        q_seg_start = np.asarray(q_seg_start, dtype=np.int64)

    o = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.full((H, B, Sq), -np.inf, dtype=np.float64)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        vis = _visible(q_pos[r0:r1], k_pos, causal,
                       None if q_seg_start is None else q_seg_start[r0:r1])
        keys = np.nonzero(vis.any(axis=0))[0]          # drop keys no row here can see
        if len(keys) == 0:
            continue
        vis = vis[:, keys]
        has_key = vis.any(axis=1)
        for b in range(B):
            for h in range(H):
                g = h // G
                s = scale * (q[b, r0:r1, h, :] @ k[b, keys, g, :].T)      # (rows, keys)
                s = np.where(vis, s, -np.inf)
                m = np.where(has_key, s.max(axis=1), 0.0)
                e = np.where(vis, np.exp(s - m[:, None]), 0.0)
                den = e.sum(axis=1)
                row_lse = np.where(has_key, m + np.log(np.where(has_key, den, 1.0)), -np.inf)
                p = e / np.where(has_key, den, 1.0)[:, None]
                o[b, r0:r1, h, :] = p @ v[b, keys, g, :]
                lse[h, b, r0:r1] = row_lse
    return o, lse


def attention_full(q, k, v, scale, causal=True, cu_seqlens=None):
    """One-shot attention of the whole sequence (global token order).

    ``cu_seqlens``: optional packed-sample boundaries (n+1 ints, from 0 to S).
    """
    S = q.shape[1]
    pos = np.arange(S, dtype=np.int64)
    seg = None
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seg = cu[np.searchsorted(cu, pos, side="right") - 1]
    return masked_attention(q, k, v, scale, pos, pos, causal, seg)


def attention_bruteforce(q, k, v, scale, causal=True, cu_seqlens=None):
    """Scalar triple loop over (row, head, key) with ``math.exp``; tiny shapes
    only.  Same conventions and outputs as :func:`attention_full`."""
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    seg = [0] * S
    if cu_seqlens is not None:
        for n in range(len(cu_seqlens) - 1):
            for i in range(int(cu_seqlens[n]), int(cu_seqlens[n + 1])):
                seg[i] = n
    o = np.zeros((B, S, H, D))
    lse = np.full((H, B, S), -math.inf)
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(S):
                logits = []
                for j in range(S):
                    if causal and j > i:
                        continue
                    if seg[j] != seg[i]:
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b, i, h, d]) * float(k[b, j, g, d])
                    logits.append((j, scale * dot))
                if not logits:
                    continue
                mx = max(x for _, x in logits)
                total = sum(math.exp(x - mx) for _, x in logits)
                lse[h, b, i] = mx + math.log(total)
                for j, x in logits:
                    w = math.exp(x - lse[h, b, i])
                    for d in range(D):
                        o[b, i, h, d] += w * float(v[b, j, g, d])
    return o, lse
