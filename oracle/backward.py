"""Gradients of the attention forward (the backward pass), in float64.

Test infrastructure only (see the package docstring).

The pages use the method for training: [YunChang] runs its tests with a
backward flag and [USP review] section 六 reports end-to-end training.  The
backward computes the derivative of the forward definition (``attention``).
For one query head, with logits s = scale * q k^T on the visible pairs,
P = softmax over each row, o = P v and an upstream gradient dO:

    dV   = P^T dO
    dP   = dO v^T
    dS   = P * (dP - rowsum(P * dP))          (Jacobian of a row softmax)
    dQ   = scale * dS k
    dK   = scale * dS^T q

A KV head's dK and dV sum the contributions of the G query heads that read
it.  Since o = P v, the row term rowsum(P * dP) equals rowsum(dO * o).

Ring form ([CP vs Ulysses], concepts section: each step attends the rank's
queries to one KV block).  Given the final lse of the forward, P restricted
to block j is exp(s - lse) on that block's visible keys, so every step's
gradient contribution can be computed on its own and the contributions add up
to the gradients of the whole sequence.  A rank's dQ is the sum over its cp
steps; block j's dK and dV are the sums over all ranks of their step against
block j.
"""
import numpy as np

from . import index as ix
from .attention import _visible


def _head_grads(P, q_h, k_h, v_h, do_h, row_term, scale):
    """Gradient contributions of one query head for given probabilities.

    P: (rows, keys) softmax probabilities, zero on hidden pairs; row_term:
    (rows,) the softmax Jacobian's row term rowsum(P * dP).
    Returns dq (rows, D), dk (keys, D), dv (keys, D).
    """
    dP = do_h @ v_h.T
    dS = P * (dP - row_term[:, None])
    return scale * (dS @ k_h), scale * (dS.T @ q_h), P.T @ do_h


def attention_backward(q, k, v, do, scale, q_pos=None, k_pos=None, causal=True, q_seg_start=None,
                       row_block=256):
    """dq, dk, dv of the masked attention of ``attention.masked_attention``.

    q, do: (B, Sq, H, D); k, v: (B, Sk, Hkv, D).  The softmax is recomputed
    from the logits (no saved statistics) and the row term is taken as
    rowsum(P * dP).  Rows with no visible key contribute nothing.
    Returns dq (B, Sq, H, D), dk and dv (B, Sk, Hkv, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Sq, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    q_pos = np.arange(Sq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(k.shape[1], dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    if q_seg_start is not None:
        q_seg_start = np.asarray(q_seg_start, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        vis = _visible(q_pos[r0:r1], k_pos, causal, None if q_seg_start is None else q_seg_start[r0:r1])
        keys = np.nonzero(vis.any(axis=0))[0]
        if len(keys) == 0:
            continue
        vis = vis[:, keys]
        has_key = vis.any(axis=1)
        for b in range(B):
            for h in range(H):
                g = h // G
                k_h, v_h = k[b, keys, g, :], v[b, keys, g, :]
                q_h, do_h = q[b, r0:r1, h, :], do[b, r0:r1, h, :]
                s = np.where(vis, scale * (q_h @ k_h.T), -np.inf)
                m = np.where(has_key, s.max(axis=1), 0.0)
                e = np.where(vis, np.exp(s - m[:, None]), 0.0)
                P = e / np.where(has_key, e.sum(axis=1), 1.0)[:, None]
                row_term = (P * (do_h @ v_h.T)).sum(axis=1)
                gq, gk, gv = _head_grads(P, q_h, k_h, v_h, do_h, row_term, scale)
                dq[b, r0:r1, h, :] += gq
                dk[b, keys, g, :] += gk
                dv[b, keys, g, :] += gv
    return dq, dk, dv


def attention_backward_full(q, k, v, do, scale, causal=True, cu_seqlens=None):
    """Backward of one-shot attention over the whole sequence (global order)."""
    S = q.shape[1]
    pos = np.arange(S, dtype=np.int64)
    seg = None if cu_seqlens is None else ix.segment_start(cu_seqlens, pos)
    return attention_backward(q, k, v, do, scale, pos, pos, causal, seg)


def delta_rows(o, do):
    """The row term from the output: rowsum(dO * o) per (head, batch, row),
    shaped (H, B, Sq) like lse; o and dO are (B, Sq, H, D)."""
    d = (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-1)
    return np.ascontiguousarray(np.transpose(d, (2, 0, 1)))


def ring_step_backward(q, k_blk, v_blk, do, lse, delta, scale, q_pos, k_pos, causal=True, q_seg_start=None):
    """One ring step's gradient contributions against one KV block.

    q, do: (B, Sq, H, D); k_blk, v_blk: (B, Sk, Hkv, D); lse and delta:
    (H, B, Sq) of the whole forward (lse over all blocks, delta =
    rowsum(dO * o)).  P on this block is exp(scale q k^T - lse) on the visible
    pairs, zero elsewhere and on rows whose lse is -inf.
    Returns dq (B, Sq, H, D), dk and dv (B, Sk, Hkv, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    B, Sq, H, D = q.shape
    Hkv = k_blk.shape[2]
    G = H // Hkv
    vis = _visible(np.asarray(q_pos, dtype=np.int64), np.asarray(k_pos, dtype=np.int64), causal,
                   None if q_seg_start is None else np.asarray(q_seg_start, dtype=np.int64))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_blk)
    dv = np.zeros_like(v_blk)
    for b in range(B):
        for h in range(H):
            g = h // G
            k_h, v_h = k_blk[b, :, g, :], v_blk[b, :, g, :]
            row_lse = lse[h, b]
            live = vis & np.isfinite(row_lse)[:, None]
            s = scale * (q[b, :, h, :] @ k_h.T)
            P = np.where(live, np.exp(np.where(live, s - np.where(np.isfinite(row_lse), row_lse, 0.0)[:, None], 0.0)), 0.0)
            gq, gk, gv = _head_grads(P, q[b, :, h, :], k_h, v_h, do[b, :, h, :], delta[h, b], scale)
            dq[b, :, h, :] += gq
            dk[b, :, g, :] += gk
            dv[b, :, g, :] += gv
    return dq, dk, dv


def ring_backward_rank(q_local, q_pos, k_blocks, v_blocks, k_pos_blocks, do_local, lse, delta, ring_rank,
                       scale, causal=True, cu_seqlens=None):
    """The backward as seen by one ring rank: its queries against the cp
    blocks in ring order (step t holds block (r - t) mod cp).

    lse, delta: (H, B, L) of this rank's rows from the whole forward.
    Returns dq (B, L, H, D) and the rank's contributions to every block's
    gradients, dk[j] and dv[j] (B, L, Hkv, D) indexed by block.
    """
    cp = len(k_blocks)
    seg = None if cu_seqlens is None else ix.segment_start(cu_seqlens, q_pos)
    dq = np.zeros(np.shape(q_local), dtype=np.float64)
    dk = [None] * cp
    dv = [None] * cp
    for t in range(cp):
        j = ix.ring_kv_block(ring_rank, t, cp)
        gq, dk[j], dv[j] = ring_step_backward(q_local, k_blocks[j], v_blocks[j], do_local, lse, delta,
                                              scale, q_pos, k_pos_blocks[j], causal, seg)
        dq += gq
    return dq, dk, dv
