"""USP-Attention composed over a virtual (ud x rd) grid, in float64.

Test infrastructure only (see the package docstring).

[USP review] section 三: Algorithm 2 gives every (ring rank r, Ulysses rank u)
its local tokens; Algorithm 1 then runs AllToAll4D on Q, K and V over the
Ulysses group, LoadBalance-RingAttention over the ring group, and the inverse
AllToAll4D on O.  [CP vs Ulysses] (concepts section) defines the ring: each
rank keeps its queries, the KV blocks travel one rank per step, each step
yields (o_j, lse_j), and the partials are merged with the LSE rule.

Here every rank is a loop index; nothing is shared between ranks except what
the steps above pass.
"""
import numpy as np

from . import index as ix
from .attention import masked_attention
from .merge import lse_merge_many


def _seg_start(cu_seqlens, pos):
    return None if cu_seqlens is None else ix.segment_start(cu_seqlens, pos)


def ring_attention_rank(q_local, q_pos, k_blocks, v_blocks, k_pos_blocks, ring_rank, scale,
                        causal=True, cu_seqlens=None, return_partials=False):
    """LoadBalance-RingAttention as seen by one ring rank.

    q_local: (B, L, H, D) with global positions ``q_pos``; ``k_blocks`` /
    ``v_blocks``: the cp KV blocks (B, L, Hkv, D) indexed by the rank that
    holds them at step 0, with positions ``k_pos_blocks``.  At step t the rank
    computes against block (r - t) mod cp; partials are merged in that order.

    Returns (o (B, L, H, D), lse (H, B, L)) and, if asked, the list of step
    partials in ring order, each as (o_j (H, B, L, D), lse_j (H, B, L)): rows
    are merged head-major so that o_j and lse_j share their leading indices.
    """
    cp = len(k_blocks)
    seg = _seg_start(cu_seqlens, q_pos)
    partials = []
    for t in range(cp):
        j = ix.ring_kv_block(ring_rank, t, cp)
        o_j, lse_j = masked_attention(q_local, k_blocks[j], v_blocks[j], scale,
                                      q_pos, k_pos_blocks[j], causal, seg)
        partials.append((np.transpose(o_j, (2, 0, 1, 3)), lse_j))
    o, lse = lse_merge_many(partials)
    o = np.ascontiguousarray(np.transpose(o, (1, 2, 0, 3)))
    return (o, lse, partials) if return_partials else (o, lse)


def usp_attention(Q, K, V, rd, ud, scale, causal=True, cu_seqlens=None, per_sample=False):
    """Algorithm 1 with Algorithm 2's split, on all rd*ud virtual ranks.

    Q: (B, S, H, D); K, V: (B, S, Hkv, D) in global token order.  Returns
    o: (B, S, H, D) in global order and lse: (H, B, S).  ``per_sample``
    applies the split to every packed sample of ``cu_seqlens`` on its own
    (:func:`index.zigzag_per_sample_positions`) instead of to the whole
    packed stream.
    """
    B, S, H, D = Q.shape
    Hkv = K.shape[2]
    if H % ud or Hkv % ud:
        raise ValueError("head counts must divide by the Ulysses degree")

    # Algorithm 2: every rank's local tokens.
    if per_sample:
        if cu_seqlens is None:
            raise ValueError("the per-sample split needs cu_seqlens")
        local = lambda r, u: ix.zigzag_per_sample_local_positions(cu_seqlens, rd, ud, r, u)
    else:
        local = lambda r, u: ix.zigzag_local_positions(S, rd, ud, r, u)

    def shards(X):
        return [[X[:, local(r, u)].copy() for u in range(ud)] for r in range(rd)]
    Qs, Ks, Vs = shards(Q), shards(K), shards(V)

    # Algorithm 1 steps 1-3: AllToAll4D over each Ulysses group (fixed r).
    def a2a(Xs):
        return [[ulysses_to_seq_major(ix.ulysses_fwd(Xs[r], u)) for u in range(ud)]
                for r in range(rd)]
    Qh, Kh, Vh = a2a(Qs), a2a(Ks), a2a(Vs)

    # Positions after the gather: peer shards concatenated in Ulysses order.
    share_pos = [np.concatenate([local(r, u) for u in range(ud)]) for r in range(rd)]

    # Algorithm 1 step 4: the ring, per (r, u).
    Oh = [[None] * ud for _ in range(rd)]
    lse = np.full((H, B, S), -np.inf)
    hb = H // ud
    for r in range(rd):
        for u in range(ud):
            o_ru, lse_ru = ring_attention_rank(
                Qh[r][u], share_pos[r], [Kh[j][u] for j in range(rd)],
                [Vh[j][u] for j in range(rd)], share_pos, r, scale, causal, cu_seqlens)
            Oh[r][u] = np.ascontiguousarray(np.transpose(o_ru, (2, 0, 1, 3)))   # head-major
            lse[u * hb:(u + 1) * hb][:, :, share_pos[r]] = lse_ru

    # Algorithm 1 step 5: inverse AllToAll4D, then back to global order.
    O = np.zeros((B, S, H, D))
    for r in range(rd):
        for u in range(ud):
            O[:, local(r, u)] = ix.ulysses_inv(Oh[r], u)
    return O, lse


def kv_head_chunk(h0, nh, G):
    """KV heads serving query heads [h0, h0 + nh) of a head block: query head h
    reads KV head h // G, so a chunk of whole GQA groups has KV heads
    [h0 / G, (h0 + nh) / G), and a chunk inside one group (nh dividing G)
    has that group's single KV head."""
    return h0 // G, max(nh // G, 1)


def usp_attention_head_chunks(Q, K, V, rd, ud, scale, head_chunk, causal=True, cu_seqlens=None,
                              per_sample=False):
    """Algorithm 1 with each Ulysses head block pushed through the forward
    all-to-all, the ring and the inverse all-to-all ``head_chunk`` query heads
    at a time ([UPipe page] section 2, headwise chunking).

    For chunk [h0, h0 + nh) of every head block the all-to-all moves those
    query heads and their KV heads (:func:`kv_head_chunk`), the ring runs on
    them alone, and the inverse all-to-all puts their outputs back; only one
    chunk's head-major tensors exist at a time.  nh must divide the block's
    hc / ud query heads and be a multiple or a divisor of the GQA group G.
    Same arguments and results as :func:`usp_attention`.
    """
    B, S, H, D = Q.shape
    Hkv = K.shape[2]
    if H % ud or Hkv % ud or H % Hkv:
        raise ValueError("head counts must divide by the Ulysses degree")
    hb, G, nh = H // ud, H // Hkv, head_chunk
    if nh < 1 or hb % nh or (nh % G and G % nh):
        raise ValueError("the chunk must divide the head block and hold whole GQA groups or lie in one")
    if per_sample:
        if cu_seqlens is None:
            raise ValueError("the per-sample split needs cu_seqlens")
        local = lambda r, u: ix.zigzag_per_sample_local_positions(cu_seqlens, rd, ud, r, u)
    else:
        local = lambda r, u: ix.zigzag_local_positions(S, rd, ud, r, u)
    Qs = [[Q[:, local(r, u)].copy() for u in range(ud)] for r in range(rd)]
    Ks = [[K[:, local(r, u)].copy() for u in range(ud)] for r in range(rd)]
    Vs = [[V[:, local(r, u)].copy() for u in range(ud)] for r in range(rd)]
    share_pos = [np.concatenate([local(r, u) for u in range(ud)]) for r in range(rd)]
    out = [[np.zeros((B, S // (rd * ud), H, D)) for u in range(ud)] for r in range(rd)]
    lse = np.full((H, B, S), -np.inf)
    for h0 in range(0, hb, nh):
        k0, nk = kv_head_chunk(h0, nh, G)
        # forward all-to-all of the chunk, over each Ulysses group
        Qh = [[ulysses_to_seq_major(ix.ulysses_fwd_heads(Qs[r], u, h0, nh)) for u in range(ud)] for r in range(rd)]
        Kh = [[ulysses_to_seq_major(ix.ulysses_fwd_heads(Ks[r], u, k0, nk)) for u in range(ud)] for r in range(rd)]
        Vh = [[ulysses_to_seq_major(ix.ulysses_fwd_heads(Vs[r], u, k0, nk)) for u in range(ud)] for r in range(rd)]
        # the ring on the chunk's heads
        Oh = [[None] * ud for _ in range(rd)]
        for r in range(rd):
            for u in range(ud):
                o_ru, lse_ru = ring_attention_rank(
                    Qh[r][u], share_pos[r], [Kh[j][u] for j in range(rd)], [Vh[j][u] for j in range(rd)],
                    share_pos, r, scale, causal, cu_seqlens)
                Oh[r][u] = np.ascontiguousarray(np.transpose(o_ru, (2, 0, 1, 3)))
                lse[u * hb + h0:u * hb + h0 + nh][:, :, share_pos[r]] = lse_ru
        # inverse all-to-all of the chunk's outputs
        for r in range(rd):
            for u in range(ud):
                ix.ulysses_inv_heads(Oh[r], u, h0, H, out[r][u])
    O = np.zeros((B, S, H, D))
    for r in range(rd):
        for u in range(ud):
            O[:, local(r, u)] = out[r][u]
    return O, lse


def ulysses_to_seq_major(x):
    """(hc/N, bs, L, hd) -> (bs, L, hc/N, hd): a view change for the attention
    routine, which takes the [batch, seq, head, dim] layout."""
    return np.ascontiguousarray(np.transpose(x, (1, 2, 0, 3)))
