"""Index oracle: zigzag split, Ulysses layout, ring schedule, tile classes.

Test infrastructure only (see the package docstring).  Integer and copy work:
results here are exact, so GPU parity against them is bit-exact.

Notation: S global sequence length, rd (= cp) ring degree, ud Ulysses degree,
c = S / (2 rd) the zigzag chunk length.  Arrays use the user-facing layout
[batch, seq_len, num_heads, head_dim] of [YunChang] (quickstart section).
"""
import numpy as np


# --------------------------------------------------------------------------
# Algorithm 2 ([USP review] section 三, "Algorithm 2: 负载均衡序列分段")
# --------------------------------------------------------------------------

def zigzag_local_positions(S, rd, ud, ring_rank, ulysses_rank):
    """Global token positions held by ring rank ``ring_rank`` / Ulysses rank
    ``ulysses_rank``, in local order.

    The split of Algorithm 2 written as a position formula: with chunk length
    c = S / (2 rd), local row i of ring rank r's share is the token at
    r c + i for i < c and at (2 rd - 1 - r) c + (i - c) for c <= i < 2c; the
    Ulysses rank u keeps rows u T .. (u + 1) T - 1 of that share, T = 2c / ud.
    Lengths that do not divide are rejected (no page says how to pad).
    """
    if S % (2 * rd) != 0 or (S // rd) % ud != 0:
        raise ValueError(f"S = {S} does not split into 2*{rd} chunks and {ud} equal parts of a share")
    c = S // (2 * rd)
    rows_per_rank = 2 * c // ud
    i = np.arange(ulysses_rank * rows_per_rank, (ulysses_rank + 1) * rows_per_rank, dtype=np.int64)
    return np.where(i < c, ring_rank * c + i, (2 * rd - 1 - ring_rank) * c + (i - c))


def zigzag_share_positions(S, rd, ring_rank):
    """Positions of a ring rank's whole share (Algorithm 2 with ud = 1)."""
    return zigzag_local_positions(S, rd, 1, ring_rank, 0)


def zigzag_per_sample_positions(cu_seqlens, rd, ring_rank):
    """Positions held by ring rank r when Algorithm 2's split is applied to
    every packed sample on its own ([USP review] section 三, Algorithm 2, with
    the packing of [ByteScale notes]): a sample starting at b with length n
    (a multiple of 2 rd) has chunks of m = n / (2 rd) tokens, and the rank
    holds b + r m .. b + (r + 1) m - 1 followed by
    b + (2 rd - 1 - r) m .. b + (2 rd - r) m - 1; the share is these runs in
    sample order.  With one sample this is :func:`zigzag_share_positions`."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    runs = []
    for b, e in zip(cu[:-1], cu[1:]):
        if (e - b) % (2 * rd) != 0:
            raise ValueError(f"sample of length {e - b} does not split into 2*{rd} chunks")
        m = (e - b) // (2 * rd)
        runs.append(b + ring_rank * m + np.arange(m, dtype=np.int64))
        runs.append(b + (2 * rd - 1 - ring_rank) * m + np.arange(m, dtype=np.int64))
    return np.concatenate(runs)


def zigzag_per_sample_local_positions(cu_seqlens, rd, ud, ring_rank, ulysses_rank):
    """Per-sample zigzag share of ring rank r, then Algorithm 2's Ulysses
    split: rows u T .. (u + 1) T - 1 of the share, T = share length / ud."""
    share = zigzag_per_sample_positions(cu_seqlens, rd, ring_rank)
    if len(share) % ud != 0:
        raise ValueError(f"share of {len(share)} tokens does not split into {ud} equal parts")
    n = len(share) // ud
    return share[ulysses_rank * n:(ulysses_rank + 1) * n]


def zigzag_extract(x, rd, ud, ring_rank, ulysses_rank):
    """Local shard of (B, S, H, D) array ``x`` for rank (r, u): (B, 2c/ud, H, D)."""
    pos = zigzag_local_positions(x.shape[1], rd, ud, ring_rank, ulysses_rank)
    return x[:, pos].copy()


def zigzag_extract_all(x, rd, ud):
    """Every rank's shard, stacked rank-major: (rd, ud, B, 2c/ud, H, D)."""
    return np.stack([np.stack([zigzag_extract(x, rd, ud, r, u) for u in range(ud)])
                     for r in range(rd)])


def zigzag_scatter_all(shards, S):
    """Inverse of :func:`zigzag_extract_all`: put every shard back at its
    global positions.  ``shards``: (rd, ud, B, L, H, D)."""
    rd, ud, B, L, H, D = shards.shape
    out = np.zeros((B, S, H, D), dtype=shards.dtype)
    for r in range(rd):
        for u in range(ud):
            out[:, zigzag_local_positions(S, rd, ud, r, u)] = shards[r, u]
    return out


def chunk_owner(chunk, rd):
    """Ring rank that holds zigzag chunk ``chunk`` (0 <= chunk < 2 rd)."""
    return chunk if chunk < rd else 2 * rd - 1 - chunk


# --------------------------------------------------------------------------
# Ulysses 4D all-to-all as a layout ([USP review] section 三, the AllToAll4D
# box: (bs, L/N, hc, hd) -> (hc/N, bs, L, hd); Algorithm 1 steps 1-3 and 5)
# --------------------------------------------------------------------------

def ulysses_fwd(shards, ulysses_rank):
    """What Ulysses rank u holds after the forward all-to-all.

    ``shards``: the N sequence shards of the group, each (bs, L/N, hc, hd), in
    Ulysses-rank order.  Rank u receives head block u (hc/N contiguous heads)
    from every peer; the sequence is gathered in peer order.  Result:
    (hc/N, bs, L, hd).
    """
    N = len(shards)
    hc = shards[0].shape[2]
    if hc % N != 0:
        raise ValueError("head count must divide by the Ulysses degree")
    hb = hc // N
    gathered = np.concatenate([s[:, :, ulysses_rank * hb:(ulysses_rank + 1) * hb, :] for s in shards],
                              axis=1)                       # (bs, L, hc/N, hd)
    return np.ascontiguousarray(np.transpose(gathered, (2, 0, 1, 3)))


def ulysses_inv(head_shards, ulysses_rank):
    """Algorithm 1 step 5 for Ulysses rank u: the inverse all-to-all.

    ``head_shards``: the N head-major tensors of the group, each
    (hc/N, bs, L, hd).  Rank u gets back its sequence slice u (L/N tokens) with
    all hc heads, head block u' coming from peer u'.  Result: (bs, L/N, hc, hd).
    """
    N = len(head_shards)
    L = head_shards[0].shape[2]
    if L % N != 0:
        raise ValueError("sequence length must divide by the Ulysses degree")
    ls = L // N
    parts = [np.transpose(h[:, :, ulysses_rank * ls:(ulysses_rank + 1) * ls, :], (1, 2, 0, 3))
             for h in head_shards]                          # each (bs, L/N, hc/N, hd)
    return np.ascontiguousarray(np.concatenate(parts, axis=2))


def ulysses_fwd_heads(shards, ulysses_rank, h0, nh):
    """Head chunk [h0, h0 + nh) of Ulysses rank u's head block after the
    forward all-to-all ([UPipe page] section 2, headwise chunking: the
    all-to-all moves one chunk of every head block at a time).

    ``shards``: the N sequence shards of the group, each (bs, L/N, hc, hd).
    Element [i, b, u' L/N + t, :] of the result is element
    [b, t, u hc/N + h0 + i, :] of shard u'.  Result: (nh, bs, L, hd).
    """
    N = len(shards)
    bs, ls, hc, hd = shards[0].shape
    hb = hc // N
    if hc % N or h0 < 0 or nh < 1 or h0 + nh > hb:
        raise ValueError("head chunk outside the head block")
    out = np.empty((nh, bs, N * ls, hd), dtype=shards[0].dtype)
    for up, sh in enumerate(shards):
        for i in range(nh):
            out[i, :, up * ls:(up + 1) * ls, :] = sh[:, :, ulysses_rank * hb + h0 + i, :]
    return out


def ulysses_inv_heads(head_chunks, ulysses_rank, h0, hc, out):
    """Inverse all-to-all of one head chunk for Ulysses rank u, into ``out``
    ((bs, L/N, hc, hd), rank u's output shard): peer u' computed heads
    u' hc/N + h0 .. + nh of the whole gathered sequence, and rank u takes its
    sequence slice u of them.  Heads outside the chunk are left as they are.

    ``head_chunks``: the N peers' chunk outputs, each (nh, bs, L, hd).
    """
    N = len(head_chunks)
    nh, bs, L, hd = head_chunks[0].shape
    hb, ls = hc // N, L // N
    if hc % N or L % N or h0 < 0 or h0 + nh > hb:
        raise ValueError("head chunk outside the head block")
    for up, hcnk in enumerate(head_chunks):
        for i in range(nh):
            out[:, :, up * hb + h0 + i, :] = hcnk[i, :, ulysses_rank * ls:(ulysses_rank + 1) * ls, :]
    return out


# --------------------------------------------------------------------------
# Ring schedule ([CP vs Ulysses] concepts section and Figure 1)
# --------------------------------------------------------------------------

def ring_kv_block(ring_rank, step, cp):
    """KV block held by rank r at step t: the KV moves one rank forward per
    step, so after t steps rank r holds the block that started on rank r - t."""
    return (ring_rank - step) % cp


# --------------------------------------------------------------------------
# Causal tile classes and load accounting ([CP vs Ulysses] Figure 2 and the
# section "为什么要一头一尾配对"; [USP review] section 二 on the 7x imbalance)
# --------------------------------------------------------------------------

FULL, DIAGONAL, SKIP = "full", "diagonal", "skip"


def tile_class(q_chunk, kv_chunk):
    """Class of the (query chunk, key chunk) cell of the causal mask."""
    if q_chunk > kv_chunk:
        return FULL
    if q_chunk == kv_chunk:
        return DIAGONAL
    return SKIP


_WEIGHT = {FULL: 1.0, DIAGONAL: 0.5, SKIP: 0.0}   # a diagonal cell counts half


def zigzag_chunks(ring_rank, rd):
    """The two zigzag chunks of ring rank r, in local order."""
    return (ring_rank, 2 * rd - 1 - ring_rank)


def step_units(ring_rank, step, cp):
    """Causal work of rank r at ring step t, in units of one chunk-pair cell."""
    j = ring_kv_block(ring_rank, step, cp)
    return sum(_WEIGHT[tile_class(a, b)]
               for a in zigzag_chunks(ring_rank, cp) for b in zigzag_chunks(j, cp))


def zigzag_rank_units(ring_rank, cp):
    """Total causal work of a zigzag rank over its cp steps (small cells)."""
    return sum(step_units(ring_rank, t, cp) for t in range(cp))


def sequential_rank_units(rank, cp):
    """Causal work of rank ``rank`` when the sequence is cut into cp blocks in
    order (the "basic" split), in units of one big block cell."""
    return sum(_WEIGHT[tile_class(rank, b)] for b in range(cp))


def visible_pairs(q_pos, k_pos, seg_start=None):
    """Exact number of visible (query, key) pairs: key position <= query
    position (and, with packed samples, key in the query's sample)."""
    q_pos = np.asarray(q_pos)
    k_sorted = np.sort(np.asarray(k_pos))
    hi = np.searchsorted(k_sorted, q_pos, side="right")
    if seg_start is None:
        return int(hi.sum())
    lo = np.searchsorted(k_sorted, np.asarray(seg_start), side="left")
    return int(np.maximum(hi - lo, 0).sum())


# --------------------------------------------------------------------------
# Packed samples ([ByteScale notes], motivation: short samples packed into one
# long sequence).  cu_seqlens holds n+1 boundaries 0 = b_0 < ... < b_n = S.
# --------------------------------------------------------------------------

def segment_start(cu_seqlens, pos):
    """First global position of the sample that holds each position."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = np.searchsorted(cu, np.asarray(pos), side="right") - 1
    return cu[seg]
