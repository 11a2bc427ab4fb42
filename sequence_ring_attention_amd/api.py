"""The user-level calls of the pages' interface, on one GPU.

"USP" paper review, section 三 (usage): a rank's local Q, K, V come from
``EXTRACT_FUNC_DICT["zigzag"](X, rank, world_size, rd, ud)``, and attention
runs through ``LongContextAttention(...)(q, k, v, dropout_p, causal,
window_size, softcap, alibi_slopes, deterministic, return_attn_probs)``.
Here both are thin wrappers over the C entry points: ``zigzag_extract``
maps the global rank to (ring rank, Ulysses rank) and calls
usp_zigzag_extract; ``attn`` refuses the options the library does not
implement and calls usp_attn_fwd on a ring rank's share with the cp KV
blocks the ring would bring (resident in HBM on one GPU).  Argument
marshalling only: every step of the computation runs in the HIP kernels.
"""
import torch

from . import binding as B

ULYSSES_INNER = "ulysses_inner"   # rank = r * ud + u: the order of dimensions TP -> Ulysses -> Ring
RING_INNER = "ring_inner"         # rank = u * rd + r: the process-grid figure's numbering


def rank_to_grid(rank, world_size, rd, ud, order=ULYSSES_INNER):
    """Global rank -> (ring_rank, ulysses_rank) on a ud x rd grid.

    The pages number the grid two ways (the process-grid figure puts a
    Ulysses group in a column, the parallel-order tip makes Ulysses the
    innermost dimension); ``order`` selects one, Ulysses innermost by
    default.  Nothing computed depends on the choice."""
    if world_size != rd * ud:
        raise ValueError(f"world_size {world_size} != rd * ud = {rd * ud}")
    if not 0 <= rank < world_size:
        raise ValueError(f"rank {rank} outside [0, {world_size})")
    if order == ULYSSES_INNER:
        return rank // ud, rank % ud
    if order == RING_INNER:
        return rank % rd, rank // rd
    raise ValueError(f"unknown rank order {order!r}")


def zigzag_extract(X, rank, world_size, rd, ud, order=ULYSSES_INNER, stream=None):
    """Rank ``rank``'s zigzag shard of X (B, S, H, D): chunks r and 2 rd - 1 - r
    of 2 rd, then the u-th of ud equal parts ("USP" review, Algorithm 2).
    Returns a new (B, S / (rd ud), H, D) tensor on X's device."""
    r, u = rank_to_grid(rank, world_size, rd, ud, order)
    Bn, S, H, D = X.shape
    if S % (2 * rd * ud):
        raise ValueError(f"S = {S} is not divisible by 2 rd ud = {2 * rd * ud}")
    out = torch.empty((Bn, S // (rd * ud), H, D), dtype=X.dtype, device=X.device)
    return B.usp_zigzag_extract(X, out, rd, ud, r, u, stream=stream)


def _unsupported(what):
    return B.UspError(B.USP_ERR_UNSUPPORTED, f"attn: {what} is not supported")


def attn(q, k_all, v_all, ring_rank, dropout_p=0.0, causal=True, window_size=(-1, -1), softcap=0.0,
         alibi_slopes=None, deterministic=False, return_attn_probs=False, softmax_scale=None, cu_seqlens=None,
         zigzag_per_sample=False, stream=None):
    """Ring attention of one ring rank's queries over the cp KV blocks.

    q: the rank's zigzag share (B, 2c, Hq, D); k_all, v_all: the cp ring
    blocks (cp, B, 2c, Hkv, D), block j being ring rank j's share; bf16 or
    fp32, all on the GPU.  Returns o (B, 2c, Hq, D) in q's dtype, and with
    ``return_attn_probs`` also lse (Hq, B, 2c) fp32 (the pages leave what
    it returns open beyond the log-sum-exp).  ``deterministic`` is accepted
    either way: the kernels' results never depend on scheduling.  Dropout,
    a sliding window, softcap and ALiBi raise USP_ERR_UNSUPPORTED before
    anything runs."""
    if dropout_p != 0.0:
        raise _unsupported("dropout_p != 0")
    if tuple(window_size) != (-1, -1):
        raise _unsupported("a sliding window")
    if softcap != 0.0:
        raise _unsupported("softcap")
    if alibi_slopes is not None:
        raise _unsupported("ALiBi")
    cp, Bn, L, Hkv, D = k_all.shape
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[2], Bn, L), dtype=torch.float32, device=q.device)
    desc = B.attn_desc(cp * L, cp, q, k_all, v_all, o=o, causal=causal, softmax_scale=softmax_scale,
                       cu_seqlens=cu_seqlens, zigzag_per_sample=zigzag_per_sample)
    B.usp_attn_fwd(q, k_all, v_all, o, lse, desc, ring_rank, stream=stream)
    return (o, lse) if return_attn_probs else o
