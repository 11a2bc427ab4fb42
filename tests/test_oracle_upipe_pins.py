"""Pins of the oracle's headwise chunking ([UPipe page] section 2): the
Ulysses layout of a head range and its inverse, and Algorithm 1 with each
head block pushed through in chunks.

u1  the forward layout of a head chunk is that chunk of the full layout
    (itself pinned by the degenerate-grid and gather-order pins);
u2  the inverse of every chunk, over all chunks, is the full inverse, and
    forward then inverse restores the chunk's heads;
u3  the chunked USP equals the unchunked USP and the one-shot definition, for
    MHA, GQA (chunks of whole groups and chunks inside a group), packed
    samples (both splits) and non-causal attention;
u4  chunks that split a head block unevenly, or that neither hold whole GQA
    groups nor lie inside one, are refused;
u5  planted mistakes (a KV chunk that never advances; a head offset that
    forgets the Ulysses rank) fail u3.
"""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import index as ix
from oracle import usp as ou

RNG = np.random.default_rng(2024)


def shards(N, bs, ls, hc, hd):
    return [RNG.standard_normal((bs, ls, hc, hd)) for _ in range(N)]


@pytest.mark.parametrize("N,hc", [(2, 8), (4, 8), (1, 3), (3, 6)])
def test_u1_forward_chunk_is_a_slice_of_the_full_layout(N, hc):
    sh = shards(N, 2, 3, hc, 4)
    hb = hc // N
    for u in range(N):
        full = ix.ulysses_fwd(sh, u)
        for h0 in range(hb):
            for nh in range(1, hb - h0 + 1):
                assert np.array_equal(ix.ulysses_fwd_heads(sh, u, h0, nh), full[h0:h0 + nh])


@pytest.mark.parametrize("N,hc,nh", [(2, 8, 1), (2, 8, 2), (4, 8, 2), (3, 6, 2), (1, 4, 4)])
def test_u2_inverse_chunks_make_the_full_inverse_and_undo_the_forward(N, hc, nh):
    bs, ls, hd = 2, 3, 4
    hb = hc // N
    heads = [RNG.standard_normal((hb, bs, N * ls, hd)) for _ in range(N)]   # every peer's head block
    for u in range(N):
        out = np.full((bs, ls, hc, hd), np.nan)
        for h0 in range(0, hb, nh):
            ix.ulysses_inv_heads([h[h0:h0 + nh] for h in heads], u, h0, hc, out)
        assert np.array_equal(out, ix.ulysses_inv(heads, u))
    sh = shards(N, bs, ls, hc, hd)
    back = [np.full_like(s, np.nan) for s in sh]
    for h0 in range(0, hb, nh):
        chunk = [ix.ulysses_fwd_heads(sh, u, h0, nh) for u in range(N)]      # what each rank holds
        for u in range(N):
            ix.ulysses_inv_heads(chunk, u, h0, hc, back[u])
    for s, b in zip(sh, back):
        assert np.array_equal(s, b)


CASES = {  # B, S, H, Hkv, D, rd, ud, chunk, causal, cu, per_sample
    "mha_chunk1": (1, 64, 4, 4, 8, 2, 2, 1, True, None, False),
    "gqa_chunk2": (1, 96, 8, 4, 8, 3, 2, 2, True, None, False),
    "gqa_chunk2_inside_a_group_of4": (1, 64, 8, 2, 8, 2, 2, 2, True, None, False),
    "gqa_chunk1_of_group2": (1, 64, 8, 4, 8, 2, 2, 1, True, None, False),
    "gqa_b2_chunk2_of4": (2, 64, 8, 2, 8, 2, 1, 4, True, None, False),
    "packed_stream": (1, 128, 8, 4, 8, 2, 2, 2, True, [0, 24, 40, 96, 128], False),
    "packed_per_sample": (1, 128, 8, 4, 8, 2, 2, 2, True, [0, 32, 40, 96, 128], True),
    "noncausal": (1, 64, 4, 2, 8, 2, 2, 2, False, None, False),
}


def qkv(B, S, H, Hkv, D):
    return (RNG.standard_normal((B, S, H, D)), RNG.standard_normal((B, S, Hkv, D)),
            RNG.standard_normal((B, S, Hkv, D)))


@pytest.mark.parametrize("name", sorted(CASES))
def test_u3_chunked_usp_equals_unchunked_and_the_definition(name):
    B, S, H, Hkv, D, rd, ud, nh, causal, cu, ps = CASES[name]
    Q, K, V = qkv(B, S, H, Hkv, D)
    scale = D ** -0.5
    o_c, l_c = ou.usp_attention_head_chunks(Q, K, V, rd, ud, scale, nh, causal, cu, ps)
    o_u, l_u = ou.usp_attention(Q, K, V, rd, ud, scale, causal, cu, ps)
    o_d, l_d = oa.attention_full(Q, K, V, scale, causal, cu)
    np.testing.assert_allclose(o_c, o_u, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_u, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_c, o_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_d, rtol=0, atol=1e-12)


def test_u4_rejects_uneven_chunks_and_split_groups():
    Q, K, V = qkv(1, 32, 8, 4, 8)
    with pytest.raises(ValueError):
        ou.usp_attention_head_chunks(Q, K, V, 2, 2, 0.3, 3)      # 3 does not divide the block of 4
    Q, K, V = qkv(1, 32, 24, 4, 8)
    with pytest.raises(ValueError):
        ou.usp_attention_head_chunks(Q, K, V, 2, 2, 0.3, 4)      # 4 heads: neither whole groups of 6 nor in one
    with pytest.raises(ValueError):
        ix.ulysses_fwd_heads(shards(2, 1, 2, 8, 4), 0, 3, 2)     # runs past the head block


def _usp_differs(monkeypatch_target, attr, wrong):
    B, S, H, Hkv, D, rd, ud, nh, causal, cu, ps = CASES["gqa_chunk2"]
    Q, K, V = qkv(B, S, H, Hkv, D)
    o_u, _ = ou.usp_attention(Q, K, V, rd, ud, 0.35, causal)
    mp = pytest.MonkeyPatch()
    try:
        mp.setattr(monkeypatch_target, attr, wrong)
        o_c, _ = ou.usp_attention_head_chunks(Q, K, V, rd, ud, 0.35, nh, causal)
    finally:
        mp.undo()
    return np.max(np.abs(o_c - o_u)) > 1e-3


def test_u5_mutant_kv_chunk_that_never_advances_fails():
    assert _usp_differs(ou, "kv_head_chunk", lambda h0, nh, G: (0, nh // G))


def test_u5_mutant_head_offset_without_the_ulysses_rank_fails():
    original = ix.ulysses_fwd_heads
    assert _usp_differs(ix, "ulysses_fwd_heads", lambda sh, u, h0, nh: original(sh, 0, h0, nh))
