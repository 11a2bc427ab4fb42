"""GPU parity of the user-level wrappers: zigzag_extract(X, rank, world_size,
rd, ud) equals the oracle's Algorithm 2 shard of that rank in both grid
numberings, and attn equals usp_attn_fwd bit for bit and the oracle within
the parity bars."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as ix
from sequence_ring_attention_amd import api
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from tests.gpu_common import bits, check_close, device, f64, say, shares

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("order", [api.ULYSSES_INNER, api.RING_INNER])
def test_zigzag_extract_by_global_rank(order):
    Bn, S, H, D, rd, ud = 2, 96, 4, 64, 3, 2
    dev = device()
    x = inputs.randn((Bn, S, H, D), 71, "bf16")
    ref = ix.zigzag_extract_all(bits(x), rd, ud)                 # (rd, ud, B, T, H, D)
    xd = x.to(dev)
    for g in range(rd * ud):
        say("zigzag_extract rank", g, order)
        r, u = api.rank_to_grid(g, rd * ud, rd, ud, order)
        out = api.zigzag_extract(xd, g, rd * ud, rd, ud, order)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref[r, u])


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_attn_wrapper_matches_the_entry_point_and_the_oracle(dt):
    Bn, S, H, Hkv, D, cp = 1, 512, 4, 2, 64, 4
    dev = device()
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, dt, 72)
    qs, ks, vs = (shares(t.to(dev), cp) for t in (q, k, v))      # (cp, B, 2c, heads, D)
    for r in (0, cp - 1):
        say("attn wrapper", dt, "rank", r)
        o, lse = api.attn(qs[r], ks, vs, r, return_attn_probs=True, deterministic=True)
        o_only = api.attn(qs[r], ks, vs, r)
        o_ref = torch.empty_like(qs[r])
        l_ref = torch.empty_like(lse)
        desc = B.attn_desc(S, cp, qs[r], ks, vs, o=o_ref)
        B.usp_attn_fwd(qs[r], ks, vs, o_ref, l_ref, desc, r)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref) and torch.equal(o_only, o_ref)
        pos = ix.zigzag_share_positions(S, cp, r)
        o_x, l_x = oa.masked_attention(f64(q)[:, pos], f64(k), f64(v), D ** -0.5, q_pos=pos)
        check_close(f64(o), f64(lse), o_x, l_x, dt, f"attn wrapper {dt} r{r}", out_bf16=dt == "bf16")
