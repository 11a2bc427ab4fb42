"""usp_attn_bwd_noalloc through the C ABI against usp_attn_bwd: the same
kernels with the statistics rows in the library's own device array instead
of a caller buffer, so the gradients must be bitwise equal.  Two calls in a
row, the second smaller than the first, so that the array's contents from
one call cannot leak into the next."""
import numpy as np
import pytest
import torch

from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from tests.gpu_common import device, say, shares

pytestmark = pytest.mark.gpu


def _case(S, H, Hkv, D, cp, seed, dev):
    q, k, v = inputs.qkv(1, S, H, Hkv, D, "bf16", seed)
    qs, ks, vs = shares(q.to(dev), cp), shares(k.to(dev), cp), shares(v.to(dev), cp)
    o = torch.empty_like(qs)
    lse = torch.empty(cp, H, 1, S // cp, dtype=torch.float32, device=dev)
    desc = B.attn_desc(S, cp, qs, ks, vs, o=o, all_ranks=True)
    B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
    d_o = inputs.randn(tuple(qs.shape), seed + 7, "bf16").to(dev)
    return qs, ks, vs, o, d_o, lse, desc


def _grads(c, ring_rank, noalloc):
    qs, ks, vs, o, d_o, lse, desc = c
    if ring_rank >= 0:
        qs, o, d_o, lse = qs[ring_rank], o[ring_rank], d_o[ring_rank], lse[ring_rank]
        desc = B.attn_desc(desc.seq_len, desc.cp, qs, ks, vs, o=o)
    dq = torch.full_like(qs, 7.0)
    dk = torch.zeros(ks.shape, dtype=torch.float32, device=qs.device)
    dv = torch.zeros(vs.shape, dtype=torch.float32, device=qs.device)
    if noalloc:
        B.usp_attn_bwd_noalloc(qs, ks, vs, o, d_o, lse, dq, dk, dv, desc, ring_rank)
    else:
        stats = torch.empty(2 * lse.numel(), dtype=torch.float32, device=qs.device)
        B.usp_attn_bwd(qs, ks, vs, o, d_o, lse, dq, dk, dv, stats, desc, ring_rank)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_backward_matches_the_buffer_entry_point_twice():
    dev = device()
    big = _case(2048, 8, 2, 128, 4, 9100, dev)      # 4 x 8 x 512 = 16384 statistics rows
    small = _case(512, 2, 1, 64, 2, 9200, dev)      # 2 x 2 x 256 = 1024 rows, fewer than the first call left
    for name, c, rr in (("large, every rank", big, -1), ("small, every rank", small, -1), ("small, rank 1", small, 1),
                        ("large, rank 2", big, 2)):
        say("noalloc backward", name)
        ref = _grads(c, rr, False)
        got = _grads(c, rr, True)
        for a, b, what in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.isfinite(b).all(), (name, what)
            assert torch.equal(a, b), (name, what, float((a.float() - b.float()).abs().max()))
