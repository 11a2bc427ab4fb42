"""Seeded sweep of the bf16 walk over packed streams of many short samples
(20-79 samples of 2cp..22cp tokens each), both splits of the shares (R9
whole-stream zigzag and R20 per-sample zigzag), cp 2 or 4, D 64 or 128, MHA
and GQA.  Rows that see only a few keys carry the bf16 rounding of P on
almost undiluted, which is the hardest case for the max-abs bar; every rank's
walk is checked against the fp64 oracle over the whole share."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as ix
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from tests.gpu_common import check_close, device, f64, say

pytestmark = pytest.mark.gpu

N_CASES = 60


def _cases():
    rng = np.random.default_rng(1)
    out = []
    for c in range(N_CASES):
        cp = int(rng.choice([2, 4]))
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2]))
        per_sample = bool(rng.integers(0, 2))
        lens = (rng.integers(1, 12, size=int(rng.integers(20, 80))) * 2 * cp).tolist()
        out.append((c, cp, D, H, Hkv, per_sample, [0] + np.cumsum(lens).tolist()))
    return out


def test_packed_short_samples_sweep():
    dev = device()
    for c, cp, D, H, Hkv, per_sample, cu in _cases():
        S, L = cu[-1], cu[-1] // cp
        q, k, v = inputs.qkv(1, S, H, Hkv, D, "bf16", 7000 + c)
        o_ref, lse_ref = oa.attention_full(f64(q), f64(k), f64(v), D ** -0.5, True, cu)
        if per_sample:
            pos = [np.asarray(ix.zigzag_per_sample_local_positions(cu, cp, 1, r, 0)) for r in range(cp)]
        else:
            pos = [np.asarray(ix.zigzag_share_positions(S, cp, r)) for r in range(cp)]
        idx = torch.from_numpy(np.concatenate(pos)).to(dev)

        def share(x):
            return x.to(dev).index_select(1, idx).view(1, cp, L, *x.shape[2:]).transpose(0, 1).contiguous()
        qs, ks, vs = share(q), share(k), share(v)
        for r in range(cp):
            say("packed sweep case", c, "rank", r, dict(cp=cp, D=D, H=H, Hkv=Hkv, per_sample=per_sample, S=S))
            o = torch.empty_like(qs[r])
            lse = torch.empty(H, 1, L, dtype=torch.float32, device=dev)
            desc = B.attn_desc(S, cp, qs[r], ks, vs, o=o, cu_seqlens=cu, zigzag_per_sample=per_sample)
            B.usp_attn_fwd(qs[r], ks, vs, o, lse, desc, r)
            torch.cuda.synchronize()
            check_close(f64(o), f64(lse), o_ref[:, pos[r]], lse_ref[:, :, pos[r]], "bf16",
                        f"case {c} rank {r}", out_bf16=True)
