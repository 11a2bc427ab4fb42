"""GPU parity of the split walk (usp_attn_fwd_split): small launches whose
heavy query tiles walk their ring steps in two workgroups, merged by the LSE
rule, against the CPU oracle and against the unsplit walk.  Called through
the C ABI (ctypes)."""
import numpy as np
import pytest
import torch

from sequence_ring_attention_amd import binding as B
from tests.gpu_common import check_close, f64, guarded, say
from tests.test_gpu_kernels import ATTN_CASES, _layout, _oracle_rank, _out, _prepare, _to_bshd

pytestmark = pytest.mark.gpu

BF16_CASES = sorted(n for n, c in ATTN_CASES.items() if c[8] == "bf16")
# causal, unpacked, cp >= 2 and several query tiles per rank: a heavy tile is split
SPLITS = {"bf16_aligned", "bf16_ragged_gqa_b2", "bf16_cp3_headmajor", "bf16_d64_mqa", "bf16_b2_headmajor_gqa",
          "bf16_strided_views"}


def _workspace(desc, ring_rank, dev):
    n = B.usp_attn_fwd_split_workspace(desc, ring_rank)
    return torch.full(((n + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)


@pytest.mark.parametrize("name", BF16_CASES)
def test_split_walk_per_rank_and_all_ranks(name):
    P = _prepare(name)
    dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
    refs = [_oracle_rank(P, r) for r in range(cp)]
    oshape = (H, Bn, L, D) if P["layout"] == "hbsd" else (Bn, L, H, D)
    split_seen = False
    for r in range(cp):
        say("split walk", name, "rank", r)
        o, ok1 = _out(P, oshape, torch.bfloat16, dev)
        lse, ok2 = guarded((H, Bn, L), torch.float32, dev)
        desc = B.attn_desc(P["S"], cp, P["qs"][r], P["ks"], P["vs"], o=o, layout=_layout(P),
                           causal=P["causal"], cu_seqlens=P["cu_t"])
        ws = _workspace(desc, r, dev)
        B.usp_attn_fwd_split(P["qs"][r], P["ks"], P["vs"], o, lse, desc, r, ws)
        torch.cuda.synchronize()
        assert ok1() and ok2()
        split_seen |= bool(torch.isfinite(ws).any())
        check_close(_to_bshd(P, o), f64(lse), refs[r][0], refs[r][1], "bf16", f"{name} split walk r{r}",
                    out_bf16=True)
        # against the unsplit walk: the same result up to the merge's rounding
        o2, _ = _out(P, oshape, torch.bfloat16, dev)
        lse2 = torch.empty((H, Bn, L), dtype=torch.float32, device=dev)
        desc2 = B.attn_desc(P["S"], cp, P["qs"][r], P["ks"], P["vs"], o=o2, layout=_layout(P),
                            causal=P["causal"], cu_seqlens=P["cu_t"])
        B.usp_attn_fwd(P["qs"][r], P["ks"], P["vs"], o2, lse2, desc2, r)
        torch.cuda.synchronize()
        # one bf16 spacing of the value apart at most, plus the parity bar
        assert bool(((o.float() - o2.float()).abs() <= 1e-2 + o2.float().abs() * 2.0 ** -7).all())
        fin = torch.isfinite(lse2)
        assert torch.equal(fin, torch.isfinite(lse))
        if fin.any():
            assert float((lse - lse2)[fin].abs().max()) <= 1e-5
    say("split walk all ranks", name)
    o_all, ok1 = _out(P, (cp, *oshape), torch.bfloat16, dev)
    lse_all, ok2 = guarded((cp, H, Bn, L), torch.float32, dev)
    desc = B.attn_desc(P["S"], cp, P["qs"], P["ks"], P["vs"], o=o_all, layout=_layout(P),
                       causal=P["causal"], cu_seqlens=P["cu_t"], all_ranks=True)
    ws = _workspace(desc, -1, dev)
    B.usp_attn_fwd_split(P["qs"], P["ks"], P["vs"], o_all, lse_all, desc, -1, ws)
    torch.cuda.synchronize()
    assert ok1() and ok2()
    split_seen |= bool(torch.isfinite(ws).any())
    for r in range(cp):
        check_close(_to_bshd(P, o_all[r]), f64(lse_all[r]), refs[r][0], refs[r][1], "bf16",
                    f"{name} split all-ranks r{r}", out_bf16=True)
    if name in SPLITS:
        assert split_seen, "no tile was split"


def test_split_walk_reuses_its_workspace():
    """Two calls in a row on one workspace, the second on a smaller case:
    stale partials of the first must not leak into the second."""
    outs = []
    ws = None
    for name in ("bf16_b2_headmajor_gqa", "bf16_aligned"):
        P = _prepare(name)
        dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
        oshape = (H, Bn, L, D) if P["layout"] == "hbsd" else (Bn, L, H, D)
        o, ok1 = _out(P, oshape, torch.bfloat16, dev)
        lse, ok2 = guarded((H, Bn, L), torch.float32, dev)
        desc = B.attn_desc(P["S"], cp, P["qs"][0], P["ks"], P["vs"], o=o, layout=_layout(P), causal=P["causal"])
        if ws is None:
            ws = _workspace(desc, 0, dev)
        assert ws.numel() * 4 >= B.usp_attn_fwd_split_workspace(desc, 0)
        say("split walk reuse", name)
        B.usp_attn_fwd_split(P["qs"][0], P["ks"], P["vs"], o, lse, desc, 0, ws)
        torch.cuda.synchronize()
        assert ok1() and ok2()
        ref = _oracle_rank(P, 0)
        check_close(_to_bshd(P, o), f64(lse), ref[0], ref[1], "bf16", f"{name} reuse", out_bf16=True)
        outs.append(o)
    assert len(outs) == 2


def test_split_walk_rejects_a_small_workspace():
    P = _prepare("bf16_aligned")
    dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
    o = torch.empty((Bn, L, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, Bn, L), dtype=torch.float32, device=dev)
    desc = B.attn_desc(P["S"], cp, P["qs"][0], P["ks"], P["vs"], o=o)
    need = B.usp_attn_fwd_split_workspace(desc, 0)
    small = torch.empty((need // 4 - 64,), dtype=torch.float32, device=dev)
    with pytest.raises(B.UspError):
        B.usp_attn_fwd_split(P["qs"][0], P["ks"], P["vs"], o, lse, desc, 0, small)
