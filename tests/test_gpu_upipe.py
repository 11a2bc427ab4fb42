"""GPU parity of headwise chunking ([UPipe page] section 2): the Ulysses
layout of a head range (bit-exact against the oracle, in every mode, and
leaving the heads outside the chunk untouched), and the one-GPU share run
chunk by chunk: bitwise equal to the unchunked share (the heads are
independent and every kernel computes a head the same way), and within the
bf16 bars of the oracle's chunked USP."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as ix
from oracle import usp as ou
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from sequence_ring_attention_amd.pipeline import OneGpuShare
from tests.gpu_common import bits, check_close, device, f64, guarded, say

pytestmark = pytest.mark.gpu

LAYOUT_CASES = [  # B, Ls, hc, hd, dtype, N
    (1, 96, 8, 128, "bf16", 2),
    (2, 40, 12, 64, "bf16", 3),
    (1, 64, 8, 64, "fp32", 4),
    (1, 32, 4, 24, "bf16", 2),    # 48-byte head rows: the head-row copy kinds, forward and inverse
    (2, 17, 6, 128, "fp32", 1),
]


@pytest.mark.parametrize("case", LAYOUT_CASES)
def test_layout_heads_bitexact(case):
    Bn, Ls, hc, hd, dt, N = case
    dev = device()
    hb, L = hc // N, Ls * N
    tdt = torch.float32 if dt == "fp32" else torch.bfloat16
    x = inputs.randn((N, Bn, Ls, hc, hd), 61, dt)
    xd = x.to(dev)
    xs = [bits(x[i]) for i in range(N)]
    for h0, nh in sorted({(0, hb), (0, 1), (hb - 1, 1), (hb // 2, hb - hb // 2), (1, max(1, hb - 2))}):
        if h0 + nh > hb or nh < 1:
            continue
        ref = np.stack([ix.ulysses_fwd_heads(xs, u, h0, nh) for u in range(N)])     # (N, nh, B, L, hd)
        say("layout heads fwd", case, h0, nh)
        out, ok = guarded((N, nh, Bn, L, hd), tdt, dev)
        B.usp_ulysses_a2a_layout_heads(xd, out, N, -1, h0, nh)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(out), ref)
        for u in range(N):
            one, ok = guarded((nh, Bn, L, hd), tdt, dev)
            B.usp_ulysses_a2a_layout_heads(xd, one, N, u, h0, nh)
            torch.cuda.synchronize()
            assert ok() and np.array_equal(bits(one), ref[u])
        # inverse of the chunk into a prefilled output: the chunk's heads
        # come back, every other head keeps its old bits
        hin = inputs.randn((N, nh, Bn, L, hd), 62, dt)
        hs = [bits(hin[i]) for i in range(N)]
        base = inputs.randn((N, Bn, Ls, hc, hd), 63, dt)
        exp = bits(base).copy()
        for u in range(N):
            ix.ulysses_inv_heads(hs, u, h0, hc, exp[u])
        say("layout heads inv", case, h0, nh)
        back, ok = guarded((N, Bn, Ls, hc, hd), tdt, dev)
        back.copy_(base.to(dev))
        B.usp_ulysses_a2a_layout_heads(hin.to(dev), back, N, -1, h0, nh, inverse=True)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(back), exp)
        for u in range(N):
            one, ok = guarded((Bn, Ls, hc, hd), tdt, dev)
            one.copy_(base[u].to(dev))
            B.usp_ulysses_a2a_layout_heads(hin.to(dev), one, N, u, h0, nh, inverse=True)
            torch.cuda.synchronize()
            assert ok() and np.array_equal(bits(one), exp[u])


SHARE_CASES = {  # B, S, H, Hkv, D, rd, ud, chunk, cu, per_sample[, dtype, causal]
    "gqa_chunk2": (1, 2048, 8, 4, 128, 2, 2, 2, None, False),
    "gqa_chunk4_of8_rd4": (1, 4096, 16, 4, 128, 4, 2, 4, None, False),
    "gqa_chunk2_inside_a_group_of4": (1, 2048, 16, 4, 128, 2, 2, 2, None, False),
    "mha_d64_chunk1_b2": (2, 1024, 4, 4, 64, 2, 2, 1, None, False),
    "packed_per_sample_chunk2": (1, 2048, 8, 4, 128, 2, 2, 2, [0, 400, 416, 1680, 2048], True),
    "fp32_gqa_chunk1_d64": (1, 256, 8, 4, 64, 2, 2, 1, None, False, "fp32", True),
    "noncausal_chunk2": (1, 1024, 8, 2, 128, 2, 2, 2, None, False, "bf16", False),
}


def _case(name):
    c = SHARE_CASES[name]
    return c + ("bf16", True) if len(c) == 10 else c


def _run_share(q, k, v, rd, ud, r, u, chunk, cu, ps, causal=True, overlap=False, split=False):
    share = OneGpuShare(q, k, v, rd, ud, r, u, causal=causal, cu_seqlens=cu, per_sample=ps, head_chunk=chunk,
                        overlap_chunks=overlap, split_walk=split)
    share.prepare_peers()
    out = share.step().clone()
    torch.cuda.synchronize()
    return out, share.lse[u].clone()


@pytest.mark.parametrize("name", sorted(SHARE_CASES))
def test_chunked_share_equals_unchunked_and_oracle(name):
    Bn, S, H, Hkv, D, rd, ud, nh, cu, ps, dt, causal = _case(name)
    dev = device()
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, dt, 880 + sorted(SHARE_CASES).index(name))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_ref, lse_ref = ou.usp_attention_head_chunks(f64(q), f64(k), f64(v), rd, ud, D ** -0.5, nh, causal, cu, ps)
    T, hb = S // (rd * ud), H // ud
    for r, u in [(0, 0), (rd - 1, ud - 1)]:
        say("share", name, r, u, "whole head block")
        o_full, l_full = _run_share(qd, kd, vd, rd, ud, r, u, None, cu, ps, causal)
        say("share", name, r, u, "chunks of", nh)
        o_ch, l_ch = _run_share(qd, kd, vd, rd, ud, r, u, nh, cu, ps, causal)
        assert torch.equal(o_ch, o_full) and torch.equal(l_ch, l_full)
        say("share", name, r, u, "chunks of", nh, "on two streams")
        o_ov, l_ov = _run_share(qd, kd, vd, rd, ud, r, u, nh, cu, ps, causal, overlap=True)
        assert torch.equal(o_ov, o_full) and torch.equal(l_ov, l_full)
        pos = (ix.zigzag_per_sample_local_positions(cu, rd, ud, r, u) if ps
               else ix.zigzag_local_positions(S, rd, ud, r, u))
        check_close(f64(o_ch), f64(l_ch[:, :, u * T:(u + 1) * T]), o_ref[:, pos],
                    lse_ref[u * hb:(u + 1) * hb][:, :, pos], dt, f"{name} ({r},{u})", out_bf16=dt == "bf16")
        say("share", name, r, u, "chunks of", nh, "with the split walk")
        o_sp, l_sp = _run_share(qd, kd, vd, rd, ud, r, u, nh, cu, ps, causal, split=True)
        check_close(f64(o_sp), f64(l_sp[:, :, u * T:(u + 1) * T]), o_ref[:, pos],
                    lse_ref[u * hb:(u + 1) * hb][:, :, pos], dt, f"{name} ({r},{u}) split walk",
                    out_bf16=dt == "bf16")


def test_chunked_share_rejects_bad_chunks():
    dev = device()
    q, k, v = inputs.qkv(1, 256, 24, 4, 64, "bf16", 890)
    for bad in (5, 4, 0):          # does not divide 12; neither whole GQA groups of 6 nor inside one; empty
        with pytest.raises(ValueError):
            OneGpuShare(q.to(dev), k.to(dev), v.to(dev), 2, 2, 0, 0, head_chunk=bad)
    with pytest.raises(ValueError):   # two streams of chunks need chunks
        OneGpuShare(q.to(dev), k.to(dev), v.to(dev), 2, 2, 0, 0, overlap_chunks=True)


def test_usp_hybrid_s128k_share_in_head_chunks_is_bitwise_the_same():
    """The benchmark's share, its 16-head block pushed through in 8 chunks of
    2 query heads, each inside one GQA group of 4 (one eighth of the
    head-major query and output tensors at a time)."""
    w = inputs.WORKLOADS["usp_hybrid_s128k_ud2_rd4"]
    dev = device()
    q, k, v = (t.to(dev) for t in inputs.workload_qkv(w))
    say(w.name, "share (0,0) whole head block")
    o_full, l_full = _run_share(q, k, v, w.rd, w.ud, 0, 0, None, None, False)
    say(w.name, "share (0,0) chunks of 2 heads")
    o_ch, l_ch = _run_share(q, k, v, w.rd, w.ud, 0, 0, 2, None, False)
    assert torch.isfinite(o_ch).all()
    assert torch.equal(o_ch, o_full) and torch.equal(l_ch, l_full)
    say(w.name, "share (0,0) chunks of 2 heads on two streams")
    o_ov, l_ov = _run_share(q, k, v, w.rd, w.ud, 0, 0, 2, None, False, overlap=True)
    assert torch.equal(o_ov, o_full) and torch.equal(l_ov, l_full)


def test_usp_hybrid_s128k_share_in_head_chunks_with_the_split_walk():
    """The benchmark's share in 8 chunks of 2 query heads with the split walk
    (each chunk's launch is a single round, so its heavy query tiles walk
    their ring steps in two workgroups): within one bf16 spacing of the
    whole block's output, and 128 seeded rows of the shard (all 32 heads)
    against the oracle over all 131072 keys."""
    w = inputs.WORKLOADS["usp_hybrid_s128k_ud2_rd4"]
    dev = device()
    q, k, v = inputs.workload_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    say(w.name, "share (0,0) whole head block")
    o_full, l_full = _run_share(qd, kd, vd, w.rd, w.ud, 0, 0, None, None, False)
    say(w.name, "share (0,0) chunks of 2 heads, split walk")
    o_sp, l_sp = _run_share(qd, kd, vd, w.rd, w.ud, 0, 0, 2, None, False, split=True)
    assert bool(((o_sp.float() - o_full.float()).abs() <= 1e-2 + o_full.float().abs() * 2.0 ** -7).all())
    assert float((l_sp - l_full).abs().max()) <= 1e-5
    T, hb = w.S // (w.rd * w.ud), w.H // w.ud
    rows = np.sort(np.random.default_rng(4321).choice(T, size=128, replace=False))
    p = ix.zigzag_local_positions(w.S, w.rd, w.ud, 0, 0)[rows]
    o_ref, l_ref = oa.masked_attention(f64(q[:, p]), f64(k), f64(v), w.scale, q_pos=p)   # (B, n, H, D), (H, B, n)
    check_close(f64(o_sp)[:, rows], f64(l_sp)[:, :, rows], o_ref, l_ref[:hb], "bf16",
                f"{w.name} (0,0) split walk 128 rows x {w.H} heads", out_bf16=True)
