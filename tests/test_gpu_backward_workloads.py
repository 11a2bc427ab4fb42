"""Backward at the full 128K-token share, in the launch configuration the
benchmark times: usp_attn_bwd on OneGpuShare's head-major buffers after the
share's forward.  Checked against the oracle on rows it computes one by one
(query rows for dQ; keys that few queries see for dK and dV), plus what holds
at any size: keys no query of the rank sees get exactly zero, and over the
whole walk the sum of dK vanishes and the sum of dV equals the sum of dO."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import backward as ob
from oracle import index as ix
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from sequence_ring_attention_amd.pipeline import OneGpuShare
from tests.gpu_common import check_grad, device, f64, sample_rows, say, shares

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS["usp_hybrid_s128k_ud2_rd4"]


def _hm_rows(x, rows):
    """Head-major (H, B, L, D) rows -> numpy (B, rows, H, D)."""
    return np.transpose(f64(x[:, :, rows]), (1, 2, 0, 3))


@pytest.mark.parametrize("r,u", [(0, 0), (3, 1)])
def test_usp_hybrid_s128k_backward_share(r, u):
    w = W
    dev = device()
    q, k, v = inputs.workload_qkv(w)
    say(w.name, "backward share", r, u, "forward")
    share = OneGpuShare(q.to(dev), k.to(dev), v.to(dev), w.rd, w.ud, r, u)
    share.prepare_peers()
    share.step()
    qh, kh, vh, oh, lse = share.qh[u], share.kh[u], share.vh[u], share.oh[u], share.lse[u]
    d_o = inputs.randn(tuple(oh.shape), 99, "bf16").to(dev)
    dq = torch.empty_like(qh)
    dk = torch.zeros(kh.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(vh.shape, dtype=torch.float32, device=dev)
    stats = torch.empty(2 * lse.numel(), dtype=torch.float32, device=dev)
    say(w.name, "backward share", r, u, "usp_attn_bwd")
    B.usp_attn_bwd(qh, kh, vh, oh, d_o, lse, dq, dk, dv, stats, share.desc(u), r)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()

    hb, kb, c, L, S = w.H // w.ud, w.Hkv // w.ud, w.chunk, w.share, w.S
    qn = f64(q[:, :, u * hb:(u + 1) * hb])
    kn = f64(k[:, :, u * kb:(u + 1) * kb])
    vn = f64(v[:, :, u * kb:(u + 1) * kb])
    pos = [ix.zigzag_share_positions(S, w.rd, j) for j in range(w.rd)]
    all_pos = np.arange(S)

    # dQ on sampled query rows (each row's softmax over all its keys, exactly)
    rows = sample_rows(L, c, 16, 70 + r)
    gq, _, _ = ob.attention_backward(qn[:, pos[r][rows]], kn, vn, _hm_rows(d_o, rows), w.scale,
                                     q_pos=pos[r][rows], k_pos=all_pos)
    check_grad(_hm_rows(dq, rows), gq, "bf16", f"{w.name} ({r},{u}) dq rows")

    # keys that no query of this rank sees: exactly zero
    qmax = int(pos[r].max())
    for j in range(w.rd):
        hidden = np.nonzero(pos[j] > qmax)[0]
        if hidden.size:
            assert not dk[j][:, :, hidden].any() and not dv[j][:, :, hidden].any(), f"block {j} hidden keys"

    # the last keys this rank sees (its own block's second chunk ends at its
    # last query): few queries see them, so the oracle takes those queries'
    # softmax statistics exactly and their contributions to these keys
    last = np.nonzero(pos[r] == qmax)[0][0]
    keys = np.array([last, last - 2, last - 39, last - 128])
    vis_q = np.nonzero(pos[r] >= pos[r][keys].min())[0]
    o_v, lse_v = oa.masked_attention(qn[:, pos[r][vis_q]], kn, vn, w.scale, q_pos=pos[r][vis_q], k_pos=all_pos)
    do_v = _hm_rows(d_o, vis_q)
    _, gk, gv = ob.ring_step_backward(qn[:, pos[r][vis_q]], kn[:, pos[r][keys]], vn[:, pos[r][keys]], do_v, lse_v,
                                      ob.delta_rows(o_v, do_v), w.scale, pos[r][vis_q], pos[r][keys])
    check_grad(_hm_rows(dk[r], keys), gk, "bf16", f"{w.name} ({r},{u}) dk last keys")
    check_grad(_hm_rows(dv[r], keys), gv, "bf16", f"{w.name} ({r},{u}) dv last keys")

    # whole-walk identities: each softmax row sums to one and each dS row to zero
    dk_sum = f64(dk).sum(axis=(0, 3))             # (kb, B, D)
    dk_abs = np.abs(f64(dk)).sum(axis=(0, 3))
    assert np.all(np.abs(dk_sum) <= 1e-2 * dk_abs), float((np.abs(dk_sum) / dk_abs).max())
    dv_sum = f64(dv).sum(axis=(0, 3))
    G = hb // kb
    do64 = f64(d_o).reshape(kb, G, *d_o.shape[1:])  # (kb, G, B, L, D)
    ref = do64.sum(axis=(1, 3))
    assert np.all(np.abs(dv_sum - ref) <= 1e-3 * np.abs(do64).sum(axis=(1, 3))), \
        float(np.abs(dv_sum - ref).max())


def test_packed_varlen_s32k_per_sample_backward_all_ranks():
    """The per-sample split of the packed 32K workload (lengths rounded to
    multiples of 2 cp), each rank's usp_attn_bwd after its forward as the
    benchmark launches them: dQ on every piece's first and last rows and a
    seeded random set, dK and dV on the last three chunks of the shortest
    samples (few queries see them, so the oracle takes those queries exactly),
    and the whole-walk identities."""
    w = inputs.WORKLOADS["packed_varlen_s32k_cp4"]
    dev = device()
    q, k, v = inputs.workload_qkv(w)
    cu = inputs.workload_cu_seqlens(w, multiple=2 * w.rd)
    rd, S, L = w.rd, w.S, w.share

    def ps(x):
        out = torch.empty((rd, 1, w.B, L) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
        B.usp_zigzag_extract_varlen(x.to(dev), out, rd, 1, -1, -1, cu)
        return out[:, 0]

    say(w.name, "per-sample backward: extract")
    qs, ks, vs = ps(q), ps(k), ps(v)
    pos = [ix.zigzag_per_sample_positions(cu, rd, r) for r in range(rd)]
    owner = np.empty(S, dtype=np.int64)
    local = np.empty(S, dtype=np.int64)
    for j in range(rd):
        owner[pos[j]] = j
        local[pos[j]] = np.arange(L)
    qn, kn, vn = f64(q), f64(k), f64(v)
    all_pos = np.arange(S)
    lens = np.diff(cu)
    short = np.argsort(lens, kind="stable")[:2]
    for r in range(rd):
        qr = qs[r].contiguous()
        o = torch.empty_like(qr)
        lse = torch.empty(w.H, w.B, L, dtype=torch.float32, device=dev)
        desc = B.attn_desc(S, rd, qr, ks, vs, o=o, cu_seqlens=cu, zigzag_per_sample=True)
        say(w.name, "per-sample backward rank", r)
        B.usp_attn_fwd(qr, ks, vs, o, lse, desc, r)
        d_o = inputs.randn(tuple(qr.shape), 99, "bf16").to(dev)
        dq = torch.empty_like(qr)
        dk = torch.zeros(ks.shape, dtype=torch.float32, device=dev)
        dv = torch.zeros(vs.shape, dtype=torch.float32, device=dev)
        stats = torch.empty(2 * lse.numel(), dtype=torch.float32, device=dev)
        B.usp_attn_bwd(qr, ks, vs, o, d_o, lse, dq, dk, dv, stats, desc, r)
        torch.cuda.synchronize()
        assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
        don = f64(d_o)

        # dQ rows: every piece's edges and random rows
        edges, off = [], 0
        for b, e in zip(cu[:-1], cu[1:]):
            m = (e - b) // (2 * rd)
            edges += [off, off + m - 1, off + m, off + 2 * m - 1]
            off += 2 * m
        rows = sample_rows(L, w.chunk, 16, 80 + r, extra=sorted(set(edges)))
        qp = pos[r][rows]
        gq, _, _ = ob.attention_backward(qn[:, qp], kn, vn, don[:, rows], w.scale, q_pos=qp, k_pos=all_pos,
                                         q_seg_start=ix.segment_start(cu, qp))
        check_grad(f64(dq[:, rows]), gq, "bf16", f"{w.name} per-sample r{r} dq rows")

        # dK, dV: keys of the last three chunks of the two shortest samples
        for n in short:
            b, e = int(cu[n]), int(cu[n + 1])
            m = (e - b) // (2 * rd)
            kp = np.arange(e - 3 * m, e)
            vis_rows = np.nonzero((pos[r] >= kp[0]) & (pos[r] < e))[0]
            if vis_rows.size == 0:
                continue
            vq = pos[r][vis_rows]
            seg = ix.segment_start(cu, vq)
            o_v, lse_v = oa.masked_attention(qn[:, vq], kn, vn, w.scale, q_pos=vq, k_pos=all_pos, q_seg_start=seg)
            do_v = don[:, vis_rows]
            _, gk, gv = ob.ring_step_backward(qn[:, vq], kn[:, kp], vn[:, kp], do_v, lse_v, ob.delta_rows(o_v, do_v),
                                              w.scale, vq, kp, q_seg_start=seg)
            got_k = np.stack([f64(dk[owner[p]][:, local[p]]) for p in kp], axis=1)
            got_v = np.stack([f64(dv[owner[p]][:, local[p]]) for p in kp], axis=1)
            check_grad(got_k, gk, "bf16", f"{w.name} per-sample r{r} dk sample {n}")
            check_grad(got_v, gv, "bf16", f"{w.name} per-sample r{r} dv sample {n}")

        # whole-walk identities: every dS row sums to zero, every softmax row to one
        dk64, dv64 = f64(dk), f64(dv)                                  # (rd, B, L, Hkv, D)
        dk_sum = dk64.sum(axis=(0, 2))
        assert np.all(np.abs(dk_sum) <= 1e-2 * np.abs(dk64).sum(axis=(0, 2))), "sum of dK"
        G = w.H // w.Hkv
        ref = don.reshape(w.B, L, w.Hkv, G, w.D).sum(axis=(1, 3))
        scale_v = np.abs(don).reshape(w.B, L, w.Hkv, G, w.D).sum(axis=(1, 3))
        assert np.all(np.abs(dv64.sum(axis=(0, 2)) - ref) <= 1e-3 * scale_v), "sum of dV"


def test_backward_key_tile_groups_match_the_ring_steps():
    """A 49900-row share at cp = 4 (2 query heads on 1 KV head, D = 128): its
    195 key tiles x 4 blocks exceed the dK/dV pass's table of work items, so
    the walk's entries group two consecutive key tiles (the last group one
    tile short).  Each ring step alone orders its 195 tiles one by one.  Each
    dK/dV workgroup owns its keys and accumulates in the same order either
    way, so the walk's dK and dV must be bitwise those of the four steps
    summed (a tile lost or doubled by the grouping would show); dQ (bf16,
    from registers) against the steps' fp32 sum at the gradient bar."""
    dev = device()
    Bn, H, Hkv, D, cp, L = 1, 2, 1, 128, 4, 49900
    S = cp * L
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, "bf16", 990)
    do = inputs.randn((Bn, S, H, D), 994, "bf16")
    qs, ks, vs, dos = (shares(x.to(dev), cp) for x in (q, k, v, do))
    r = 0
    o = torch.empty_like(qs[r])
    lse = torch.empty((H, Bn, L), dtype=torch.float32, device=dev)
    desc = B.attn_desc(S, cp, qs[r], ks, vs, o=o)
    say("key tile groups: forward", S)
    B.usp_attn_fwd(qs[r], ks, vs, o, lse, desc, r)
    stats = torch.empty(2 * H * Bn * L, dtype=torch.float32, device=dev)
    dq = torch.empty_like(qs[r])
    dk = torch.zeros(ks.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(vs.shape, dtype=torch.float32, device=dev)
    say("key tile groups: walk backward")
    B.usp_attn_bwd(qs[r], ks, vs, o, dos[r], lse, dq, dk, dv, stats, desc, r)
    stats2 = torch.empty_like(stats)
    B.usp_attn_bwd_prep(o, dos[r], lse, stats2, desc, r)
    dq_acc = torch.zeros((H, Bn, L, D), dtype=torch.float32, device=dev)
    dk2, dv2 = torch.zeros_like(dk), torch.zeros_like(dv)
    for t in range(cp):
        say("key tile groups: step", t)
        B.usp_ring_attn_step_bwd(qs[r], ks, vs, dos[r], stats2, dq_acc, dk2, dv2, desc, r, t)
    torch.cuda.synchronize()
    assert torch.equal(stats, stats2)
    assert bool((dk.abs().sum(dim=(1, 2, 3, 4)) > 0).all()), "a block got no dK"
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    check_grad(f64(dq), np.transpose(f64(dq_acc), (1, 2, 0, 3)), "bf16", "dq walk vs steps")
