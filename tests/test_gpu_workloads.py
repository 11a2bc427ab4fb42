"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times, on sampled rows the oracle computes one by one (chunk
edges, sample boundaries and a seeded random set), plus properties that hold
at any size (finite outputs, canaries intact)."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as ix
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from sequence_ring_attention_amd.pipeline import OneGpuShare
from tests.gpu_common import check_close, device, f64, sample_rows, say, shares

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _oracle_rows(qn, kn, vn, q_pos, scale, cu=None):
    seg = None if cu is None else ix.segment_start(cu, q_pos)
    return oa.masked_attention(qn[:, q_pos], kn, vn, scale, q_pos=q_pos, causal=True, q_seg_start=seg)


def _load(w):
    q, k, v = inputs.workload_qkv(w)
    return q, k, v, f64(k), f64(v)


def test_causal_mha_s8k_all_ranks_one_launch():
    w = W["causal_mha_s8k_cp4"]
    dev = device()
    q, k, v, kn, vn = _load(w)
    qs, ks, vs = shares(q.to(dev), w.rd), shares(k.to(dev), w.rd), shares(v.to(dev), w.rd)
    o = torch.empty_like(qs)
    lse = torch.empty(w.rd, w.H, w.B, w.share, dtype=torch.float32, device=dev)
    desc = B.attn_desc(w.S, w.rd, qs, ks, vs, o=o, all_ranks=True)
    say(w.name, "walk all ranks")
    B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qn = f64(q)
    for r in range(w.rd):
        rows = sample_rows(w.share, w.chunk, 24, 10 + r)
        pos = ix.zigzag_share_positions(w.S, w.rd, r)[rows]
        o_ref, l_ref = _oracle_rows(qn, kn, vn, pos, w.scale)
        check_close(f64(o[r][:, rows]), f64(lse[r][:, :, rows]), o_ref, l_ref, "bf16", f"{w.name} r{r}")


@pytest.mark.parametrize("rank", [0, 7])
def test_causal_gqa_s32k_cp8_rank(rank):
    w = W["causal_gqa_s32k_cp8"]
    dev = device()
    q, k, v, kn, vn = _load(w)
    ks, vs = shares(k.to(dev), w.rd), shares(v.to(dev), w.rd)
    qr = shares(q.to(dev), w.rd)[rank].contiguous()
    o = torch.empty_like(qr)
    lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
    desc = B.attn_desc(w.S, w.rd, qr, ks, vs, o=o)
    say(w.name, "walk rank", rank)
    B.usp_attn_fwd(qr, ks, vs, o, lse, desc, rank)
    # the ring-step path of the same rank: cp partials merged in ring order
    acc = torch.empty(w.H, w.B, w.share, w.D, dtype=torch.float32, device=dev)
    lacc = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
    o_st, l_st = torch.empty_like(acc), torch.empty_like(lacc)
    for t in range(w.rd):
        say(w.name, "step", t)
        B.usp_ring_attn_step_fwd(qr, ks, vs, acc if t == 0 else o_st, lacc if t == 0 else l_st, desc, rank, t)
        if t:
            B.usp_lse_merge(acc, lacc, o_st, l_st)
    # the same steps with the merge fused into the step kernel: bitwise the chain above
    facc = torch.empty_like(acc)
    flacc = torch.full_like(lacc, float("-inf"))
    for t in range(w.rd):
        say(w.name, "merged step", t)
        B.usp_ring_attn_step_fwd_merge(qr, ks, vs, facc, flacc, desc, rank, t)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all() and torch.isfinite(acc).all()
    assert torch.equal(flacc, lacc) and torch.equal(facc, acc)
    rows = sample_rows(w.share, w.chunk, 32, 20 + rank)
    pos = ix.zigzag_share_positions(w.S, w.rd, rank)[rows]
    o_ref, l_ref = _oracle_rows(f64(q), kn, vn, pos, w.scale)
    check_close(f64(o[:, rows]), f64(lse[:, :, rows]), o_ref, l_ref, "bf16", f"{w.name} walk r{rank}")
    check_close(np.transpose(f64(acc[:, :, rows]), (1, 2, 0, 3)), f64(lacc[:, :, rows]), o_ref, l_ref,
                "bf16", f"{w.name} steps+merge r{rank}")


@pytest.mark.parametrize("r,u", [(0, 0), (3, 1)])
def test_usp_hybrid_s128k_one_gpu_share(r, u):
    """The benchmark's workload and calls: OneGpuShare.step on the 2 x 4 grid."""
    w = W["usp_hybrid_s128k_ud2_rd4"]
    dev = device()
    q, k, v, kn, vn = _load(w)
    say(w.name, "share", r, u, "prepare")
    share = OneGpuShare(q.to(dev), k.to(dev), v.to(dev), w.rd, w.ud, r, u)
    share.prepare_peers()
    say(w.name, "share", r, u, "step")
    out = share.step()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(share.lse[u]).all()
    T = w.S // (w.rd * w.ud)
    c = w.chunk
    # shard rows: the chunk edges as they fall in this Ulysses slice, plus random rows
    edge = [l - u * T for l in (0, 1, c - 1, c, c + 1, 2 * c - 1) if 0 <= l - u * T < T]
    rows = sample_rows(T, T // 2, 24, 30 + r, extra=edge)
    pos = ix.zigzag_local_positions(w.S, w.rd, w.ud, r, u)[rows]
    o_ref, l_ref = _oracle_rows(f64(q), kn, vn, pos, w.scale)
    hb = w.H // w.ud
    lse_rows = f64(share.lse[u][:, :, u * T + rows])
    check_close(f64(out[:, rows]), lse_rows, o_ref, l_ref[u * hb:(u + 1) * hb], "bf16",
                f"{w.name} share ({r},{u})")


def test_packed_varlen_s32k_all_ranks():
    w = W["packed_varlen_s32k_cp4"]
    dev = device()
    q, k, v, kn, vn = _load(w)
    cu = inputs.workload_cu_seqlens(w)
    cu_t = torch.from_numpy(cu).to(dev)
    qs, ks, vs = shares(q.to(dev), w.rd), shares(k.to(dev), w.rd), shares(v.to(dev), w.rd)
    qn = f64(q)
    for r in range(w.rd):
        o = torch.empty_like(qs[r])
        lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
        desc = B.attn_desc(w.S, w.rd, qs[r], ks, vs, o=o, cu_seqlens=cu_t)
        say(w.name, "walk rank", r)
        B.usp_attn_fwd(qs[r], ks, vs, o, lse, desc, r)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        share_pos = ix.zigzag_share_positions(w.S, w.rd, r)
        # rows at sample starts and ends that fall in this share
        bnd = set()
        for b in cu[1:-1]:
            for p in (b - 1, b, b + 1):
                hit = np.nonzero(share_pos == p)[0]
                bnd.update(hit.tolist())
        rows = sample_rows(w.share, w.chunk, 24, 40 + r, extra=sorted(bnd))
        o_ref, l_ref = _oracle_rows(qn, kn, vn, share_pos[rows], w.scale, cu)
        check_close(f64(o[:, rows]), f64(lse[:, :, rows]), o_ref, l_ref, "bf16", f"{w.name} r{r}")


def _piece_edges(cu, cp):
    """Local rows of each ring rank's per-sample share at the first and last
    row of each of its pieces: a sample of length n contributes its chunks r
    and 2 cp - 1 - r, m = n / (2 cp) rows each, in sample order."""
    out = []
    for r in range(cp):
        rows, off = [], 0
        for b, e in zip(cu[:-1], cu[1:]):
            m = (e - b) // (2 * cp)
            rows += [off, off + m - 1, off + m, off + 2 * m - 1]
            off += 2 * m
        out.append(sorted(set(rows)))
    return out


def _per_sample_shares(x, w, cu, dev):
    """Every rank's per-sample share (rd, B, S/rd, H, D) by the library's
    extract, as the benchmark makes them."""
    out = torch.empty((w.rd, 1, w.B, w.share) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
    B.usp_zigzag_extract_varlen(x.to(dev), out, w.rd, 1, -1, -1, cu)
    return out[:, 0]


def test_packed_varlen_s32k_per_sample_all_ranks():
    """The per-sample split of the packed 32K workload (lengths rounded to
    multiples of 2 cp), each rank's walk as the benchmark launches it; every
    piece's first and last rows and a seeded random set against the oracle."""
    w = W["packed_varlen_s32k_cp4"]
    dev = device()
    q, k, v, kn, vn = _load(w)
    cu = inputs.workload_cu_seqlens(w, multiple=2 * w.rd)
    say(w.name, "per-sample extract")
    qs, ks, vs = (_per_sample_shares(x, w, cu, dev) for x in (q, k, v))
    pos = [ix.zigzag_per_sample_positions(cu, w.rd, r) for r in range(w.rd)]
    for r in range(w.rd):
        assert torch.equal(qs[r].cpu(), q[:, pos[r]]) and torch.equal(ks[r].cpu(), k[:, pos[r]])
    edges = _piece_edges(cu, w.rd)
    qn = f64(q)
    for r in range(w.rd):
        qr = qs[r].contiguous()
        o = torch.empty_like(qr)
        lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
        desc = B.attn_desc(w.S, w.rd, qr, ks, vs, o=o, cu_seqlens=cu, zigzag_per_sample=True)
        say(w.name, "per-sample walk rank", r)
        B.usp_attn_fwd(qr, ks, vs, o, lse, desc, r)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        rows = sample_rows(w.share, w.chunk, 24, 50 + r, extra=edges[r])
        o_ref, l_ref = _oracle_rows(qn, kn, vn, pos[r][rows], w.scale, cu)
        check_close(f64(o[:, rows]), f64(lse[:, :, rows]), o_ref, l_ref, "bf16", f"{w.name} per-sample r{r}")


def test_usp_hybrid_s128k_share_384_rows():
    """The benchmark's own comparison as a test: 384 seeded rows of the
    share's head-major output (all 16 heads of the Ulysses rank, both
    Ulysses halves of the ring share) after OneGpuShare.step, against the
    oracle over all 131072 keys."""
    w = W["usp_hybrid_s128k_ud2_rd4"]
    r, u = 0, 0
    dev = device()
    q, k, v, kn, vn = _load(w)
    say(w.name, "share", r, u, "384 rows")
    share = OneGpuShare(q.to(dev), k.to(dev), v.to(dev), w.rd, w.ud, r, u)
    share.prepare_peers()
    share.step()
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1234).choice(w.share, size=384, replace=False))
    hb, kb = w.H // w.ud, w.Hkv // w.ud
    rt = torch.from_numpy(rows).to(dev)
    o = np.transpose(f64(share.oh[u].index_select(2, rt)), (1, 2, 0, 3))        # (B, n, hb, D)
    lse = f64(share.lse[u].index_select(2, rt))
    qp = ix.zigzag_share_positions(w.S, w.rd, r)[rows]
    o_ref, l_ref = oa.masked_attention(f64(q[:, :, u * hb:(u + 1) * hb])[:, qp], kn[:, :, u * kb:(u + 1) * kb],
                                       vn[:, :, u * kb:(u + 1) * kb], w.scale, q_pos=qp)
    check_close(o, lse, o_ref, l_ref, "bf16", f"{w.name} share ({r},{u}) 384 rows x {hb} heads")


def test_tiny_fp32_workload_all_ranks():
    w = W["tiny_causal_mha_fp32_s256_cp4"]
    dev = device()
    q, k, v = inputs.workload_qkv(w)
    qs, ks, vs = shares(q.to(dev), w.rd), shares(k.to(dev), w.rd), shares(v.to(dev), w.rd)
    o = torch.empty_like(qs)
    lse = torch.empty(w.rd, w.H, w.B, w.share, dtype=torch.float32, device=dev)
    desc = B.attn_desc(w.S, w.rd, qs, ks, vs, o=o, all_ranks=True)
    say(w.name)
    B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
    torch.cuda.synchronize()
    o_ref, l_ref = oa.attention_full(f64(q), f64(k), f64(v), w.scale)
    for r in range(w.rd):
        p = ix.zigzag_share_positions(w.S, w.rd, r)
        check_close(f64(o[r]), f64(lse[r]), o_ref[:, p], l_ref[:, :, p], "fp32", f"{w.name} r{r}")


@pytest.mark.parametrize("D,Hq,Hkv,c", [(64, 64, 8, 1000), (128, 64, 16, 1100)])
def test_eight_wave_walk_ragged(D, Hq, Hkv, c):
    """Launches large enough for eight-wave workgroups (at least two per CU)
    whose shares do not divide into 256-row query tiles: the walk of every
    rank in one launch and rank 1's ring steps (fp32 partials, merged), on
    sampled rows including the ragged tail, against the oracle."""
    cp = 2
    S = 2 * cp * c
    dev = device()
    q, k, v = inputs.qkv(1, S, Hq, Hkv, D, "bf16", 9300 + D)
    kn, vn, qn = f64(k), f64(v), f64(q)
    qs, ks, vs = shares(q.to(dev), cp), shares(k.to(dev), cp), shares(v.to(dev), cp)
    L = S // cp
    o = torch.empty_like(qs)
    lse = torch.empty(cp, Hq, 1, L, dtype=torch.float32, device=dev)
    desc = B.attn_desc(S, cp, qs, ks, vs, o=o, all_ranks=True)
    say("eight-wave walk", D, Hq, Hkv, c)
    B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
    r = 1
    qr = qs[r].contiguous()
    d1 = B.attn_desc(S, cp, qr, ks, vs)
    acc = torch.empty(Hq, 1, L, D, dtype=torch.float32, device=dev)
    lacc = torch.empty(Hq, 1, L, dtype=torch.float32, device=dev)
    o_st, l_st = torch.empty_like(acc), torch.empty_like(lacc)
    for t in range(cp):
        B.usp_ring_attn_step_fwd(qr, ks, vs, acc if t == 0 else o_st, lacc if t == 0 else l_st, d1, r, t)
        if t:
            B.usp_lse_merge(acc, lacc, o_st, l_st)
    torch.cuda.synchronize()
    tail = list(range(L - 210, L))   # the last, partial 256-row tile and the one before
    for rr in range(cp):
        rows = sample_rows(L, c, 24, 60 + rr, extra=tail[::7] + [L - 1])
        pos = ix.zigzag_share_positions(S, cp, rr)[rows]
        o_ref, l_ref = _oracle_rows(qn, kn, vn, pos, D ** -0.5)
        check_close(f64(o[rr][:, rows]), f64(lse[rr][:, :, rows]), o_ref, l_ref, "bf16", f"eight-wave walk D{D} r{rr}")
        if rr == r:
            check_close(np.transpose(f64(acc[:, :, rows]), (1, 2, 0, 3)), f64(lacc[:, :, rows]), o_ref, l_ref, "bf16",
                        f"eight-wave steps D{D} r{rr}")
