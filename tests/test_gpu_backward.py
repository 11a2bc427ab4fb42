"""GPU parity of the backward entry points against the CPU oracle, through the
C ABI: the per-row statistics, the ring walk per rank and for every rank, the
ring steps one at a time, and the forward -> backward pipeline.

The oracle's gradients come from the exact (float64) forward of the same
bf16/fp32 inputs; the kernels get O and lse as the forward would hand them
over (O rounded to the input dtype, lse in fp32).
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import backward as ob
from oracle import index as ix
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from tests.gpu_common import check_grad, device, f64, guarded, say, shares

pytestmark = pytest.mark.gpu

BWD_CASES = {  # name: B, S, H, Hkv, D, cp, causal, cu_seqlens, dtype, layout
    "tiny_fp32_workload": (1, 256, 2, 2, 64, 4, True, None, "fp32", "bshd"),
    "fp32_gqa_ragged_headmajor": (2, 200, 4, 2, 128, 2, True, None, "fp32", "hbsd"),
    "fp32_packed_cp3": (1, 96, 2, 2, 64, 3, True, [0, 5, 40, 96], "fp32", "bshd"),
    "bf16_aligned": (1, 1024, 4, 4, 128, 4, True, None, "bf16", "bshd"),
    "bf16_ragged_gqa_b2": (2, 1000, 4, 2, 64, 4, True, None, "bf16", "bshd"),
    "bf16_cp3_headmajor_gqa": (1, 1536, 8, 2, 128, 3, True, None, "bf16", "hbsd"),
    "bf16_noncausal": (1, 520, 2, 1, 128, 2, False, None, "bf16", "bshd"),
    "bf16_packed": (1, 2048, 4, 2, 128, 4, True, [0, 100, 101, 700, 1990, 2048], "bf16", "bshd"),
    "bf16_tiny_rows": (1, 16, 2, 2, 128, 4, True, None, "bf16", "bshd"),
    "bf16_d64_mqa": (1, 2048, 4, 1, 64, 2, True, None, "bf16", "hbsd"),
}


def _prepare(name):
    Bn, S, H, Hkv, D, cp, causal, cu, dt, layout = BWD_CASES[name]
    dev = device()
    seed = 500 + sorted(BWD_CASES).index(name) * 10
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, dt, seed)
    do = inputs.randn((Bn, S, H, D), seed + 4, dt)
    scale = D ** -0.5
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    o, lse = oa.attention_full(qn, kn, vn, scale, causal, cu)          # global order
    delta = ob.delta_rows(o, don)
    pos = [ix.zigzag_share_positions(S, cp, r) for r in range(cp)]
    kb, vb = [kn[:, p] for p in pos], [vn[:, p] for p in pos]
    refs = [ob.ring_backward_rank(qn[:, pos[r]], pos[r], kb, vb, pos, don[:, pos[r]], lse[:, :, pos[r]],
                                  delta[:, :, pos[r]], r, scale, causal, cu) for r in range(cp)]
    tdt = q.dtype
    o_t = torch.from_numpy(o).to(tdt)                                   # O as the forward hands it over
    sh = [shares(x.to(dev), cp) for x in (q, k, v, do, o_t)]            # (cp, B, L, H, D)
    if layout == "hbsd":
        sh = [t.permute(0, 3, 1, 2, 4).contiguous() for t in sh]
    lse_sh = torch.from_numpy(np.stack([lse[:, :, p] for p in pos])).float().contiguous().to(dev)  # (cp, H, B, L)
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    return dict(Bn=Bn, S=S, H=H, Hkv=Hkv, D=D, cp=cp, causal=causal, cu=cu, cu_t=cu_t, dt=dt, layout=layout,
                qs=sh[0], ks=sh[1], vs=sh[2], dos=sh[3], os=sh[4], lse=lse_sh, lse64=lse, delta=delta, pos=pos,
                refs=refs, dev=dev, L=S // cp, scale=scale, qn=qn, don=don)


def _bshd(P, x):
    """A GPU tensor of one rank / block in the case's layout -> numpy (B, L, H, D)."""
    x = f64(x)
    return np.transpose(x, (1, 2, 0, 3)) if P["layout"] == "hbsd" else x


def _desc(P, r=None):
    all_ranks = r is None
    q = P["qs"] if all_ranks else P["qs"][r]
    o = P["os"] if all_ranks else P["os"][r]
    return B.attn_desc(P["S"], P["cp"], q, P["ks"], P["vs"], o=o, layout=P["layout"], causal=P["causal"],
                       cu_seqlens=P["cu_t"], all_ranks=all_ranks)


def _grads_like(P):
    dk, ok1 = guarded(tuple(P["ks"].shape), torch.float32, P["dev"])
    dv, ok2 = guarded(tuple(P["vs"].shape), torch.float32, P["dev"])
    return dk, dv, lambda: ok1() and ok2()


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_backward_stats(name):
    P = _prepare(name)
    cp, H, Bn, L = P["cp"], P["H"], P["Bn"], P["L"]
    for r in (0, cp - 1):
        say("bwd prep", name, "rank", r)
        stats, ok = guarded((2 * H * Bn * L,), torch.float32, P["dev"])
        B.usp_attn_bwd_prep(P["os"][r], P["dos"][r], P["lse"][r], stats, _desc(P, r), r)
        torch.cuda.synchronize()
        assert ok()
        st = f64(stats).reshape(2, H, Bn, L)
        # delta of the rounded O the kernel reads: the products are exact, only the fp32 sum rounds
        o_r, do_r = _bshd(P, P["os"][r]), _bshd(P, P["dos"][r])
        terms = np.transpose(o_r * do_r, (2, 0, 1, 3))
        exact = terms.sum(-1)
        assert np.all(np.abs(st[0] - exact) <= 1e-6 * np.abs(terms).sum(-1) + 1e-30), name
        lse2 = f64(P["lse"][r]) * np.log2(np.e)
        bad = np.abs(st[1] - lse2) > 4 * np.spacing(np.abs(lse2).astype(np.float32))
        assert not bad.any(), (name, int(bad.sum()))


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_backward_walk_per_rank_and_all_ranks(name):
    P = _prepare(name)
    cp, H, Bn, L, dev = P["cp"], P["H"], P["Bn"], P["L"], P["dev"]
    dt = P["dt"]
    for r in range(cp):
        say("bwd walk", name, "rank", r)
        dq, ok_q = guarded(tuple(P["qs"][r].shape), P["qs"].dtype, dev)
        dk, dv, ok_kv = _grads_like(P)
        stats = torch.empty(2 * H * Bn * L, dtype=torch.float32, device=dev)
        B.usp_attn_bwd(P["qs"][r], P["ks"], P["vs"], P["os"][r], P["dos"][r], P["lse"][r], dq, dk, dv, stats,
                       _desc(P, r), r)
        torch.cuda.synchronize()
        assert ok_q() and ok_kv()
        dq_ref, dk_ref, dv_ref = P["refs"][r]
        worst = [check_grad(_bshd(P, dq), dq_ref, dt, f"{name} r{r} dq")]
        for j in range(cp):
            worst.append(check_grad(_bshd(P, dk[j]), dk_ref[j], dt, f"{name} r{r} dk[{j}]"))
            worst.append(check_grad(_bshd(P, dv[j]), dv_ref[j], dt, f"{name} r{r} dv[{j}]"))
        say("bwd walk", name, "rank", r, "worst norm %.2e max %.2e" % (max(w["norm"] for w in worst),
                                                                      max(w["max"] for w in worst)))
    say("bwd walk all ranks", name)
    dq, ok_q = guarded(tuple(P["qs"].shape), P["qs"].dtype, dev)
    dk, dv, ok_kv = _grads_like(P)
    stats = torch.empty(2 * cp * H * Bn * L, dtype=torch.float32, device=dev)
    B.usp_attn_bwd(P["qs"], P["ks"], P["vs"], P["os"], P["dos"], P["lse"], dq, dk, dv, stats, _desc(P), -1)
    torch.cuda.synchronize()
    assert ok_q() and ok_kv()
    for r in range(cp):
        check_grad(_bshd(P, dq[r]), P["refs"][r][0], dt, f"{name} all dq[{r}]")
    for j in range(cp):
        check_grad(_bshd(P, dk[j]), sum(P["refs"][r][1][j] for r in range(cp)), dt, f"{name} all dk[{j}]")
        check_grad(_bshd(P, dv[j]), sum(P["refs"][r][2][j] for r in range(cp)), dt, f"{name} all dv[{j}]")


@pytest.mark.parametrize("name", ["tiny_fp32_workload", "fp32_packed_cp3", "bf16_aligned", "bf16_ragged_gqa_b2",
                                  "bf16_cp3_headmajor_gqa", "bf16_packed", "bf16_noncausal"])
def test_backward_steps(name):
    """Each ring step's contribution alone, and their sum, against the oracle's
    ring step on the same block."""
    P = _prepare(name)
    cp, H, Bn, L, D, dev, dt = P["cp"], P["H"], P["Bn"], P["L"], P["D"], P["dev"], P["dt"]
    pos = P["pos"]
    for r in sorted({0, cp - 1}):
        desc = _desc(P, r)
        stats = torch.empty(2 * H * Bn * L, dtype=torch.float32, device=dev)
        B.usp_attn_bwd_prep(P["os"][r], P["dos"][r], P["lse"][r], stats, desc, r)
        dq_acc, ok_q = guarded((H, Bn, L, D), torch.float32, dev)
        dk, dv, ok_kv = _grads_like(P)
        seg = None if P["cu"] is None else ix.segment_start(P["cu"], pos[r])
        for t in range(cp):
            j = ix.ring_kv_block(r, t, cp)
            say("bwd step", name, "rank", r, "step", t)
            before = (dq_acc.clone(), dk[j].clone(), dv[j].clone())
            B.usp_ring_attn_step_bwd(P["qs"][r], P["ks"], P["vs"], P["dos"][r], stats, dq_acc, dk, dv, desc, r, t)
            torch.cuda.synchronize()
            assert ok_q() and ok_kv()
            kb, vb = _bshd(P, P["ks"][j]), _bshd(P, P["vs"][j])
            gq, gk, gv = ob.ring_step_backward(P["qn"][:, pos[r]], kb, vb, P["don"][:, pos[r]], P["lse64"][:, :, pos[r]],
                                               P["delta"][:, :, pos[r]], P["scale"], pos[r], pos[j], P["causal"], seg)
            check_grad(np.transpose(f64(dq_acc - before[0]), (1, 2, 0, 3)), gq, dt, f"{name} r{r} t{t} dq")
            check_grad(_bshd(P, dk[j] - before[1]), gk, dt, f"{name} r{r} t{t} dk")
            check_grad(_bshd(P, dv[j] - before[2]), gv, dt, f"{name} r{r} t{t} dv")
        check_grad(np.transpose(f64(dq_acc), (1, 2, 0, 3)), P["refs"][r][0], dt, f"{name} r{r} steps dq")


def test_forward_then_backward_pipeline():
    """GPU forward (O, lse) feeding the GPU backward for every rank, against
    the oracle's gradients of the whole sequence."""
    dev = device()
    Bn, S, H, Hkv, D, cp = 1, 2048, 8, 2, 128, 4
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, "bf16", 777)
    do = inputs.randn((Bn, S, H, D), 781, "bf16")
    scale = D ** -0.5
    qs, ks, vs, dos = (shares(x.to(dev), cp) for x in (q, k, v, do))
    L = S // cp
    o = torch.empty_like(qs)
    lse = torch.empty(cp, H, Bn, L, dtype=torch.float32, device=dev)
    desc = B.attn_desc(S, cp, qs, ks, vs, o=o, all_ranks=True)
    say("pipeline forward")
    B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
    dq = torch.empty_like(qs)
    dk = torch.zeros(ks.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(vs.shape, dtype=torch.float32, device=dev)
    stats = torch.empty(2 * cp * H * Bn * L, dtype=torch.float32, device=dev)
    say("pipeline backward")
    B.usp_attn_bwd(qs, ks, vs, o, dos, lse, dq, dk, dv, stats, desc, -1)
    torch.cuda.synchronize()
    gq, gk, gv = ob.attention_backward_full(f64(q), f64(k), f64(v), f64(do), scale)
    for r in range(cp):
        p = ix.zigzag_share_positions(S, cp, r)
        check_grad(f64(dq[r]), gq[:, p], "bf16", f"pipeline dq[{r}]")
        check_grad(f64(dk[r]), gk[:, p], "bf16", f"pipeline dk[{r}]")
        check_grad(f64(dv[r]), gv[:, p], "bf16", f"pipeline dv[{r}]")
