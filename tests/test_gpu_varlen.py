"""GPU parity of the per-sample zigzag split (Algorithm 2 applied to every
packed sample): the extract in every mode (bit-exact), ring steps and walks,
the backward, and the one-GPU share pipeline, against the oracle on the same
positions."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import backward as ob
from oracle import index as ix
from oracle import usp as ou
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from sequence_ring_attention_amd.pipeline import OneGpuShare
from tests.gpu_common import bits, check_close, check_grad, device, f64, guarded, say

pytestmark = pytest.mark.gpu


def ps_positions(cu, cp):
    return [ix.zigzag_per_sample_positions(cu, cp, r) for r in range(cp)]


def ps_shares(X, cu, cp):
    """(B, S, H, D) -> (cp, B, S/cp, H, D): every rank's per-sample share,
    gathered with the oracle's positions."""
    idx = torch.from_numpy(np.concatenate(ps_positions(cu, cp))).to(X.device)
    g = X.index_select(1, idx)
    return g.view(X.shape[0], cp, X.shape[1] // cp, *X.shape[2:]).transpose(0, 1).contiguous()


# ------------------------------------------------------------------ extract --

EXTRACT_CASES = [  # B, S, H, D, rd, ud, cu, dtype
    (1, 128, 4, 64, 4, 2, [0, 16, 24, 80, 128], "bf16"),
    (2, 96, 2, 8, 3, 1, [0, 6, 60, 66, 96], "fp32"),
    (1, 256, 8, 128, 2, 4, [0, 256], "bf16"),
    (1, 64, 1, 8, 1, 2, [0, 2, 10, 64], "bf16"),
]


@pytest.mark.parametrize("case", EXTRACT_CASES)
def test_zigzag_varlen_extract_bitexact(case):
    Bn, S, H, D, rd, ud, cu, dt = case
    dev = device()
    x = inputs.randn((Bn, S, H, D), 41, dt)
    xd = x.to(dev)
    T = S // (rd * ud)
    ref = np.stack([np.stack([bits(x)[:, ix.zigzag_per_sample_local_positions(cu, rd, ud, r, u)]
                              for u in range(ud)]) for r in range(rd)])      # (rd, ud, B, T, H, D)
    say("varlen extract", case)
    out, ok = guarded((rd, ud, Bn, T, H, D), x.dtype, dev)
    B.usp_zigzag_extract_varlen(xd, out, rd, ud, -1, -1, cu)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(out), ref)
    for r in range(rd):
        grp, ok = guarded((ud, Bn, T, H, D), x.dtype, dev)
        B.usp_zigzag_extract_varlen(xd, grp, rd, ud, r, -1, cu)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(grp), ref[r])
        for u in range(ud):
            one, ok = guarded((Bn, T, H, D), x.dtype, dev)
            B.usp_zigzag_extract_varlen(xd, one, rd, ud, r, u, cu)
            torch.cuda.synchronize()
            assert ok() and np.array_equal(bits(one), ref[r, u])
    back, ok = guarded((Bn, S, H, D), x.dtype, dev)
    B.usp_zigzag_extract_varlen(out, back, rd, ud, -1, -1, cu, inverse=True)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(back), bits(x))
    if len(cu) == 2:   # one sample: the same split as Algorithm 2 on the whole sequence
        stream = torch.empty_like(out)
        B.usp_zigzag_extract(xd, stream, rd, ud, -1, -1)
        torch.cuda.synchronize()
        assert torch.equal(stream, out)


# ---------------------------------------------------------------- attention --

ATTN_CASES = {  # name: B, S, H, Hkv, D, cp, cu, dtype
    "bf16_cp4_gqa": (1, 2048, 4, 2, 128, 4, [0, 64, 72, 512, 1024, 1032, 2048], "bf16"),
    "bf16_cp3_d64_mqa_b2": (2, 1536, 4, 1, 64, 3, [0, 6, 600, 606, 1536], "bf16"),
    "fp32_cp2": (1, 96, 2, 2, 64, 2, [0, 4, 28, 96], "fp32"),
    # 108 samples: pieces of 1, 65, 128 and 129 rows among many short ones,
    # so the query tiles cut at pieces take every shape
    "bf16_cp2_108_samples": (1, None, 2, 1, 64, 2, "many", "bf16"),
    # D = 128 with pieces of 257, 129, 513 and 1 rows: query tiles cut at
    # pieces longer than one 128-row tile, in the walk and the dQ pass
    "bf16_cp2_d128_long_pieces": (1, 3600, 4, 2, 128, 2, [0, 1028, 1544, 3596, 3600], "bf16"),
}


def _many_samples_cu():
    lens = [4, 512, 516, 260, 8, 132, 4, 1028] + [4 * (1 + (7 * i) % 23) for i in range(100)]
    return [0] + np.cumsum(lens).tolist()


def _prepare(name):
    Bn, S, H, Hkv, D, cp, cu, dt = ATTN_CASES[name]
    if cu == "many":
        cu = _many_samples_cu()
        S = cu[-1]
    dev = device()
    seed = 800 + sorted(ATTN_CASES).index(name) * 10
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, dt, seed)
    pos = ps_positions(cu, cp)
    return dict(Bn=Bn, S=S, H=H, Hkv=Hkv, D=D, cp=cp, cu=cu, dt=dt, dev=dev, q=q, k=k, v=v, pos=pos,
                qs=ps_shares(q.to(dev), cu, cp), ks=ps_shares(k.to(dev), cu, cp), vs=ps_shares(v.to(dev), cu, cp),
                qn=f64(q), kn=f64(k), vn=f64(v), L=S // cp, scale=D ** -0.5)


def _oracle_rank(P, r):
    kb = [P["kn"][:, p] for p in P["pos"]]
    vb = [P["vn"][:, p] for p in P["pos"]]
    return ou.ring_attention_rank(P["qn"][:, P["pos"][r]], P["pos"][r], kb, vb, P["pos"], r, P["scale"], True,
                                  P["cu"], return_partials=True)


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_per_sample_steps_and_walks(name):
    P = _prepare(name)
    cp, H, Bn, L, D, dev = P["cp"], P["H"], P["Bn"], P["L"], P["D"], P["dev"]
    tdt = torch.float32 if P["dt"] == "fp32" else torch.bfloat16
    for r in range(cp):
        o_ref, lse_ref, parts = _oracle_rank(P, r)
        desc = B.attn_desc(P["S"], cp, P["qs"][r], P["ks"], P["vs"], cu_seqlens=P["cu"], zigzag_per_sample=True)
        for t in range(cp):
            say("per-sample step", name, r, t)
            o_st = torch.empty(H, Bn, L, D, dtype=torch.float32, device=dev)
            l_st = torch.empty(H, Bn, L, dtype=torch.float32, device=dev)
            B.usp_ring_attn_step_fwd(P["qs"][r], P["ks"], P["vs"], o_st, l_st, desc, r, t)
            torch.cuda.synchronize()
            check_close(f64(o_st), f64(l_st), parts[t][0], parts[t][1], P["dt"], f"{name} r{r} t{t}")
        say("per-sample walk", name, r)
        o, ok = guarded((Bn, L, H, D), tdt, dev)
        lse = torch.empty(H, Bn, L, dtype=torch.float32, device=dev)
        desc = B.attn_desc(P["S"], cp, P["qs"][r], P["ks"], P["vs"], o=o, cu_seqlens=P["cu"],
                           zigzag_per_sample=True)
        B.usp_attn_fwd(P["qs"][r], P["ks"], P["vs"], o, lse, desc, r)
        torch.cuda.synchronize()
        assert ok()
        check_close(f64(o), f64(lse), o_ref, lse_ref, P["dt"], f"{name} walk r{r}", out_bf16=P["dt"] == "bf16")


def test_one_sample_per_sample_split_matches_the_stream_path_bitwise():
    """With one sample the per-sample map gives the stream split's positions,
    so both paths of the kernels produce identical bits."""
    dev = device()
    S, H, D, cp = 1024, 4, 128, 4
    q, k, v = inputs.qkv(1, S, H, 2, D, "bf16", 850)
    qs, ks, vs = (ps_shares(x.to(dev), [0, S], cp) for x in (q, k, v))
    outs = []
    for per_sample in (False, True):
        o = torch.empty_like(qs)
        lse = torch.empty(cp, H, 1, S // cp, dtype=torch.float32, device=dev)
        desc = B.attn_desc(S, cp, qs, ks, vs, o=o, cu_seqlens=[0, S], zigzag_per_sample=per_sample,
                           all_ranks=True)
        say("one sample, per_sample =", per_sample)
        B.usp_attn_fwd(qs, ks, vs, o, lse, desc, -1)
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_per_sample_backward(name):
    P = _prepare(name)
    cp, H, Bn, L, D, dev, dt = P["cp"], P["H"], P["Bn"], P["L"], P["D"], P["dev"], P["dt"]
    do = inputs.randn((Bn, P["S"], H, D), 859, dt)
    don = f64(do)
    o, lse = oa.attention_full(P["qn"], P["kn"], P["vn"], P["scale"], True, P["cu"])
    delta = ob.delta_rows(o, don)
    pos = P["pos"]
    kb, vb = [P["kn"][:, p] for p in pos], [P["vn"][:, p] for p in pos]
    refs = [ob.ring_backward_rank(P["qn"][:, pos[r]], pos[r], kb, vb, pos, don[:, pos[r]], lse[:, :, pos[r]],
                                  delta[:, :, pos[r]], r, P["scale"], True, P["cu"]) for r in range(cp)]
    o_t = ps_shares(torch.from_numpy(o).to(P["q"].dtype).to(dev), P["cu"], cp)
    do_t = ps_shares(do.to(dev), P["cu"], cp)
    lse_t = torch.from_numpy(np.stack([lse[:, :, p] for p in pos])).float().contiguous().to(dev)
    say("per-sample backward all ranks", name)
    dq = torch.empty_like(P["qs"])
    dk = torch.zeros(P["ks"].shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(P["vs"].shape, dtype=torch.float32, device=dev)
    stats = torch.empty(2 * cp * H * Bn * L, dtype=torch.float32, device=dev)
    desc = B.attn_desc(P["S"], cp, P["qs"], P["ks"], P["vs"], o=o_t, cu_seqlens=P["cu"], zigzag_per_sample=True,
                       all_ranks=True)
    B.usp_attn_bwd(P["qs"], P["ks"], P["vs"], o_t, do_t, lse_t, dq, dk, dv, stats, desc, -1)
    torch.cuda.synchronize()
    for r in range(cp):
        check_grad(f64(dq[r]), refs[r][0], dt, f"{name} dq[{r}]")
    for j in range(cp):
        check_grad(f64(dk[j]), sum(refs[r][1][j] for r in range(cp)), dt, f"{name} dk[{j}]")
        check_grad(f64(dv[j]), sum(refs[r][2][j] for r in range(cp)), dt, f"{name} dv[{j}]")


def test_per_sample_usp_pipeline():
    """OneGpuShare with the per-sample split on a 2 x 2 grid: extract, layout,
    walk, inverse layout; every share against the oracle's USP with the same
    split."""
    dev = device()
    Bn, S, H, Hkv, D, rd, ud = 1, 2048, 8, 4, 128, 2, 2
    cu = [0, 100 * 4, 104 * 4, 420 * 4, 512 * 4]
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, "bf16", 870)
    o_ref, lse_ref = ou.usp_attention(f64(q), f64(k), f64(v), rd, ud, D ** -0.5, True, cu, per_sample=True)
    T = S // (rd * ud)
    for r in range(rd):
        for u in range(ud):
            say("per-sample pipeline share", r, u)
            share = OneGpuShare(q.to(dev), k.to(dev), v.to(dev), rd, ud, r, u, cu_seqlens=cu, per_sample=True)
            share.prepare_peers()
            out = share.step()
            torch.cuda.synchronize()
            pos = ix.zigzag_per_sample_local_positions(cu, rd, ud, r, u)
            hb = H // ud
            lse = f64(share.lse[u][:, :, u * T:(u + 1) * T])
            check_close(f64(out), lse, o_ref[:, pos], lse_ref[u * hb:(u + 1) * hb][:, :, pos], "bf16",
                        f"pipeline ({r},{u})", out_bf16=True)
