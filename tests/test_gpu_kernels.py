"""GPU parity of every entry point against the CPU oracle at small sizes that
span several tiles and ragged tails.  Called through the C ABI (ctypes)."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import index as ix
from oracle import merge as om
from oracle import usp as ou
from sequence_ring_attention_amd import binding as B
from sequence_ring_attention_amd import inputs
from tests.gpu_common import bits, check_close, device, f64, guarded, say, shares

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------- zigzag --

ZZ_CASES = [  # B, S, H, D, rd, ud, dtype
    (1, 96, 4, 64, 3, 2, "bf16"),
    (2, 256, 2, 64, 4, 1, "fp32"),
    (1, 1024, 8, 128, 4, 2, "bf16"),
    (3, 40, 1, 8, 2, 2, "bf16"),       # rows of 16 bytes, odd batch
    (1, 48, 3, 8, 1, 3, "fp32"),       # rd = 1, row of 96 bytes (not a power-of-two vector count)
]


@pytest.mark.parametrize("case", ZZ_CASES)
def test_zigzag_extract_all_modes_bitexact(case):
    Bn, S, H, D, rd, ud, dt = case
    dev = device()
    x = inputs.randn((Bn, S, H, D), 7, dt)
    T = S // (rd * ud)
    xd = x.to(dev)
    ref_all = ix.zigzag_extract_all(bits(x), rd, ud)                 # (rd, ud, B, T, H, D)
    say("zigzag all", case)
    out, ok = guarded((rd, ud, Bn, T, H, D), x.dtype, dev)
    B.usp_zigzag_extract(xd, out, rd, ud, -1, -1)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(out), ref_all)
    for r in range(rd):
        say("zigzag group", case, r)
        grp, ok = guarded((ud, Bn, T, H, D), x.dtype, dev)
        B.usp_zigzag_extract(xd, grp, rd, ud, r, -1)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(grp), ref_all[r])
        for u in range(ud):
            one, ok = guarded((Bn, T, H, D), x.dtype, dev)
            B.usp_zigzag_extract(xd, one, rd, ud, r, u)
            torch.cuda.synchronize()
            assert ok() and np.array_equal(bits(one), ref_all[r, u])
    say("zigzag inverse", case)
    back, ok = guarded((Bn, S, H, D), x.dtype, dev)
    B.usp_zigzag_extract(out, back, rd, ud, -1, -1, inverse=True)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(back), bits(x))
    # inverse of one rank writes only that rank's positions
    part, ok = guarded((Bn, S, H, D), x.dtype, dev, fill=0)
    r, u = rd - 1, ud - 1
    B.usp_zigzag_extract(out[r, u].contiguous(), part, rd, ud, r, u, inverse=True)
    torch.cuda.synchronize()
    pos = ix.zigzag_local_positions(S, rd, ud, r, u)
    exp = np.zeros_like(bits(x))
    exp[:, pos] = bits(x)[:, pos]
    assert ok() and np.array_equal(bits(part), exp)


# ---------------------------------------------------------------- ulysses --

ULY_CASES = [  # N, bs, L, hc, hd, dtype
    (2, 1, 64, 4, 64, "bf16"),
    (4, 2, 96, 8, 128, "bf16"),
    (3, 1, 30, 6, 8, "fp32"),
    (1, 2, 16, 4, 64, "bf16"),         # N = 1: plain (bs,L,hc,hd) -> (hc,bs,L,hd) transpose
    (2, 2, 32, 4, 24, "bf16"),         # 48-byte heads (three vectors): the head-row copy kinds
]


@pytest.mark.parametrize("case", ULY_CASES)
def test_ulysses_layout_bitexact(case):
    N, bs, L, hc, hd, dt = case
    dev = device()
    xs = inputs.randn((N, bs, L // N, hc, hd), 11, dt)
    xd = xs.to(dev)
    shards = [bits(xs[u]) for u in range(N)]
    ref = np.stack([ix.ulysses_fwd(shards, u) for u in range(N)])      # (N, hc/N, bs, L, hd)
    say("ulysses fwd all", case)
    out, ok = guarded((N, hc // N, bs, L, hd), xs.dtype, dev)
    B.usp_ulysses_a2a_layout(xd, out, N, -1)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(out), ref)
    for u in range(N):
        one, ok = guarded((hc // N, bs, L, hd), xs.dtype, dev)
        B.usp_ulysses_a2a_layout(xd, one, N, u)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(one), ref[u])
    say("ulysses inv", case)
    back, ok = guarded((N, bs, L // N, hc, hd), xs.dtype, dev)
    B.usp_ulysses_a2a_layout(out, back, N, -1, inverse=True)
    torch.cuda.synchronize()
    assert ok() and np.array_equal(bits(back), bits(xs))
    ref_inv = [ix.ulysses_inv(list(ref), u) for u in range(N)]
    for u in range(N):
        one, ok = guarded((bs, L // N, hc, hd), xs.dtype, dev)
        B.usp_ulysses_a2a_layout(out, one, N, u, inverse=True)
        torch.cuda.synchronize()
        assert ok() and np.array_equal(bits(one), ref_inv[u])


# ----------------------------------------------------- batched copies (n) --

ZZN_CASES = [  # B, S, D, rd, ud, heads of each tensor, dtype
    (1, 96, 64, 3, 2, (4, 2, 2), "bf16"),
    (2, 256, 64, 4, 1, (2, 1), "fp32"),
    (1, 1024, 128, 4, 2, (8, 2, 2, 2), "bf16"),
    (3, 40, 8, 2, 2, (1, 3, 2), "bf16"),      # rows of 16 and 48 bytes in one launch
]


@pytest.mark.parametrize("case", ZZN_CASES)
def test_zigzag_extract_n_bitexact(case):
    """Several tensors in one launch: each equals the oracle's Algorithm 2
    gather, in every rank mode, and the inverse restores every tensor."""
    Bn, S, D, rd, ud, heads, dt = case
    dev = device()
    T = S // (rd * ud)
    xs = [inputs.randn((Bn, S, H, D), 30 + i, dt) for i, H in enumerate(heads)]
    xds = [x.to(dev) for x in xs]
    refs = [ix.zigzag_extract_all(bits(x), rd, ud) for x in xs]          # (rd, ud, B, T, H, D) each
    say("zigzag_n all", case)
    outs = [guarded((rd, ud, Bn, T, H, D), xs[0].dtype, dev) for H in heads]
    B.usp_zigzag_extract_n(xds, [o for o, _ in outs], rd, ud, -1, -1)
    torch.cuda.synchronize()
    for (o, ok), ref in zip(outs, refs):
        assert ok() and np.array_equal(bits(o), ref)
    for r, u in ((0, -1), (rd - 1, ud - 1)):
        say("zigzag_n ranks", case, r, u)
        shp = (Bn, T) if u >= 0 else (ud, Bn, T)
        part = [guarded((*shp, H, D), xs[0].dtype, dev) for H in heads]
        B.usp_zigzag_extract_n(xds, [o for o, _ in part], rd, ud, r, u)
        torch.cuda.synchronize()
        for (o, ok), ref in zip(part, refs):
            assert ok() and np.array_equal(bits(o), ref[r, u] if u >= 0 else ref[r])
    say("zigzag_n inverse", case)
    backs = [guarded((Bn, S, H, D), xs[0].dtype, dev) for H in heads]
    B.usp_zigzag_extract_n([o for o, _ in outs], [b for b, _ in backs], rd, ud, -1, -1, inverse=True)
    torch.cuda.synchronize()
    for (b, ok), x in zip(backs, xs):
        assert ok() and np.array_equal(bits(b), bits(x))


ULYN_CASES = [  # N, bs, L, heads of each tensor, hd, dtype
    (2, 1, 64, (4, 2, 2), 64, "bf16"),
    (4, 2, 96, (8, 4, 4), 128, "bf16"),
    (3, 1, 30, (6, 3), 8, "fp32"),
    (2, 1, 32, (4, 2), 24, "bf16"),    # 48-byte heads: the head-row copy kinds
]


@pytest.mark.parametrize("case", ULYN_CASES)
def test_ulysses_layout_n_bitexact(case):
    """Q, K and V layouts in one launch, both directions: each equals the
    oracle's AllToAll4D permutation."""
    N, bs, L, heads, hd, dt = case
    dev = device()
    xs = [inputs.randn((N, bs, L // N, hc, hd), 40 + i, dt) for i, hc in enumerate(heads)]
    xds = [x.to(dev) for x in xs]
    refs = [np.stack([ix.ulysses_fwd([bits(x[u]) for u in range(N)], u) for u in range(N)]) for x in xs]
    for u in (-1, N - 1):
        say("ulysses_n fwd", case, u)
        outs = [guarded(((N,) if u < 0 else ()) + (hc // N, bs, L, hd), xs[0].dtype, dev) for hc in heads]
        B.usp_ulysses_a2a_layout_n(xds, [o for o, _ in outs], N, u)
        torch.cuda.synchronize()
        for (o, ok), ref in zip(outs, refs):
            assert ok() and np.array_equal(bits(o), ref if u < 0 else ref[u])
    hm = [torch.from_numpy(ref).view(xs[0].dtype).to(dev) for ref in refs]   # (N, hc/N, bs, L, hd) each
    for u in (-1, 0):
        say("ulysses_n inv", case, u)
        outs = [guarded(((N,) if u < 0 else ()) + (bs, L // N, hc, hd), xs[0].dtype, dev) for hc in heads]
        B.usp_ulysses_a2a_layout_n(hm, [o for o, _ in outs], N, u, inverse=True)
        torch.cuda.synchronize()
        for (o, ok), x, ref in zip(outs, xs, refs):
            exp = bits(x) if u < 0 else ix.ulysses_inv(list(ref), u)
            assert ok() and np.array_equal(bits(o), exp)


# ------------------------------------------------------------------ merge --

@pytest.mark.parametrize("rows,D", [(1000, 128), (77, 64), (5, 4), (33, 96), (300, 256)])
def test_lse_merge(rows, D):
    dev = device()
    g = torch.Generator().manual_seed(rows * 1000 + D)
    o1 = torch.randn(rows, D, generator=g)
    o2 = torch.randn(rows, D, generator=g)
    l1 = torch.randn(rows, generator=g) * 4
    l2 = torch.randn(rows, generator=g) * 4
    l1[::7] = -float("inf")       # empty accumulator rows
    l2[::5] = -float("inf")       # empty step rows (and both, where 7 and 5 meet)
    o1[::7] = 0
    o2[::5] = 0
    l1[3] = l2[3] = 80.0          # large equal lse
    ro, rl = om.lse_merge(o1.double().numpy(), l1.double().numpy(), o2.double().numpy(), l2.double().numpy())
    say("merge", rows, D)
    acc, ok1 = guarded((rows, D), torch.float32, dev)
    acc.copy_(o1.to(dev))
    lacc, ok2 = guarded((rows,), torch.float32, dev)
    lacc.copy_(l1.to(dev))
    B.usp_lse_merge(acc, lacc, o2.to(dev), l2.to(dev))
    torch.cuda.synchronize()
    assert ok1() and ok2()
    # The kernel evaluates the merge in double and rounds once to fp32, so each
    # output is within one fp32 ulp of the exact merge (inputs reach |lse| = 80
    # here, where an absolute 1e-6 bar would be below half an ulp).
    go, gl = f64(acc), f64(lacc)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.all(np.abs(gl[fin] - rl[fin]) <= np.spacing(np.abs(rl[fin]).astype(np.float32)))
    assert np.all(np.abs(go - ro) <= np.spacing(np.maximum(np.abs(ro), 1e-30).astype(np.float32)) * 1.5)
    assert np.all(go[np.isneginf(rl)] == 0)


# -------------------------------------------------------------- attention --

ATTN_CASES = {  # name: B, S, H, Hkv, D, cp, causal, cu_seqlens, dtype, layout
    "tiny_fp32_workload": (1, 256, 2, 2, 64, 4, True, None, "fp32", "bshd"),
    "fp32_gqa_ragged": (2, 200, 4, 2, 128, 2, True, None, "fp32", "hbsd"),
    "bf16_aligned": (1, 1024, 4, 4, 128, 4, True, None, "bf16", "bshd"),
    "bf16_ragged_gqa_b2": (2, 1000, 4, 2, 64, 4, True, None, "bf16", "bshd"),
    "bf16_cp3_headmajor": (1, 1536, 8, 2, 128, 3, True, None, "bf16", "hbsd"),
    "bf16_noncausal": (1, 520, 2, 1, 128, 2, False, None, "bf16", "bshd"),
    "bf16_packed": (1, 2048, 4, 2, 128, 4, True, [0, 100, 101, 700, 1990, 2048], "bf16", "bshd"),
    "bf16_cp1": (1, 384, 2, 2, 64, 1, True, None, "bf16", "bshd"),
    "bf16_d64_mqa": (1, 2048, 4, 1, 64, 2, True, None, "bf16", "hbsd"),
    "bf16_tiny_rows": (1, 16, 2, 2, 128, 4, True, None, "bf16", "bshd"),
    "bf16_one_token_chunks": (1, 8, 2, 1, 128, 4, True, None, "bf16", "bshd"),
    "bf16_b2_headmajor_gqa": (2, 768, 8, 2, 128, 3, True, None, "bf16", "hbsd"),
    "bf16_strided_views": (2, 640, 4, 2, 128, 4, True, None, "bf16", "bshd_padded"),
    "bf16_packed_chunk_edges": (1, 1024, 4, 4, 64, 4, True, [0, 1, 128, 256, 257, 640, 1023, 1024], "bf16", "bshd"),
    "fp32_packed_cp3": (1, 96, 2, 2, 64, 3, True, [0, 5, 40, 96], "fp32", "bshd"),
}


def _prepare(name):
    Bn, S, H, Hkv, D, cp, causal, cu, dt, layout = ATTN_CASES[name]
    dev = device()
    seed = 100 + sorted(ATTN_CASES).index(name) * 10
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, dt, seed)
    qs, ks, vs = shares(q.to(dev), cp), shares(k.to(dev), cp), shares(v.to(dev), cp)   # (cp,B,L,H,D)
    if layout == "hbsd":
        qs, ks, vs = (t.permute(0, 3, 1, 2, 4).contiguous() for t in (qs, ks, vs))
    if layout == "bshd_padded":   # views into wider buffers: head and sequence strides are not the dense ones
        def pad(t):
            big = torch.full(t.shape[:3] + (t.shape[3] + 3, t.shape[4]), float("nan"), dtype=t.dtype, device=t.device)
            big[:, :, :, 1:1 + t.shape[3]] = t
            return big[:, :, :, 1:1 + t.shape[3]]
        qs, ks, vs = pad(qs), pad(ks), pad(vs)
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    pos = [ix.zigzag_share_positions(S, cp, r) for r in range(cp)]
    qn, kn, vn = f64(q), f64(k), f64(v)
    return dict(Bn=Bn, S=S, H=H, Hkv=Hkv, D=D, cp=cp, causal=causal, cu=cu, cu_t=cu_t, dt=dt,
                layout=layout, qs=qs, ks=ks, vs=vs, pos=pos, qn=qn, kn=kn, vn=vn, dev=dev,
                L=S // cp, scale=D ** -0.5)


def _oracle_rank(P, r):
    kb = [P["kn"][:, p] for p in P["pos"]]
    vb = [P["vn"][:, p] for p in P["pos"]]
    return ou.ring_attention_rank(P["qn"][:, P["pos"][r]], P["pos"][r], kb, vb, P["pos"], r, P["scale"],
                                  P["causal"], P["cu"], return_partials=True)


def _to_bshd(P, o):
    """GPU o of one rank in the case's layout -> numpy (B, L, H, D)."""
    o = f64(o)
    return np.transpose(o, (1, 2, 0, 3)) if P["layout"] == "hbsd" else o


def _layout(P):
    return "hbsd" if P["layout"] == "hbsd" else "bshd"


def _out(P, shape, dt, dev):
    """Output buffer (with a canary tail); strided into a wider buffer for the padded layout."""
    if P["layout"] != "bshd_padded":
        return guarded(shape, dt, dev)
    Bn, L, H, D = shape[-4:]
    big, tail_ok = guarded(shape[:-2] + (H + 3, D), dt, dev)

    def ok():  # canary tail and the padding heads around the view both untouched
        return tail_ok() and not big[..., 0, :].any() and not big[..., H + 1:, :].any()
    return big[..., 1:1 + H, :], ok


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_ring_steps_and_merge(name):
    P = _prepare(name)
    dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
    desc = B.attn_desc(P["S"], cp, P["qs"][0], P["ks"], P["vs"], layout=_layout(P), causal=P["causal"],
                       cu_seqlens=P["cu_t"])
    for r in range(cp):
        o_ref, lse_ref, parts = _oracle_rank(P, r)
        acc = lacc = None
        for t in range(cp):
            say("step", name, "rank", r, "step", t)
            o_st, ok1 = guarded((H, Bn, L, D), torch.float32, dev)
            l_st, ok2 = guarded((H, Bn, L), torch.float32, dev)
            B.usp_ring_attn_step_fwd(P["qs"][r], P["ks"], P["vs"], o_st, l_st, desc, r, t)
            torch.cuda.synchronize()
            assert ok1() and ok2()
            check_close(f64(o_st), f64(l_st), parts[t][0], parts[t][1],
                        P["dt"] if P["dt"] == "fp32" else "bf16", f"{name} r{r} t{t}")
            if acc is None:
                acc, lacc = o_st.clone(), l_st.clone()
            else:
                B.usp_lse_merge(acc, lacc, o_st, l_st)
        torch.cuda.synchronize()
        check_close(np.transpose(f64(acc), (1, 2, 0, 3)), f64(lacc), o_ref, lse_ref, P["dt"],
                    f"{name} r{r} merged")


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_ring_steps_merged_in_the_step_kernel(name):
    """usp_ring_attn_step_fwd_merge step after step: bitwise the step-then-
    usp_lse_merge chain on an accumulator starting at (0, -inf), from an
    accumulator whose o starts as NaN (an empty row's o is not read), and
    within the bars of the oracle."""
    P = _prepare(name)
    dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
    desc = B.attn_desc(P["S"], cp, P["qs"][0], P["ks"], P["vs"], layout=_layout(P), causal=P["causal"],
                       cu_seqlens=P["cu_t"])
    for r in range(cp):
        o_ref, lse_ref, _ = _oracle_rank(P, r)
        acc = torch.zeros((H, Bn, L, D), dtype=torch.float32, device=dev)
        lacc = torch.full((H, Bn, L), float("-inf"), dtype=torch.float32, device=dev)
        facc, ok1 = guarded((H, Bn, L, D), torch.float32, dev, fill=float("nan"))
        flacc, ok2 = guarded((H, Bn, L), torch.float32, dev, fill=float("-inf"))
        o_st = torch.empty_like(acc)
        l_st = torch.empty_like(lacc)
        for t in range(cp):
            say("merged step", name, "rank", r, "step", t)
            B.usp_ring_attn_step_fwd(P["qs"][r], P["ks"], P["vs"], o_st, l_st, desc, r, t)
            B.usp_lse_merge(acc, lacc, o_st, l_st)
            B.usp_ring_attn_step_fwd_merge(P["qs"][r], P["ks"], P["vs"], facc, flacc, desc, r, t)
        torch.cuda.synchronize()
        assert ok1() and ok2()
        assert np.array_equal(bits(flacc), bits(lacc)), f"{name} r{r} lse"
        live = torch.isfinite(lacc)
        assert np.array_equal(bits(facc[live]), bits(acc[live])), f"{name} r{r} o"
        check_close(np.transpose(f64(facc), (1, 2, 0, 3)), f64(flacc), o_ref, lse_ref, P["dt"],
                    f"{name} r{r} merged in the step kernel")


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_ring_walk_per_rank_and_all_ranks(name):
    P = _prepare(name)
    dev, cp, H, Bn, L, D = P["dev"], P["cp"], P["H"], P["Bn"], P["L"], P["D"]
    dt = torch.float32 if P["dt"] == "fp32" else torch.bfloat16
    refs = [_oracle_rank(P, r) for r in range(cp)]
    oshape = (H, Bn, L, D) if P["layout"] == "hbsd" else (Bn, L, H, D)
    for r in range(cp):
        say("walk", name, "rank", r)
        o, ok1 = _out(P, oshape, dt, dev)
        lse, ok2 = guarded((H, Bn, L), torch.float32, dev)
        desc = B.attn_desc(P["S"], cp, P["qs"][r], P["ks"], P["vs"], o=o, layout=_layout(P),
                           causal=P["causal"], cu_seqlens=P["cu_t"])
        B.usp_attn_fwd(P["qs"][r], P["ks"], P["vs"], o, lse, desc, r)
        torch.cuda.synchronize()
        assert ok1() and ok2()
        check_close(_to_bshd(P, o), f64(lse), refs[r][0], refs[r][1], P["dt"], f"{name} walk r{r}",
                    out_bf16=P["dt"] == "bf16")
    say("walk all ranks", name)
    o_all, ok1 = _out(P, (cp, *oshape), dt, dev)
    lse_all, ok2 = guarded((cp, H, Bn, L), torch.float32, dev)
    desc = B.attn_desc(P["S"], cp, P["qs"], P["ks"], P["vs"], o=o_all, layout=_layout(P),
                       causal=P["causal"], cu_seqlens=P["cu_t"], all_ranks=True)
    B.usp_attn_fwd(P["qs"], P["ks"], P["vs"], o_all, lse_all, desc, -1)
    torch.cuda.synchronize()
    assert ok1() and ok2()
    for r in range(cp):
        check_close(_to_bshd(P, o_all[r]), f64(lse_all[r]), refs[r][0], refs[r][1], P["dt"],
                    f"{name} all-ranks r{r}", out_bf16=P["dt"] == "bf16")


def test_first_row_is_exactly_v0():
    """Position 0 sees only itself: o = v_0 exactly (after bf16 rounding of an
    exact value) and lse = scale * q0.k0."""
    dev = device()
    S, H, D, cp = 512, 2, 128, 4
    q, k, v = inputs.qkv(1, S, H, H, D, "bf16", 900)
    qs, ks, vs = shares(q.to(dev), cp), shares(k.to(dev), cp), shares(v.to(dev), cp)
    o = torch.empty(1, S // cp, H, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(H, 1, S // cp, dtype=torch.float32, device=dev)
    desc = B.attn_desc(S, cp, qs[0], ks, vs, o=o)
    say("first row", S)
    B.usp_attn_fwd(qs[0], ks, vs, o, lse, desc, 0)
    torch.cuda.synchronize()
    assert torch.equal(o[0, 0].cpu(), v[0, 0])
    exp = (q[0, 0].double() * k[0, 0].double()).sum(-1) * D ** -0.5
    assert np.allclose(f64(lse[:, 0, 0]), exp.numpy(), atol=1e-4)


# ---------------------------------------------------------------- pipeline --

def test_usp_pipeline_small():
    """zigzag -> Ulysses fwd (Q, K, V) -> ring walk -> Ulysses inv -> zigzag
    inverse, on a 2 x 2 virtual grid, against one-shot attention."""
    dev = device()
    Bn, S, H, Hkv, D, rd, ud = 1, 2048, 8, 4, 128, 2, 2
    q, k, v = inputs.qkv(Bn, S, H, Hkv, D, "bf16", 321)
    T, L = S // (rd * ud), S // rd
    o_ref, lse_ref = oa.attention_full(f64(q), f64(k), f64(v), D ** -0.5)

    def to_heads(X, Hx):
        z = torch.empty(rd, ud, Bn, T, Hx, D, dtype=X.dtype, device=dev)
        B.usp_zigzag_extract(X.to(dev), z, rd, ud, -1, -1)
        hm = torch.empty(rd, ud, Hx // ud, Bn, L, D, dtype=X.dtype, device=dev)
        for r in range(rd):
            B.usp_ulysses_a2a_layout(z[r], hm[r], ud, -1)
        return hm
    say("pipeline layouts")
    qh, kh, vh = to_heads(q, H), to_heads(k, Hkv), to_heads(v, Hkv)
    oh = torch.empty(rd, ud, H // ud, Bn, L, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(rd, ud, H // ud, Bn, L, dtype=torch.float32, device=dev)
    for r in range(rd):
        for u in range(ud):
            say("pipeline walk", r, u)
            kall, vall = kh[:, u], vh[:, u]
            desc = B.attn_desc(S, rd, qh[r, u], kall, vall, o=oh[r, u], layout="hbsd")
            B.usp_attn_fwd(qh[r, u], kall, vall, oh[r, u], lse[r, u], desc, r)
    zs = torch.empty(rd, ud, Bn, T, H, D, dtype=torch.bfloat16, device=dev)
    for r in range(rd):
        B.usp_ulysses_a2a_layout(oh[r], zs[r], ud, -1, inverse=True)
    out = torch.empty(Bn, S, H, D, dtype=torch.bfloat16, device=dev)
    B.usp_zigzag_extract(zs, out, rd, ud, -1, -1, inverse=True)
    torch.cuda.synchronize()
    lse_g = np.full((H, Bn, S), np.nan)
    for r in range(rd):
        p = ix.zigzag_share_positions(S, rd, r)
        for u in range(ud):
            lse_g[u * (H // ud):(u + 1) * (H // ud)][:, :, p] = f64(lse[r, u])
    check_close(f64(out), lse_g, o_ref, lse_ref, "bf16", "pipeline")
