"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and the host-side validation rejects bad arguments before any launch.

Error-path calls pass fake (but aligned) addresses that validation must
reject; they are skipped where a GPU is visible so that a validation bug can
never turn into a launch on real hardware.
"""
import ctypes
import os
import re

import pytest
import torch

from sequence_ring_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "usp.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer error paths run on CPU only")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:usp_status|const char \*|int32_t|int64_t)\s*(usp_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) == 19, names
    lib = B.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(B.EXPORTED)


def test_abi_version_and_status_strings():
    lib = B.lib()
    assert lib.usp_abi_version() == 7
    assert lib.usp_status_string(0) == b"USP_OK"
    assert lib.usp_status_string(2) == b"USP_ERR_UNSUPPORTED"
    assert lib.usp_status_string(99) == b"USP_ERR_UNKNOWN"


FAKE = 0x10000      # aligned, never dereferenced: validation must reject first
FAKE2 = 0x20000
FAKE3 = 0x30000


def _zz(**kw):
    a = dict(x=FAKE, out=FAKE2, dtype=0, B=1, S=64, H=2, D=64, rd=4, ud=1, r=0, u=0, inv=0)
    a.update(kw)
    return B.lib().usp_zigzag_extract(a["x"], a["out"], a["dtype"], a["B"], a["S"], a["H"], a["D"],
                                      a["rd"], a["ud"], a["r"], a["u"], a["inv"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(x=FAKE + 2), 1), (dict(out=FAKE), 1), (dict(dtype=7), 1),
    (dict(S=60), 1), (dict(rd=0), 1), (dict(r=4), 1), (dict(u=1), 1), (dict(r=-1, u=0), 1),
    (dict(inv=2), 1), (dict(H=1, D=2, dtype=0), 2), (dict(B=0), 1),
])
def test_zigzag_rejects(kw, status):
    assert _zz(**kw) == status
    assert B.lib().usp_last_error_detail()


def _uly(**kw):
    a = dict(i=FAKE, o=FAKE2, dtype=0, B=1, L=64, H=4, D=64, N=2, u=0, inv=0)
    a.update(kw)
    return B.lib().usp_ulysses_a2a_layout(a["i"], a["o"], a["dtype"], a["B"], a["L"], a["H"], a["D"],
                                          a["N"], a["u"], a["inv"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(i=None), 1), (dict(o=FAKE + 8), 1), (dict(o=FAKE), 1), (dict(H=3), 1), (dict(L=63), 1),
    (dict(u=2), 1), (dict(u=-2), 1), (dict(N=0), 1), (dict(D=4), 2), (dict(inv=-1), 1),
])
def test_ulysses_rejects(kw, status):
    assert _uly(**kw) == status


def _uly_heads(**kw):
    a = dict(i=FAKE, o=FAKE2, dtype=0, B=1, L=64, H=8, D=64, N=2, u=0, h0=0, nh=2, inv=0)
    a.update(kw)
    return B.lib().usp_ulysses_a2a_layout_heads(a["i"], a["o"], a["dtype"], a["B"], a["L"], a["H"], a["D"],
                                                a["N"], a["u"], a["h0"], a["nh"], a["inv"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(h0=-1), 1), (dict(nh=0), 1), (dict(h0=3, nh=2), 1), (dict(nh=5), 1), (dict(h0=4, nh=1), 1),
    (dict(i=None), 1), (dict(o=FAKE), 1), (dict(H=7), 1), (dict(L=63), 1), (dict(u=2), 1), (dict(D=4), 2),
    (dict(inv=2), 1), (dict(inv=1, h0=2, nh=3), 1),
])
def test_ulysses_heads_rejects(kw, status):
    assert _uly_heads(**kw) == status
    assert b"ulysses_a2a_layout_heads" in B.lib().usp_last_error_detail()


@no_gpu
def test_merge_rejects():
    lib = B.lib()
    assert lib.usp_lse_merge(FAKE, FAKE2, FAKE3, FAKE, -1, 64, None) == 1
    assert lib.usp_lse_merge(FAKE, FAKE2, FAKE3, FAKE, 4, 6, None) == 1
    assert lib.usp_lse_merge(None, FAKE2, FAKE3, FAKE, 4, 64, None) == 1
    assert lib.usp_lse_merge(FAKE + 4, FAKE2, FAKE3, FAKE, 4, 64, None) == 1
    assert lib.usp_lse_merge(None, None, None, None, 0, 64, None) == 0    # rows = 0: no-op


def _desc(**kw):
    d = B.UspAttnDesc()
    d.batch, d.seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim = 1, 256, 4, 2, 128
    d.dtype, d.softmax_scale, d.causal, d.cp = 0, 128 ** -0.5, 1, 4
    d.q = B.UspStrides(64 * 4 * 128, 4 * 128, 128)
    d.k = B.UspStrides(64 * 2 * 128, 2 * 128, 128)
    d.v = B.UspStrides(64 * 2 * 128, 2 * 128, 128)
    d.o = B.UspStrides(64 * 4 * 128, 4 * 128, 128)
    d.kv_block_stride = 64 * 2 * 128
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=250), 1), (dict(num_q_heads=3), 1), (dict(head_dim=96), 2), (dict(head_dim=32), 2),
    (dict(softmax_scale=0.0), 1), (dict(softmax_scale=float("inf")), 1), (dict(cp=0), 1),
    (dict(causal=2), 1), (dict(dtype=5), 1), (dict(cu_seqlens=FAKE, num_seqs=2, causal=0), 2),
    (dict(cu_seqlens=FAKE, num_seqs=0), 1), (dict(kv_block_stride=3), 1),
    (dict(q=B.UspStrides(1, 4 * 128, 128)), 1), (dict(batch=0), 1),
])
def test_attention_descriptor_rejects(kw, status):
    lib = B.lib()
    d = _desc(**kw)
    assert lib.usp_ring_attn_step_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, 0, None) == status
    assert lib.usp_ring_attn_step_fwd_merge(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, 0, None) == status
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == status


@no_gpu
def test_attention_rank_and_step_ranges():
    lib = B.lib()
    d = _desc()
    step = lambda r, t: lib.usp_ring_attn_step_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), r, t, None)
    assert step(4, 0) == 1 and step(-1, 0) == 1 and step(0, 4) == 1 and step(0, -1) == 1
    merged = lambda r, t: lib.usp_ring_attn_step_fwd_merge(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), r, t,
                                                           None)
    assert merged(4, 0) == 1 and merged(-1, 0) == 1 and merged(0, 4) == 1 and merged(0, -1) == 1
    walk = lambda r: lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), r, None)
    assert walk(4) == 1 and walk(-2) == 1
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, None, 0, None) == 1
    assert lib.usp_attn_fwd(None, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == 1


def test_split_walk_workspace_size():
    lib = B.lib()
    d = _desc()
    rows = d.num_q_heads * d.batch * (d.seq_len // d.cp)
    assert lib.usp_attn_fwd_split_workspace(ctypes.byref(d), 0) == 2 * rows * (d.head_dim + 1) * 4
    assert lib.usp_attn_fwd_split_workspace(ctypes.byref(d), -1) == 2 * d.cp * rows * (d.head_dim + 1) * 4
    assert lib.usp_attn_fwd_split_workspace(ctypes.byref(d), d.cp) == -1
    assert lib.usp_attn_fwd_split_workspace(None, 0) == -1


@no_gpu
def test_split_walk_rejects_bad_workspace():
    lib = B.lib()
    d = _desc()
    need = lib.usp_attn_fwd_split_workspace(ctypes.byref(d), 0)
    ws = 0x1000000
    call = lambda w, n, **kw: lib.usp_attn_fwd_split(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(_desc(**kw)), 0,
                                                     w, n, None)
    assert call(None, need) == 1
    assert call(ws + 16, need) == 1
    assert call(ws, need - 1) == 1
    assert call(ws, need, head_dim=96) == 2


def _arrays(xs, outs, heads):
    n = len(xs)
    return ((ctypes.c_void_p * n)(*xs), (ctypes.c_void_p * n)(*outs), (ctypes.c_int64 * n)(*heads))


# distinct, far-apart fake buffers (1 MiB apart): extents of the small shapes below never meet
F = [0x1000000 * (i + 1) for i in range(8)]


def _zz_n(n=3, xs=None, outs=None, heads=None, **kw):
    a = dict(dtype=0, B=1, S=64, D=64, rd=4, ud=1, r=0, u=0, inv=0)
    a.update(kw)
    xs = F[:3] if xs is None else xs
    outs = F[3:6] if outs is None else outs
    heads = [4, 2, 2] if heads is None else heads
    x, o, h = _arrays(xs, outs, heads)
    return B.lib().usp_zigzag_extract_n(n, x, o, h, a["dtype"], a["B"], a["S"], a["D"], a["rd"], a["ud"], a["r"],
                                        a["u"], a["inv"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(n=0), 1), (dict(n=5, xs=F[:5], outs=[F[5], F[6], F[7], F[7] + 4096, F[7] + 8192], heads=[2] * 5), 1),
    (dict(xs=[F[0], None, F[2]]), 1), (dict(outs=[F[3], F[4] + 8, F[5]]), 1), (dict(heads=[4, 0, 2]), 1),
    (dict(S=60), 1), (dict(r=4), 1), (dict(inv=2), 1), (dict(heads=[4, 1, 2], D=2), 2),
    # output 1 lies inside input 0 (the global tensor of 64 rows x 4 heads x 64 x 2 bytes)
    (dict(outs=[F[3], F[0] + 1024, F[5]]), 1),
    # outputs 0 and 2 share their first bytes
    (dict(outs=[F[3], F[4], F[3] + 16]), 1),
])
def test_zigzag_n_rejects(kw, status):
    assert _zz_n(**kw) == status
    assert b"zigzag_extract_n" in B.lib().usp_last_error_detail()


@no_gpu
def test_zigzag_n_rejects_more_pieces_than_one_launch_counts():
    """Four every-rank extracts of 64 KiB rows (one row per piece), 2^31 pieces
    each: the batch holds 2^33 pieces, beyond the device's 32-bit piece index.
    (Validation only: the fake buffers are never touched.)"""
    S = (1 << 31) - 32                           # below the row limit, divisible by 2 rd ud = 8
    assert _zz_n(n=4, xs=F[:4], outs=F[4:8], heads=[256] * 4, S=S, D=128, r=-1, u=-1) == 2
    assert b"too many pieces" in B.lib().usp_last_error_detail()


@no_gpu
def test_zigzag_n_rejects_null_arrays():
    x, o, h = _arrays(F[:3], F[3:6], [4, 2, 2])
    lib = B.lib()
    assert lib.usp_zigzag_extract_n(3, None, o, h, 0, 1, 64, 64, 4, 1, 0, 0, 0, None) == 1
    assert lib.usp_zigzag_extract_n(3, x, o, None, 0, 1, 64, 64, 4, 1, 0, 0, 0, None) == 1
    assert lib.usp_ulysses_a2a_layout_n(3, x, None, h, 0, 1, 64, 64, 2, 0, 0, None) == 1


def _uly_n(n=3, ins=None, outs=None, heads=None, **kw):
    a = dict(dtype=0, B=1, L=64, D=64, N=2, u=0, inv=0)
    a.update(kw)
    ins = F[:3] if ins is None else ins
    outs = F[3:6] if outs is None else outs
    heads = [8, 2, 2] if heads is None else heads
    i, o, h = _arrays(ins, outs, heads)
    return B.lib().usp_ulysses_a2a_layout_n(n, i, o, h, a["dtype"], a["B"], a["L"], a["D"], a["N"], a["u"],
                                            a["inv"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(n=0), 1), (dict(n=5), 1), (dict(heads=[8, 3, 2]), 1), (dict(L=63), 1), (dict(u=2), 1),
    (dict(D=4), 2), (dict(inv=-1), 1), (dict(ins=[F[0], F[1] + 4, F[2]]), 1),
    (dict(outs=[F[3], F[1] + 512, F[5]]), 1), (dict(outs=[F[3], F[4], F[4] + 1024]), 1),
])
def test_ulysses_n_rejects(kw, status):
    assert _uly_n(**kw) == status
    assert b"ulysses_a2a_layout_n" in B.lib().usp_last_error_detail()


@no_gpu
def test_batched_copies_reach_the_runtime():
    """Valid batches pass validation and fail only at launch without a GPU."""
    assert _zz_n() == 3
    assert b"launch" in B.lib().usp_last_error_detail()
    assert _zz_n(n=1, heads=[4]) == 3
    assert _uly_n() == 3
    assert _uly_n(inv=1, u=-1) == 3
    assert b"launch" in B.lib().usp_last_error_detail()


@no_gpu
def test_bf16_attention_rejects_rows_beyond_32_bit_offsets():
    """A sequence-major (B, 2c, H, D) MHA share of 512K + 64 tokens with 32 heads:
    a K/V slice spans just over 512K rows x 8 KiB = 4 GiB, beyond the bf16 kernels'
    32-bit offsets, so the call is refused; the head-major layout (row
    stride D) of the same share is accepted (it then fails only at launch,
    there being no GPU).  fp32 kernels take 64-bit offsets and are not
    limited.  Fake buffers: validation only."""
    L, cp, H, D = (1 << 19) + 64, 4, 32, 128
    lib = B.lib()
    d = B.UspAttnDesc()
    d.batch, d.seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim = 1, L * cp, H, H, D
    d.dtype, d.softmax_scale, d.causal, d.cp = 0, D ** -0.5, 1, cp
    for st in (d.q, d.k, d.v, d.o):                      # (B, 2c, H, D)
        st.s, st.h, st.b = H * D, D, L * H * D
    d.kv_block_stride = L * H * D
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, 0x40000, 0x50000, ctypes.byref(d), 0, None) == 2
    assert b"4 GiB" in lib.usp_last_error_detail()
    for st in (d.q, d.k, d.v, d.o):                      # (H, B, 2c, D)
        st.s, st.h, st.b = D, L * D, L * D
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, 0x40000, 0x50000, ctypes.byref(d), 0, None) == 3


@no_gpu
def test_valid_arguments_reach_the_runtime_and_report_hip_errors():
    """With no GPU present, a call that passes validation fails at launch with
    USP_ERR_HIP and a message, never a crash."""
    lib = B.lib()
    assert _zz() == 3
    assert b"launch" in lib.usp_last_error_detail()


def test_binding_refuses_host_tensors():
    x = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.usp_zigzag_extract(x, out, 4, 1, 0, 0)


FAKE4, FAKE5, FAKE6, FAKE7 = 0x40000, 0x50000, 0x60000, 0x70000


def _bwd(d, r=0, **kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, do=FAKE5, lse=FAKE6, dq=FAKE7, dk=0x80000, dv=0x90000,
             stats=0xA0000)
    a.update(kw)
    return B.lib().usp_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["stats"], ctypes.byref(d), r, None)


def _step_bwd(d, r=0, t=0, **kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, do=FAKE5, stats=0xA0000, dq=FAKE7, dk=0x80000, dv=0x90000)
    a.update(kw)
    return B.lib().usp_ring_attn_step_bwd(a["q"], a["k"], a["v"], a["do"], a["stats"], a["dq"], a["dk"], a["dv"],
                                          ctypes.byref(d), r, t, None)


@no_gpu
def test_bf16_backward_rejects_q_rows_beyond_32_bit_offsets():
    """K and V head-major (dense rows), Q and dO sequence-major with 32 heads
    over just over 512K rows: the key-stationary passes' Q/dO slices span
    4 GiB or more, so the backward is refused before launch."""
    L, cp, H, D = (1 << 19) + 64, 4, 32, 128
    d = B.UspAttnDesc()
    d.batch, d.seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim = 1, L * cp, H, 1, D
    d.dtype, d.softmax_scale, d.causal, d.cp = 0, D ** -0.5, 1, cp
    for st in (d.q, d.o):                                # (B, 2c, H, D)
        st.s, st.h, st.b = H * D, D, L * H * D
    for st in (d.k, d.v):                                # (Hkv, B, 2c, D)
        st.s, st.h, st.b = D, L * D, L * D
    d.kv_block_stride = L * D
    assert _bwd(d) == 2
    assert b"Q/dO" in B.lib().usp_last_error_detail()


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=250), 1), (dict(head_dim=96), 2), (dict(softmax_scale=-1.0), 1), (dict(cp=0), 1),
    (dict(cu_seqlens=FAKE, num_seqs=2, causal=0), 2), (dict(o=B.UspStrides(64 * 4 * 128, 4 * 128 + 4, 128)), 1),
])
def test_backward_descriptor_rejects(kw, status):
    d = _desc(**kw)
    assert _bwd(d) == status
    assert _step_bwd(d) == status
    assert B.lib().usp_attn_bwd_prep(FAKE4, FAKE5, FAKE6, 0xA0000, ctypes.byref(d), 0, None) == status


@no_gpu
def test_backward_pointer_rank_and_step_checks():
    d = _desc()
    assert _bwd(d, dq=None) == 1 and _bwd(d, dk=0x80004) == 1 and _bwd(d, lse=None) == 1
    assert _bwd(d, dq=FAKE) == 1            # dq aliases q
    assert _bwd(d, dk=FAKE2) == 1           # dk aliases k
    assert _bwd(d, dv=0x80000) == 1         # dv aliases dk
    assert _bwd(d, do=FAKE4) == 1           # d_o aliases o
    assert _bwd(d, r=4) == 1 and _bwd(d, r=-2) == 1
    assert _step_bwd(d, r=-1) == 1 and _step_bwd(d, t=4) == 1 and _step_bwd(d, t=-1) == 1
    assert _step_bwd(d, stats=None) == 1 and _step_bwd(d, do=FAKE5 + 8) == 1
    lib = B.lib()
    assert lib.usp_attn_bwd_prep(FAKE4, FAKE4, FAKE6, 0xA0000, ctypes.byref(d), 0, None) == 1
    assert lib.usp_attn_bwd_prep(FAKE4, FAKE5, None, 0xA0000, ctypes.byref(d), 0, None) == 1
    assert lib.usp_attn_bwd_prep(FAKE4, FAKE5, FAKE6, 0xA0000, None, 0, None) == 1
    big = _desc(batch=1 << 14, seq_len=1 << 16, num_q_heads=1 << 10, num_kv_heads=1 << 10)
    assert _bwd(big) in (1, 2)              # too many statistics rows / indices


@no_gpu
def test_backward_valid_arguments_reach_the_runtime():
    d = _desc()
    assert _bwd(d) == 3 and _step_bwd(d) == 3
    assert B.lib().usp_attn_bwd_prep(FAKE4, FAKE5, FAKE6, 0xA0000, ctypes.byref(d), 0, None) == 3


def test_binding_refuses_strided_lse():
    """lse is read and written as a dense (ranks, Hq, B, 2c) array: a strided
    view must be refused before the call."""
    d = _desc()
    lse = torch.zeros(1, 64, 4).permute(2, 0, 1)          # (Hq, B, 2c) elements, wrong memory order
    kv = torch.zeros(4, 1)
    B._check_attn(kv, kv, lse.contiguous(), d, 1)
    with pytest.raises(ValueError):
        B._check_attn(kv, kv, lse, d, 1)


def _host_cu(vals):
    import numpy as np
    return np.ascontiguousarray(np.asarray(vals, dtype=np.int32))


@no_gpu
@pytest.mark.parametrize("cu,per_sample,status", [
    ([0, 100, 256], 0, 3),          # valid: reaches the launch (no GPU here)
    ([1, 100, 256], 0, 1),          # does not start at 0
    ([0, 100, 200], 0, 1),          # does not end at seq_len
    ([0, 100, 100, 256], 0, 1),     # not strictly increasing
    ([0, 96, 256], 1, 3),           # per-sample, lengths multiples of 2*cp = 8
    ([0, 100, 256], 1, 1),          # per-sample, 100 does not divide into 8 chunks
])
def test_attention_host_cu_seqlens_checks(cu, per_sample, status):
    arr = _host_cu(cu)
    d = _desc(cu_seqlens=arr.ctypes.data, num_seqs=arr.size - 1, zigzag_per_sample=per_sample)
    assert B.lib().usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == status


@no_gpu
def test_attention_per_sample_needs_cu_and_sample_count_limit():
    lib = B.lib()
    d = _desc(zigzag_per_sample=1)
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == 1
    d = _desc(zigzag_per_sample=2)
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == 1
    many = _host_cu(list(range(0, 257)) + [256])   # 257 samples
    d = _desc(cu_seqlens=many.ctypes.data, num_seqs=257)
    assert lib.usp_attn_fwd(FAKE, FAKE2, FAKE3, FAKE, FAKE2, ctypes.byref(d), 0, None) == 1


@no_gpu
@pytest.mark.parametrize("cu,kw,status", [
    ([0, 32, 64], {}, 3), ([0, 36, 64], {}, 1), ([0, 32, 60], {}, 1), (None, {}, 1),
    ([0, 32, 64], dict(u=2), 1), ([0, 32, 64], dict(r=-1, u=0), 1), ([0, 32, 64], dict(S=60), 1),
])
def test_zigzag_varlen_rejects(cu, kw, status):
    a = dict(x=FAKE, out=FAKE2, dtype=0, B=1, S=64, H=2, D=64, rd=4, ud=2, r=0, u=0, inv=0)
    a.update(kw)
    arr = None if cu is None else _host_cu(cu)
    ptr = None if arr is None else arr.ctypes.data
    n = 0 if arr is None else arr.size - 1
    assert B.lib().usp_zigzag_extract_varlen(a["x"], a["out"], a["dtype"], a["B"], a["S"], a["H"], a["D"], a["rd"],
                                             a["ud"], a["r"], a["u"], a["inv"], ptr, n, None) == status


def test_noalloc_backward_rejects_more_rows_than_its_array():
    """usp_attn_bwd_noalloc refuses a call whose statistics rows exceed the
    library's array before anything touches the GPU (fake pointers)."""
    lib = B.lib()
    args = (FAKE, FAKE2, FAKE3, FAKE4, FAKE5, FAKE6, FAKE7, 0x80000, 0x90000)
    big = _desc(num_q_heads=64, num_kv_heads=8, seq_len=4 * 65536)            # 64 x 65536 rows for one rank
    assert lib.usp_attn_bwd_noalloc(*args, ctypes.byref(big), 0, None) == 1
    assert b"statistics rows" in lib.usp_last_error_detail()
    every = _desc(num_q_heads=32, num_kv_heads=8, seq_len=131072)              # 4 ranks x 32 x 32768 rows
    assert lib.usp_attn_bwd_noalloc(*args, ctypes.byref(every), -1, None) == 1
    assert lib.usp_attn_bwd_noalloc(*args, None, 0, None) == 1
    assert B.NOALLOC_MAX_STATS_ROWS == 1 << 21
