"""ctypes binding of libusp.so: one Python function per C entry point, same
names, argument marshalling only.  Every step of the path runs in the HIP
library; nothing here computes.

Tensors are torch tensors used as device buffers; the stream defaults to
torch's current stream.  A non-OK status raises ``UspError``.  If the library
is not built the first call raises ``RuntimeError``: there is no fallback.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libusp.so")

USP_OK, USP_ERR_INVALID_ARG, USP_ERR_UNSUPPORTED, USP_ERR_HIP = 0, 1, 2, 3
USP_DTYPE_BF16, USP_DTYPE_FP32 = 0, 1

EXPORTED = ["usp_zigzag_extract", "usp_zigzag_extract_n", "usp_zigzag_extract_varlen", "usp_ulysses_a2a_layout",
            "usp_ulysses_a2a_layout_n", "usp_ulysses_a2a_layout_heads", "usp_ring_attn_step_fwd",
            "usp_ring_attn_step_fwd_merge",
            "usp_lse_merge", "usp_attn_fwd", "usp_attn_fwd_split", "usp_attn_fwd_split_workspace",
            "usp_attn_bwd_prep", "usp_ring_attn_step_bwd", "usp_attn_bwd", "usp_attn_bwd_noalloc",
            "usp_status_string", "usp_last_error_detail", "usp_abi_version"]

NOALLOC_MAX_STATS_ROWS = 1 << 21


class UspError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")


_STATUS = {0: "USP_OK", 1: "USP_ERR_INVALID_ARG", 2: "USP_ERR_UNSUPPORTED", 3: "USP_ERR_HIP"}


class UspStrides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64)]


class UspAttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("num_q_heads", ctypes.c_int64), ("num_kv_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("cp", ctypes.c_int32),
                ("q", UspStrides), ("k", UspStrides), ("v", UspStrides), ("o", UspStrides),
                ("kv_block_stride", ctypes.c_int64), ("q_rank_stride", ctypes.c_int64),
                ("o_rank_stride", ctypes.c_int64), ("cu_seqlens", ctypes.c_void_p),
                ("num_seqs", ctypes.c_int32), ("zigzag_per_sample", ctypes.c_int32)]


_lib = None


def lib():
    """Load libusp.so (once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
        L.usp_zigzag_extract.argtypes = [vp, vp, st, i64, i64, i64, i64, i32, i32, i32, i32, i32, vp]
        L.usp_zigzag_extract_varlen.argtypes = [vp, vp, st, i64, i64, i64, i64, i32, i32, i32, i32, i32, vp, i32,
                                                vp]
        L.usp_ulysses_a2a_layout.argtypes = [vp, vp, st, i64, i64, i64, i64, i32, i32, i32, vp]
        L.usp_ulysses_a2a_layout_heads.argtypes = [vp, vp, st, i64, i64, i64, i64, i32, i32, i64, i64, i32, vp]
        L.usp_zigzag_extract_n.argtypes = [i32, vp, vp, vp, st, i64, i64, i64, i32, i32, i32, i32, i32, vp]
        L.usp_ulysses_a2a_layout_n.argtypes = [i32, vp, vp, vp, st, i64, i64, i64, i32, i32, i32, vp]
        L.usp_ring_attn_step_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, i32, vp]
        L.usp_ring_attn_step_fwd_merge.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, i32, vp]
        L.usp_lse_merge.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.usp_attn_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, vp]
        L.usp_attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, vp, i64, vp]
        L.usp_attn_fwd_split_workspace.argtypes = [ctypes.POINTER(UspAttnDesc), i32]
        L.usp_attn_fwd_split_workspace.restype = i64
        L.usp_attn_bwd_prep.argtypes = [vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, vp]
        L.usp_ring_attn_step_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc),
                                             i32, i32, vp]
        L.usp_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, vp]
        L.usp_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(UspAttnDesc), i32, vp]
        for f in ("usp_zigzag_extract", "usp_zigzag_extract_n", "usp_zigzag_extract_varlen", "usp_ulysses_a2a_layout",
                  "usp_ulysses_a2a_layout_n",
                  "usp_ulysses_a2a_layout_heads", "usp_ring_attn_step_fwd", "usp_ring_attn_step_fwd_merge",
                  "usp_lse_merge", "usp_attn_fwd", "usp_attn_fwd_split", "usp_attn_bwd_prep", "usp_ring_attn_step_bwd",
                  "usp_attn_bwd", "usp_attn_bwd_noalloc"):
            getattr(L, f).restype = st
        L.usp_status_string.argtypes = [st]
        L.usp_status_string.restype = ctypes.c_char_p
        L.usp_last_error_detail.argtypes = []
        L.usp_last_error_detail.restype = ctypes.c_char_p
        L.usp_abi_version.argtypes = []
        L.usp_abi_version.restype = i32
        _lib = L
    return _lib


def check(status):
    if status != USP_OK:
        raise UspError(status, lib().usp_last_error_detail().decode())


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return USP_DTYPE_BF16
    if t.dtype == torch.float32:
        return USP_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")


def _contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def usp_zigzag_extract(x, out, rd, ud, ring_rank, ulysses_rank, inverse=False, stream=None):
    """Forward: x global (B, S, H, D) -> out shard(s).  Inverse: x shard(s) ->
    out global.  Shapes as in include/usp.h."""
    _dev(x, out)
    _contig(x, out)
    B, S, H, D = (out if inverse else x).shape
    groups = rd * ud if ring_rank < 0 else (ud if ulysses_rank < 0 else 1)
    shard_elems = groups * B * (S // (rd * ud)) * H * D
    if (x if inverse else out).numel() != shard_elems:
        raise ValueError(f"shard buffer must hold {shard_elems} elements")
    check(lib().usp_zigzag_extract(x.data_ptr(), out.data_ptr(), _dtype(x), B, S, H, D, rd, ud,
                                   ring_rank, ulysses_rank, int(inverse), _stream(stream)))
    return out


def _ptr_arrays(srcs, dsts, heads):
    n = len(srcs)
    if n != len(dsts) or n != len(heads):
        raise ValueError("one output and one head count per input")
    return (n, (ctypes.c_void_p * n)(*[t.data_ptr() for t in srcs]),
            (ctypes.c_void_p * n)(*[t.data_ptr() for t in dsts]), (ctypes.c_int64 * n)(*heads))


def usp_zigzag_extract_n(xs, outs, rd, ud, ring_rank, ulysses_rank, inverse=False, stream=None):
    """usp_zigzag_extract of several tensors (same dtype, B, S, D; own head
    counts) in one launch."""
    xs, outs = list(xs), list(outs)
    _dev(*xs, *outs)
    _contig(*xs, *outs)
    heads = []
    for x, out in zip(xs, outs):
        if x.dtype != xs[0].dtype:
            raise ValueError("all tensors must share the dtype")
        B, S, H, D = (out if inverse else x).shape
        if (B, S, D) != tuple((outs[0] if inverse else xs[0]).shape[i] for i in (0, 1, 3)):
            raise ValueError("all tensors must share B, S and D")
        groups = rd * ud if ring_rank < 0 else (ud if ulysses_rank < 0 else 1)
        if (x if inverse else out).numel() != groups * B * (S // (rd * ud)) * H * D:
            raise ValueError("a shard buffer has the wrong number of elements")
        heads.append(H)
    B, S, _, D = (outs[0] if inverse else xs[0]).shape
    n, src, dst, hs = _ptr_arrays(xs, outs, heads)
    check(lib().usp_zigzag_extract_n(n, src, dst, hs, _dtype(xs[0]), B, S, D, rd, ud, ring_rank, ulysses_rank,
                                     int(inverse), _stream(stream)))
    return outs


def host_cu_seqlens(cu_seqlens):
    """Packed-sample boundaries as a contiguous host int32 array (the C calls
    read them from host memory; a GPU tensor is copied back first)."""
    if isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)


def usp_zigzag_extract_varlen(x, out, rd, ud, ring_rank, ulysses_rank, cu_seqlens, inverse=False, stream=None):
    """Per-sample zigzag: as usp_zigzag_extract, with Algorithm 2's split
    applied to every packed sample (lengths multiples of 2*rd)."""
    _dev(x, out)
    _contig(x, out)
    B, S, H, D = (out if inverse else x).shape
    groups = rd * ud if ring_rank < 0 else (ud if ulysses_rank < 0 else 1)
    shard_elems = groups * B * (S // (rd * ud)) * H * D
    if (x if inverse else out).numel() != shard_elems:
        raise ValueError(f"shard buffer must hold {shard_elems} elements")
    cu = host_cu_seqlens(cu_seqlens)
    check(lib().usp_zigzag_extract_varlen(x.data_ptr(), out.data_ptr(), _dtype(x), B, S, H, D, rd, ud,
                                          ring_rank, ulysses_rank, int(inverse), cu.ctypes.data, cu.size - 1,
                                          _stream(stream)))
    return out


def usp_ulysses_a2a_layout(inp, out, degree, rank, inverse=False, stream=None):
    """Forward: inp (N, bs, L/N, hc, hd) -> out (hc/N, bs, L, hd) [rank u] or
    (N, ...) [rank -1].  Inverse: inp (N, hc/N, bs, L, hd) -> (bs, L/N, hc, hd)
    [or (N, ...)]."""
    _dev(inp, out)
    _contig(inp, out)
    if not inverse:
        N, bs, ls, hc, hd = inp.shape
        L = ls * N
    else:
        N, hb, bs, L, hd = inp.shape
        hc = hb * N
    if N != degree:
        raise ValueError("leading dimension of inp must equal the Ulysses degree")
    if out.numel() != (degree if rank < 0 else 1) * bs * L * (hc // degree) * hd:
        raise ValueError("out has the wrong number of elements")
    check(lib().usp_ulysses_a2a_layout(inp.data_ptr(), out.data_ptr(), _dtype(inp), bs, L, hc, hd,
                                       degree, rank, int(inverse), _stream(stream)))
    return out


def usp_ulysses_a2a_layout_n(inps, outs, degree, rank, inverse=False, stream=None):
    """usp_ulysses_a2a_layout of several tensors (same dtype, bs, L, hd; own
    head counts) in one launch; shapes per tensor as usp_ulysses_a2a_layout."""
    inps, outs = list(inps), list(outs)
    _dev(*inps, *outs)
    _contig(*inps, *outs)
    heads, dims = [], None
    for inp, out in zip(inps, outs):
        if inp.dtype != inps[0].dtype:
            raise ValueError("all tensors must share the dtype")
        if not inverse:
            N, bs, ls, hc, hd = inp.shape
            L = ls * N
        else:
            N, hb, bs, L, hd = inp.shape
            hc = hb * N
        if N != degree:
            raise ValueError("leading dimension of every input must equal the Ulysses degree")
        if dims is not None and (bs, L, hd) != dims:
            raise ValueError("all tensors must share bs, L and hd")
        dims = (bs, L, hd)
        if out.numel() != (degree if rank < 0 else 1) * bs * L * (hc // degree) * hd:
            raise ValueError("an output has the wrong number of elements")
        heads.append(hc)
    bs, L, hd = dims
    n, src, dst, hs = _ptr_arrays(inps, outs, heads)
    check(lib().usp_ulysses_a2a_layout_n(n, src, dst, hs, _dtype(inps[0]), bs, L, hd, degree, rank, int(inverse),
                                         _stream(stream)))
    return outs


def usp_ulysses_a2a_layout_heads(inp, out, degree, rank, head_offset, num_heads, inverse=False, stream=None):
    """Heads [head_offset, head_offset + num_heads) of every head block.
    Forward: inp (N, bs, L/N, hc, hd) -> out (num_heads, bs, L, hd) [rank u]
    or (N, ...) [rank -1].  Inverse: inp (N, num_heads, bs, L, hd) -> the
    chunk's heads of out (bs, L/N, hc, hd) [or (N, ...)], hc read from out."""
    _dev(inp, out)
    _contig(inp, out)
    if not inverse:
        N, bs, ls, hc, hd = inp.shape
        L = ls * N
        want = (degree if rank < 0 else 1) * num_heads * bs * L * hd
    else:
        N, nh, bs, L, hd = inp.shape
        hc = out.shape[-2]
        if nh != num_heads:
            raise ValueError("inp must hold num_heads heads per peer")
        want = (degree if rank < 0 else 1) * bs * (L // degree) * hc * hd
    if N != degree:
        raise ValueError("leading dimension of inp must equal the Ulysses degree")
    if out.numel() != want:
        raise ValueError("out has the wrong number of elements")
    check(lib().usp_ulysses_a2a_layout_heads(inp.data_ptr(), out.data_ptr(), _dtype(inp), bs, L, hc, hd, degree,
                                             rank, head_offset, num_heads, int(inverse), _stream(stream)))
    return out


def _check_attn(k_all, v_all, lse, desc, n_ranks):
    if k_all.shape[0] != desc.cp or v_all.shape[0] != desc.cp:
        raise ValueError("k_all / v_all need a leading dim of cp blocks")
    L = desc.seq_len // desc.cp
    if lse.dtype != torch.float32 or not lse.is_contiguous() or \
            lse.numel() != n_ranks * desc.num_q_heads * desc.batch * L:
        raise ValueError("lse must be contiguous fp32 with (ranks, Hq, B, 2c) elements")


def usp_ring_attn_step_fwd(q, k_all, v_all, o_step, lse_step, desc, ring_rank, step, stream=None):
    _dev(q, k_all, v_all, o_step, lse_step)
    _check_attn(k_all, v_all, lse_step, desc, 1)
    if o_step.dtype != torch.float32 or not o_step.is_contiguous() or \
            o_step.numel() != lse_step.numel() * desc.head_dim:
        raise ValueError("o_step must be contiguous fp32 (Hq, B, 2c, D)")
    check(lib().usp_ring_attn_step_fwd(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(),
                                       o_step.data_ptr(), lse_step.data_ptr(), ctypes.byref(desc),
                                       ring_rank, step, _stream(stream)))
    return o_step, lse_step


def usp_ring_attn_step_fwd_merge(q, k_all, v_all, o_acc, lse_acc, desc, ring_rank, step, stream=None):
    """One ring step merged into (o_acc, lse_acc) in place (layouts of usp_ring_attn_step_fwd's partial)."""
    _dev(q, k_all, v_all, o_acc, lse_acc)
    _check_attn(k_all, v_all, lse_acc, desc, 1)
    if o_acc.dtype != torch.float32 or not o_acc.is_contiguous() or \
            o_acc.numel() != lse_acc.numel() * desc.head_dim:
        raise ValueError("o_acc must be contiguous fp32 (Hq, B, 2c, D)")
    check(lib().usp_ring_attn_step_fwd_merge(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(),
                                             o_acc.data_ptr(), lse_acc.data_ptr(), ctypes.byref(desc),
                                             ring_rank, step, _stream(stream)))
    return o_acc, lse_acc


def usp_lse_merge(o_acc, lse_acc, o_step, lse_step, stream=None):
    """In place on (o_acc, lse_acc); o tensors (..., D) fp32, lse (...) fp32."""
    _dev(o_acc, lse_acc, o_step, lse_step)
    _contig(o_acc, lse_acc, o_step, lse_step)
    D = o_acc.shape[-1]
    rows = lse_acc.numel()
    if o_acc.numel() != rows * D or o_step.numel() != rows * D or lse_step.numel() != rows:
        raise ValueError("o (rows, D) and lse (rows) shapes disagree")
    check(lib().usp_lse_merge(o_acc.data_ptr(), lse_acc.data_ptr(), o_step.data_ptr(),
                              lse_step.data_ptr(), rows, D, _stream(stream)))
    return o_acc, lse_acc


def usp_attn_fwd(q, k_all, v_all, o, lse, desc, ring_rank, stream=None):
    _dev(q, k_all, v_all, o, lse)
    _check_attn(k_all, v_all, lse, desc, desc.cp if ring_rank < 0 else 1)
    check(lib().usp_attn_fwd(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), ctypes.byref(desc), ring_rank, _stream(stream)))
    return o, lse


def usp_attn_fwd_split_workspace(desc, ring_rank):
    """Bytes of workspace usp_attn_fwd_split needs (host only)."""
    n = lib().usp_attn_fwd_split_workspace(ctypes.byref(desc), ring_rank)
    if n < 0:
        raise ValueError("bad descriptor or ring_rank")
    return n


def usp_attn_fwd_split(q, k_all, v_all, o, lse, desc, ring_rank, workspace, stream=None):
    """usp_attn_fwd with heavy query tiles' ring steps split over two
    workgroups when the launch is small; `workspace` is a contiguous GPU tensor
    of at least usp_attn_fwd_split_workspace(desc, ring_rank) bytes."""
    _dev(q, k_all, v_all, o, lse, workspace)
    _contig(workspace)
    _check_attn(k_all, v_all, lse, desc, desc.cp if ring_rank < 0 else 1)
    check(lib().usp_attn_fwd_split(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), ctypes.byref(desc), ring_rank, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, lse


def _stats_rows(desc, n_ranks):
    return n_ranks * desc.num_q_heads * desc.batch * (desc.seq_len // desc.cp)


def _check_stats(stats, desc, n_ranks):
    if stats.dtype != torch.float32 or not stats.is_contiguous() or stats.numel() != 2 * _stats_rows(desc, n_ranks):
        raise ValueError("stats must be contiguous fp32 with 2 * (ranks, Hq, B, 2c) elements")


def _same_layout(a, b):
    """Same shape and the same element strides on every dim that has more than one index."""
    return a.shape == b.shape and all(n == 1 or sa == sb for n, sa, sb in zip(a.shape, a.stride(), b.stride()))


def _check_dkv(k_all, v_all, dk_all, dv_all):
    for g, x in ((dk_all, k_all), (dv_all, v_all)):
        if g.dtype != torch.float32 or not _same_layout(g, x):
            raise ValueError("dk_all / dv_all must be fp32 with the shape and element strides of k_all / v_all")


def usp_attn_bwd_prep(o, d_o, lse, stats, desc, ring_rank, stream=None):
    """stats = [rowsum(dO * O) | lse * log2(e)] per query row (layout in include/usp.h)."""
    _dev(o, d_o, lse, stats)
    n = desc.cp if ring_rank < 0 else 1
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != _stats_rows(desc, n):
        raise ValueError("lse must be contiguous fp32 with (ranks, Hq, B, 2c) elements")
    _check_stats(stats, desc, n)
    check(lib().usp_attn_bwd_prep(o.data_ptr(), d_o.data_ptr(), lse.data_ptr(), stats.data_ptr(),
                                  ctypes.byref(desc), ring_rank, _stream(stream)))
    return stats


def usp_ring_attn_step_bwd(q, k_all, v_all, d_o, stats, dq_acc, dk_all, dv_all, desc, ring_rank, step,
                           stream=None):
    """Adds step ``step``'s gradient contributions into dq_acc (fp32 (Hq, B, 2c, D)) and into
    block (r - step) mod cp of dk_all / dv_all (fp32, k_all's / v_all's strides)."""
    _dev(q, k_all, v_all, d_o, stats, dq_acc, dk_all, dv_all)
    _check_stats(stats, desc, 1)
    _check_dkv(k_all, v_all, dk_all, dv_all)
    if dq_acc.dtype != torch.float32 or not dq_acc.is_contiguous() or \
            dq_acc.numel() != _stats_rows(desc, 1) * desc.head_dim:
        raise ValueError("dq_acc must be contiguous fp32 (Hq, B, 2c, D)")
    check(lib().usp_ring_attn_step_bwd(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(), d_o.data_ptr(),
                                       stats.data_ptr(), dq_acc.data_ptr(), dk_all.data_ptr(), dv_all.data_ptr(),
                                       ctypes.byref(desc), ring_rank, step, _stream(stream)))
    return dq_acc, dk_all, dv_all


def usp_attn_bwd(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all, stats, desc, ring_rank, stream=None):
    """The ring backward of one rank (or every rank, ring_rank = -1): writes dq (dtype, Q's
    strides) and adds the rank's contributions into dk_all / dv_all."""
    _dev(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all, stats)
    n = desc.cp if ring_rank < 0 else 1
    _check_attn(k_all, v_all, lse, desc, n)
    _check_stats(stats, desc, n)
    _check_dkv(k_all, v_all, dk_all, dv_all)
    if dq.dtype != q.dtype or not _same_layout(dq, q):
        raise ValueError("dq must have q's dtype, shape and strides")
    if d_o.dtype != o.dtype or not _same_layout(d_o, o):
        raise ValueError("d_o must have o's dtype, shape and strides")
    check(lib().usp_attn_bwd(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(), o.data_ptr(), d_o.data_ptr(),
                             lse.data_ptr(), dq.data_ptr(), dk_all.data_ptr(), dv_all.data_ptr(),
                             stats.data_ptr(), ctypes.byref(desc), ring_rank, _stream(stream)))
    return dq, dk_all, dv_all


def usp_attn_bwd_noalloc(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all, desc, ring_rank, stream=None):
    """usp_attn_bwd with its statistics rows in the library's own device array
    (no caller buffer, nothing allocated); at most NOALLOC_MAX_STATS_ROWS rows."""
    _dev(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all)
    n = desc.cp if ring_rank < 0 else 1
    _check_attn(k_all, v_all, lse, desc, n)
    _check_dkv(k_all, v_all, dk_all, dv_all)
    if dq.dtype != q.dtype or not _same_layout(dq, q):
        raise ValueError("dq must have q's dtype, shape and strides")
    if d_o.dtype != o.dtype or not _same_layout(d_o, o):
        raise ValueError("d_o must have o's dtype, shape and strides")
    check(lib().usp_attn_bwd_noalloc(q.data_ptr(), k_all.data_ptr(), v_all.data_ptr(), o.data_ptr(),
                                     d_o.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk_all.data_ptr(),
                                     dv_all.data_ptr(), ctypes.byref(desc), ring_rank, _stream(stream)))
    return dq, dk_all, dv_all


def attn_desc(seq_len, cp, q, k_all, v_all, o=None, layout="bshd", causal=True, softmax_scale=None,
              cu_seqlens=None, all_ranks=False, zigzag_per_sample=False):
    """Build a ``UspAttnDesc`` from tensors.

    ``layout`` names the order of the last four dims of every tensor: "bshd"
    (sequence-major, [batch, seq, head, dim]) or "hbsd" (head-major, after the
    Ulysses layout).  ``k_all``/``v_all`` have a leading cp (block) dim; with
    ``all_ranks`` so do ``q`` and ``o``.  ``cu_seqlens``: packed-sample
    boundaries (any int sequence; kept as a host array on the descriptor);
    ``zigzag_per_sample``: the shares are the per-sample zigzag split.
    """
    pos = {"bshd": (0, 1, 2), "hbsd": (1, 2, 0)}[layout]

    def strides(t, lead):
        st = t.stride()[lead:]
        if st[3] != 1:
            raise ValueError("head_dim must be the contiguous dim")
        return UspStrides(st[pos[0]], st[pos[1]], st[pos[2]])

    ql = 1 if all_ranks else 0
    shp = q.shape[ql:]
    B, Hq, D = shp[pos[0]], shp[pos[2]], shp[3]
    Hkv = k_all.shape[1:][pos[2]]
    d = UspAttnDesc()
    d.batch, d.seq_len, d.num_q_heads, d.num_kv_heads, d.head_dim = B, seq_len, Hq, Hkv, D
    d.dtype = _dtype(q)
    d.softmax_scale = (D ** -0.5) if softmax_scale is None else softmax_scale
    d.causal = int(causal)
    d.cp = cp
    d.q = strides(q, ql)
    d.k = strides(k_all, 1)
    d.v = strides(v_all, 1)
    if v_all.stride(0) != k_all.stride(0):
        raise ValueError("k_all and v_all must share the block stride")
    d.kv_block_stride = k_all.stride(0)
    if o is not None:
        d.o = strides(o, ql)
        d.o_rank_stride = o.stride(0) if all_ranks else 0
    d.q_rank_stride = q.stride(0) if all_ranks else 0
    if cu_seqlens is not None:
        d._cu_host = host_cu_seqlens(cu_seqlens)   # the descriptor points into this array
        d.cu_seqlens = d._cu_host.ctypes.data
        d.num_seqs = d._cu_host.size - 1
    d.zigzag_per_sample = int(zigzag_per_sample)
    return d
