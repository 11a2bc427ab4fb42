"""Shared helpers of the GPU parity tests: device setup, zigzag shares built
with the oracle's positions, and the tolerance checks of the parity bar.

Tolerances (floating point): bf16 inputs -- o max-abs <= 1e-2, o mean-abs <=
1e-3, lse max-abs <= 1e-3; fp32 inputs -- o max-abs <= 2e-5, o mean-abs <=
1e-6, lse max-abs <= 1e-6.  Rows with no visible key must carry lse = -inf
on both sides.  Index and layout work must be bit-exact.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

from oracle import index as ix

TOL = {"bf16": (1e-2, 1e-3, 1e-3), "fp32": (2e-5, 1e-6, 1e-6)}


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*msg):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def bits(t):
    """Raw bits of a CPU/GPU tensor as a numpy integer array (bf16 -> int16)."""
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def share_positions(S, rd):
    return [ix.zigzag_share_positions(S, rd, r) for r in range(rd)]


def shares(X, rd):
    """(B, S, H, D) -> (rd, B, S/rd, H, D): every ring rank's zigzag share,
    gathered with the oracle's positions (a library gather, no method math)."""
    S = X.shape[1]
    idx = torch.from_numpy(np.concatenate(share_positions(S, rd))).to(X.device)
    g = X.index_select(1, idx)
    return g.view(X.shape[0], rd, S // rd, *X.shape[2:]).transpose(0, 1).contiguous()


def bf16_rounding_floor(o_ref):
    """Expected |error| of rounding the exact values to bf16: a quarter of
    the bf16 spacing at each value, averaged.  Rounding alone contributes
    this much to a mean-abs comparison of a bf16 output with the exact one."""
    a = np.abs(np.asarray(o_ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a > 0, 2.0 ** (e - 7), 0.0)
    return float((ulp / 4).mean()) if a.size else 0.0


def log_stats(kind, what, stats):
    """Append one JSON line per check to $USP_PARITY_LOG (when set), so a GPU
    run leaves the raw errors of every case beside the pass/fail verdict."""
    path = os.environ.get("USP_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"kind": kind, "case": what, **stats}) + "\n")


def check_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what="", out_bf16=False):
    """o arrays in the same layout; lse arrays in the same layout.

    ``out_bf16``: o was rounded to bf16 by the kernel.  The max-abs bar stays
    the flat 1e-2 wherever |o_ref| < 2, where a correctly rounded output
    misses the exact value by at most 2^-8 (0.0039) and the bar is left to
    the kernel's own error.  Only where |o_ref| >= 2 does it add half a bf16
    spacing of the exact value, which rounding alone may cost there (0.0078
    in [2, 4), more than the bar itself from 4 on).  The mean-abs bar adds
    the expected error of that rounding, a quarter spacing averaged
    (negligible where |o| << 1, as in the long-sequence workloads; about 1e-3
    on rows that average only a few values and |o| ~ 1).  The raw errors are
    returned (and logged) whatever the bars."""
    omax_tol, omean_tol, lse_tol = TOL[dtype]
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    omax_bar = np.full(o_ref.shape, omax_tol)
    if out_bf16:
        omean_tol = omean_tol + bf16_rounding_floor(o_ref)
        a = np.abs(o_ref)
        big = a >= 2.0
        omax_bar = np.where(big, omax_tol + 2.0 ** (np.floor(np.log2(np.where(big, a, 1.0))) - 8), omax_tol)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite o"
    ninf_g, ninf_r = np.isneginf(lse_gpu), np.isneginf(lse_ref)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf rows differ"
    assert not np.any(np.isnan(lse_gpu)), f"{what}: NaN lse"
    d = np.abs(o_gpu - o_ref)
    dl = np.abs(np.where(ninf_r, 0.0, lse_gpu - np.where(ninf_r, 0.0, lse_ref)))
    stats = dict(o_max=float(d.max()) if d.size else 0.0, o_mean=float(d.mean()) if d.size else 0.0,
                 lse_max=float(dl.max()) if dl.size else 0.0,
                 o_max_below2=float(d[np.abs(o_ref) < 2].max()) if np.any(np.abs(o_ref) < 2) else 0.0,
                 o_frac_of_bar=float((d / omax_bar).max()) if d.size else 0.0, o_mean_bar=float(omean_tol))
    log_stats("fwd", what, stats)
    assert np.all(d <= omax_bar), f"{what}: {stats}"
    assert stats["o_mean"] <= omean_tol, f"{what}: {stats}"
    assert stats["lse_max"] <= lse_tol, f"{what}: {stats}"
    return stats


def guarded(shape, dtype, dev, fill=0):
    """A tensor followed by a canary tail; returns (view, check_fn)."""
    n = int(np.prod(shape))
    tail = 4096
    buf = torch.full((n + tail,), fill, dtype=dtype, device=dev)
    canary = torch.full((tail,), -7, dtype=dtype, device=dev)
    buf[n:] = canary

    def intact():
        return bool(torch.equal(buf[n:], canary))
    return buf[:n].view(shape), intact


def sample_rows(L, c, n_random, seed, extra=()):
    """Local row indices: the edges of both chunks, optional extra rows and a
    seeded random set."""
    rng = np.random.default_rng(seed)
    base = {0, 1, c - 1, c, c + 1, L - 2, L - 1, *extra}
    base |= set(rng.choice(L, size=min(n_random, L), replace=False).tolist())
    return np.array(sorted(i for i in base if 0 <= i < L))


# Gradient bar (the backward): normwise relative error and worst element
# relative to the largest reference magnitude, per tensor.  bf16 -- the
# kernels round P and dS to bf16 (relative error up to 2^-8) before the
# fp32-accumulated products and take delta from the bf16 O, so errors of one
# to two 2^-8 of the gradient's scale are expected where rows see few keys
# (measured at worst: 5.9e-3 normwise, 8.9e-3 worst element); fp32 -- double
# internally, with lse and delta passed as fp32 (relative 2^-24 of |lse| on
# P), a few 1e-7 (measured at worst: 3.7e-7 and 4.6e-7).
GTOL = {"bf16": (1e-2, 2e-2), "fp32": (1e-6, 2e-6)}


def check_grad(g_gpu, g_ref, dtype, what=""):
    g = np.asarray(g_gpu, dtype=np.float64)
    r = np.asarray(g_ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    nrm_tol, max_tol = GTOL[dtype]
    scale = float(np.abs(r).max()) if r.size else 0.0
    if scale == 0.0:
        assert np.all(g == 0), f"{what}: expected zeros"
        return dict(norm=0.0, max=0.0)
    d = g - r
    stats = dict(norm=float(np.linalg.norm(d) / np.linalg.norm(r)), max=float(np.abs(d).max() / scale))
    log_stats("grad_" + dtype, what, stats)
    assert stats["norm"] <= nrm_tol and stats["max"] <= max_tol, f"{what}: {stats}"
    return stats
