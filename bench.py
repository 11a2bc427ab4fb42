#!/usr/bin/env python3
"""Benchmark: one GPU's share of USP-Attention at the 128K-token hybrid
workload (S = 131072, 32 query heads, 8 KV heads, head dim 128, bf16, ring
degree 4 x Ulysses degree 2), on one MI355X.

A step is the per-GPU hot path (OneGpuShare.step): zigzag extract of Q, K, V,
Ulysses layout of Q, K, V, the fused ring walk over 4 KV blocks (attention
+ LSE merge + bf16 epilogue) and the inverse layout of O.  Inputs are seeded
synthetic tensors already resident in HBM; the peers' pieces (other ring
ranks' KV blocks, the other Ulysses rank's shards and output) are produced
once before timing.

Prints one JSON line.  ``value`` is causal-effective attention TFLOP/s over
the whole step; ``roofline`` rates the dominant kernel (the ring walk)
against the bf16 dense MFMA peak using HIP-event times of that kernel alone;
``kernels`` rates each kernel of the step; ``cpu_baseline`` is the fp64
oracle on a bounded row sample of the same workload, timed on the host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "usp_hybrid_s128k_ud2_rd4"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WALK_KERNEL = "attn_bf16_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_walk_usp_hybrid_s128k.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--ring-rank", type=int, default=0)
    p.add_argument("--ulysses-rank", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads' timings")
    p.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    p.add_argument("--cpu-rows", type=int, default=384, help="query rows of the oracle sample")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (for scaling HBM byte counters)")
    p.add_argument("--calls-per-rep", type=int, default=0,
                   help="calls per timed repetition of a short launch (0: enough for about 2 ms); a fixed count "
                        "gives counter runs the same dispatch sequence")
    p.add_argument("--only-workloads", action="store_true",
                   help="only the other configurations' launches (for profiling them), no oracle")
    return p.parse_args()


def share_walk_flops(D, heads, B, rd, c):
    """Work of one ring rank's walk over its zigzag share (chunks r and
    2 rd - 1 - r of c rows each) against all 2 rd chunks of keys, at 4 D flops
    per visible (query, key) pair: the half-diagonal convention counts
    2 rd c^2 pairs per head (each chunk-pair cell c^2, the two diagonal cells
    c^2 / 2 each), the exact count 2 rd c^2 + c (the diagonals' c (c + 1) / 2).
    Returns (half-diagonal, exact) flops; the same on every rank."""
    return 4.0 * D * heads * B * 2 * rd * c * c, 4.0 * D * heads * B * (2 * rd * c * c + c)


def per_sample_pairs(cu, rd):
    """Visible pairs of one rank's per-sample share (every sample of length
    n = 2 rd m cut into 2 rd chunks, the rank holding chunks r and
    2 rd - 1 - r of each), under the causal same-sample mask: per sample
    (2 rd - 1) m^2 + m (m + 1), the same on every rank."""
    import numpy as np
    m = np.diff(np.asarray(cu)).astype(np.int64) // (2 * rd)
    return int(((2 * rd - 1) * m * m + m * (m + 1)).sum())


def copy_calibration(mib):
    """A plain torch device-to-device copy of known size, three times; its
    FETCH_SIZE / WRITE_SIZE counters give the factor between counted and
    moved bytes."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))


WALK_SOURCES = ("attn_bf16.hip", "attn_tiles.h", "positions.h")


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the walk kernel's sources, in order."""
    h = hashlib.sha256()
    for name in WALK_SOURCES:
        h.update(open(os.path.join(ROOT, "sequence_ring_attention_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per walk launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def plain_copy_reference(nbytes):
    """A plain torch device copy of the size of one layout launch, with a
    1 GiB buffer written between repetitions so the 256 MB last-level cache
    does not serve it: the practical ceiling of a read+write stream here."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    flush = torch.empty(2**30, dtype=torch.uint8, device="cuda:0")
    times = []
    for _ in range(9):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    return {"bytes": 2 * nbytes, "ms": ms, "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": 2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


_CALLS_PER_REP = [0]


def _timed(fn, reps=20, batch_ms=2.0):
    """HIP-event times (ms) of fn() on the current stream after one untimed
    call: median, min and max over ``reps`` repetitions of the time per call.
    A call shorter than ``batch_ms`` is timed as a run of back-to-back calls
    between one pair of events (as a ring loop issues its launches), so that
    the events' own latency, tens of microseconds, does not count against a
    kernel that runs for a fraction of a millisecond."""
    import torch

    def run(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    fn()
    torch.cuda.synchronize()
    per = 1
    est = run(1)
    if _CALLS_PER_REP[0] > 0:
        per = _CALLS_PER_REP[0]
    elif est < batch_ms:
        per = min(16, max(1, int(batch_ms / max(est, 1e-3))))
    out = sorted(run(per) for _ in range(reps))
    return {"ms": out[len(out) // 2], "ms_min": out[0], "ms_max": out[-1], "reps": reps, "calls_per_rep": per}


def _time(fn, reps=20):
    """Median HIP-event time (ms) of fn() on the current stream."""
    return _timed(fn, reps)["ms"]


def _rate(t, flops):
    """A timing dict from _timed with the causal-effective rate of `flops`."""
    t = dict(t)
    t["TFLOP/s"] = flops / (t["ms"] * 1e-3) / 1e12
    t["frac_mfma"] = t["TFLOP/s"] / PEAK_BF16_TFLOPS
    return t


def clock_during(fn, min_snapshots=3, max_seconds=8.0):
    """The shader clock while fn() runs back to back: the firmware's gfx clock
    (amdsmi gpu metrics: the mean over XCDs of current_gfxclks, MHz).  The
    firmware refreshes that table about once a second (its
    system_clock_counter moves in steps), so the table is polled every 10 ms
    and each refresh counted once; the snapshot already there when the
    launches start predates them and is dropped.  fn() runs until
    `min_snapshots` refreshes were seen or `max_seconds` passed.  Median, min
    and max of the snapshots, or the reason it could not be read."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
        amdsmi.amdsmi_get_gpu_metrics_info(h)
    except Exception as e:                      # no amdsmi or no access: say so
        return {"mhz": None, "error": repr(e)[:200]}

    def snapshot():
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if xs:
            mhz = sum(xs) / len(xs)
        elif isinstance(m.get("current_gfxclk"), (int, float)):
            mhz = float(m["current_gfxclk"])
        else:
            mhz = None
        return m.get("system_clock_counter"), mhz

    fn()
    torch.cuda.synchronize()
    seen, snaps, stop = set(), [], threading.Event()
    try:
        seen.add(snapshot()[0])                 # the refresh before the launches
    except Exception:
        pass

    def poll():
        while not stop.is_set():
            try:
                stamp, mhz = snapshot()
                if stamp not in seen:
                    seen.add(stamp)
                    if mhz is not None:
                        snaps.append(mhz)
            except Exception:
                pass
            time.sleep(0.01)

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while len(snaps) < min_snapshots and time.perf_counter() - t0 < max_seconds:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not snaps:
        return {"mhz": None, "error": "no refresh of the gpu metrics table while the launches ran"}
    xs = sorted(snaps)
    return {"mhz": xs[len(xs) // 2], "mhz_min": xs[0], "mhz_max": xs[-1], "snapshots": len(xs),
            "seconds": time.perf_counter() - t0,
            "source": "amdsmi gpu metrics current_gfxclks, mean over XCDs, one value per table refresh",
            "launches": n}


def host_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def oracle_rows(w, q, k, v, rows_pos, cu=None, heads=None):
    """The fp64 oracle on query positions `rows_pos` against the whole
    sequence, timed on the host: (o, lse, seconds, causal-effective flops)."""
    import numpy as np
    import torch
    from oracle import attention as oa
    from oracle import index as ix
    h0, h1 = heads if heads else (0, w.H)
    g = w.H // w.Hkv
    qn = q[:, :, h0:h1].to(torch.float64).numpy()
    kn = k[:, :, h0 // g:h1 // g].to(torch.float64).numpy()
    vn = v[:, :, h0 // g:h1 // g].to(torch.float64).numpy()
    seg = None if cu is None else ix.segment_start(cu, rows_pos)
    t0 = time.perf_counter()
    o, lse = oa.masked_attention(qn[:, rows_pos], kn, vn, w.scale, q_pos=rows_pos, q_seg_start=seg)
    dt = time.perf_counter() - t0
    start = np.zeros_like(rows_pos) if cu is None else seg
    pairs = int((np.asarray(rows_pos) - start + 1).sum())
    return o, lse, dt, 4.0 * w.D * (h1 - h0) * w.B * pairs


def baseline_entry(dt, flops, unit_flops, what, errors=None):
    """One cpu_baseline object: the oracle's rate on its sample and the
    sample time scaled to the configuration's whole unit (labelled as an
    extrapolation)."""
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "kind": "oracle",
            "sample": what, "seconds": dt, "sample_tflop": flops / 1e12,
            "extrapolated_unit_seconds": dt * unit_flops / flops, "extrapolation": "sample time x unit/sample flops",
            "host_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "gpu_vs_oracle": errors}


def compare(o_gpu, lse_gpu, o_ref, lse_ref):
    """Errors of the GPU rows against the oracle's.  Beside the plain maxima:
    |o_ref| where the largest o error sits, and the largest o error where
    |o_ref| < 2 (above 2, the bf16 rounding of the output alone reaches half a
    spacing of 2^-7 |o_ref|, which the parity tests add to the 1e-2 bar)."""
    import numpy as np
    eo, el = np.abs(o_gpu - o_ref), np.abs(lse_gpu - lse_ref)
    i = int(np.argmax(eo))
    small = np.abs(o_ref) < 2.0
    return {"o_max_abs": float(eo.max()), "o_mean_abs": float(eo.mean()), "lse_max_abs": float(el.max()),
            "o_ref_abs_at_o_max": float(np.abs(o_ref).reshape(-1)[i]),
            "o_max_abs_where_ref_below_2": float(eo[small].max()) if small.any() else 0.0,
            "bars": {"o_max_abs": 1e-2, "o_mean_abs": 1e-3, "lse_max_abs": 1e-3}}


def worst_of(errs):
    """The worst of several compare() results (|o_ref| at the overall max)."""
    keys = ("o_max_abs", "o_mean_abs", "lse_max_abs", "o_max_abs_where_ref_below_2")
    worst = {kk: max(e[kk] for e in errs) for kk in keys}
    worst["o_ref_abs_at_o_max"] = max(errs, key=lambda e: e["o_max_abs"])["o_ref_abs_at_o_max"]
    worst["bars"] = errs[0]["bars"]
    return worst


def index_oracle_copies():
    """The CPU index oracle's copies timed on the host (bytes read + written
    per second): the zigzag split of every rank of the 32K GQA workload's Q
    (256 MiB) and the Ulysses layout of the 128K share's Q shards (256 MiB),
    NumPy gathers of the bf16 bits."""
    import numpy as np
    from oracle import index as ix
    rng = np.random.default_rng(7)
    out = {}
    x = rng.integers(-32768, 32767, size=(1, 32768, 32, 128), dtype=np.int16)
    t0 = time.perf_counter()
    ix.zigzag_extract_all(x, 8, 1)
    dt = time.perf_counter() - t0
    out["zigzag_extract_all_ranks_q_gqa_s32k_cp8"] = {"bytes": 2 * x.nbytes, "seconds": dt,
                                                      "GB/s": 2 * x.nbytes / dt / 1e9}
    shards = [rng.integers(-32768, 32767, size=(1, 16384, 32, 128), dtype=np.int16) for _ in range(2)]
    t0 = time.perf_counter()
    ix.ulysses_fwd(shards, 0)
    ix.ulysses_fwd(shards, 1)
    dt = time.perf_counter() - t0
    nb = 2 * sum(s.nbytes for s in shards)
    out["ulysses_layout_fwd_q_usp_hybrid_s128k"] = {"bytes": nb, "seconds": dt, "GB/s": nb / dt / 1e9}
    out["kind"] = "oracle"
    out["cores"] = 1
    return out


_FLUSH = []


def _time_flushed(fn, nbytes, reps=20):
    """HIP-event times of fn() with a 1 GiB buffer written before every
    repetition, so the 256 MB last-level cache holds none of fn's data:
    median, min and max ms, and the median rate for `nbytes` moved."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.empty(2**30, dtype=torch.uint8, device="cuda:0"))
    flush = _FLUSH[0]
    fn()
    times = []
    for _ in range(reps):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    ms = times[len(times) // 2]
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bytes": nbytes, "ms": ms, "ms_min": times[0], "ms_max": times[-1], "GB/s": gbs,
            "frac_hbm": gbs / PEAK_HBM_GBS, "reps": reps}


def copy_launches(share, w):
    """Each copy entry point and the merge as one launch at the bench
    workload's sizes, timed with the last-level cache flushed: the zigzag
    extract of the whole Q for every (ring, Ulysses) rank and its inverse,
    one rank's extract, the step's batched extract and layout of the share's
    Q, K and V, the Ulysses layout of the ring group's Q shards for both
    Ulysses ranks and its inverse, and the LSE merge of one step's partials
    of the share."""
    import torch
    from sequence_ring_attention_amd import binding as B
    Q, rd, ud = share.Q, w.rd, w.ud
    e = Q.element_size()
    res = {}
    allz = torch.empty((rd * ud,) + tuple(share.qz.shape[1:]), dtype=Q.dtype, device=Q.device)
    res["zigzag_extract_all_ranks_q"] = _time_flushed(lambda: B.usp_zigzag_extract(Q, allz, rd, ud, -1, -1),
                                                      2 * Q.numel() * e)
    back = torch.empty_like(Q)
    res["zigzag_extract_inverse_all_ranks_q"] = _time_flushed(
        lambda: B.usp_zigzag_extract(allz, back, rd, ud, -1, -1, inverse=True), 2 * Q.numel() * e)
    del allz, back
    one = torch.empty_like(share.qz[0])
    res["zigzag_extract_one_rank_q"] = _time_flushed(lambda: B.usp_zigzag_extract(Q, one, rd, ud, 0, 0),
                                                     2 * one.numel() * e)
    del one
    # the step's two batched launches: Q, K and V of the share together
    r, u = share.r, share.u
    qkv_out = (share.qz[u], share.kz[u], share.vz[u])
    res["zigzag_extract_one_rank_qkv"] = _time_flushed(
        lambda: B.usp_zigzag_extract_n((Q, share.K, share.V), qkv_out, rd, ud, r, u),
        2 * sum(t.numel() for t in qkv_out) * e)
    qkv_hm = (share.qh[u], share.kh[u, r], share.vh[u, r])
    res["ulysses_layout_fwd_one_rank_qkv"] = _time_flushed(
        lambda: B.usp_ulysses_a2a_layout_n((share.qz, share.kz, share.vz), qkv_hm, ud, u),
        2 * sum(t.numel() for t in qkv_hm) * e)
    res["ulysses_layout_fwd_all_q"] = _time_flushed(lambda: B.usp_ulysses_a2a_layout(share.qz, share.qh, ud, -1),
                                                    2 * share.qz.numel() * e)
    outs = torch.empty((ud,) + tuple(share.out.shape), dtype=Q.dtype, device=Q.device)
    res["ulysses_layout_inv_all_o"] = _time_flushed(
        lambda: B.usp_ulysses_a2a_layout(share.oh, outs, ud, -1, inverse=True), 2 * share.oh.numel() * e)
    del outs
    hb, L = w.H // ud, w.S // rd
    rows = hb * w.B * L
    acc = torch.zeros(hb, w.B, L, w.D, dtype=torch.float32, device=Q.device)
    lacc = torch.zeros(hb, w.B, L, dtype=torch.float32, device=Q.device)
    ost, lst = torch.zeros_like(acc), torch.zeros_like(lacc)
    res["lse_merge_step"] = _time_flushed(lambda: B.usp_lse_merge(acc, lacc, ost, lst),
                                          3 * rows * w.D * 4 + 3 * rows * 4)
    return res


def other_share_walk(Q, K, V, w, r, u, flops, steps=20):
    """The walk of another ring rank's share of the same grid (every share
    holds the same causal work under the zigzag split)."""
    import torch
    from sequence_ring_attention_amd.pipeline import OneGpuShare
    sh = OneGpuShare(Q, K, V, w.rd, w.ud, r, u)
    sh.prepare_peers()
    sh.step()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(5)] for _ in range(steps)]
    for s in range(steps):
        sh.step(marks[s])
    torch.cuda.synchronize()
    walk = sorted(marks[s][2].elapsed_time(marks[s][3]) for s in range(steps))
    ms = walk[len(walk) // 2]
    return {"share": {"ring_rank": r, "ulysses_rank": u}, "walk_ms": ms, "walk_ms_min": walk[0],
            "walk_ms_max": walk[-1], "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_mfma": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def head_chunk_steps(Q, K, V, w, r, u, flops, whole_ms, whole_bytes, chunks=(8, 4, 2), overlapped=(4, 2), split=(2,),
                     steps=20):
    """The share stepped with its head block pushed through in chunks
    (headwise chunking): step time and the head-major bytes the chunks in
    flight work on, beside the whole block's; chunks run one after another,
    and for ``overlapped`` also alternating between two streams; for
    ``split`` on one stream with the split walk."""
    import torch
    from sequence_ring_attention_amd.pipeline import OneGpuShare
    res = {"whole_block": {"heads": w.H // w.ud, "ms": whole_ms, "TFLOP/s": flops / (whole_ms * 1e-3) / 1e12,
                           "head_major_bytes": whole_bytes}}
    runs = [(nh, False, False) for nh in chunks] + [(nh, True, False) for nh in overlapped] + \
           [(nh, False, True) for nh in split]
    for nh, ov, sp in runs:
        sh = OneGpuShare(Q, K, V, w.rd, w.ud, r, u, head_chunk=nh, overlap_chunks=ov, split_walk=sp)
        sh.prepare_peers()
        sh.step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            sh.step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        res[f"chunks_of_{nh}" + ("_two_streams" if ov else "") + ("_split_walk" if sp else "")] = {
                                  "heads": nh, "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                                  "head_major_bytes": sh.head_major_bytes(),
                                  "head_major_fraction": sh.head_major_bytes() / whole_bytes,
                                  "step_time_ratio": ms / whole_ms}
        if sp:
            res[f"chunks_of_{nh}_split_walk"]["split_workspace_bytes"] = sum(t.numel() for t in sh._ws.values())
        del sh
        torch.cuda.empty_cache()
    return res


def packed_pairs(cu, pos):
    """Visible (query, key) pairs of queries at `pos` under the causal
    same-sample mask: a query at p sees p - start(sample of p) + 1 keys."""
    import numpy as np
    start = np.asarray(cu)[np.searchsorted(cu, pos, side="right") - 1]
    return int((np.asarray(pos) - start + 1).sum())


def extra_workloads(cpu=True):
    """The other configurations, each launch timed on its own (20 reps: median,
    min, max): the tiny fp32 workload's walk of every rank, the 8K MHA walk of
    every rank in one launch, the 32K GQA walk of ranks 0 and 7 (zigzag
    balance) with rank 0's per-step launches and merges, and the packed 32K
    walk of each rank.  With ``cpu``, each configuration's unit is also run
    through the fp64 oracle on a seeded row sample (the tiny workload whole),
    timed on the host and compared with the GPU's rows."""
    import numpy as np
    import torch
    from sequence_ring_attention_amd import binding as B
    from sequence_ring_attention_amd import inputs
    from oracle import index as ix
    dev = torch.device("cuda:0")
    res = {}

    def zig_shares(x, rd):
        out = torch.empty((rd, 1) + (x.shape[0], x.shape[1] // rd) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
        B.usp_zigzag_extract(x, out, rd, 1, -1, -1)
        return out[:, 0]                                       # (rd, B, 2c, H, D)

    def gpu_rows(o, lse, rows):
        """(B, n, H, D) o and (H, B, n) lse of local rows of one rank, as float64 numpy."""
        rt = torch.from_numpy(np.asarray(rows)).to(dev)
        return (o.index_select(1, rt).double().cpu().numpy(), lse.index_select(2, rt).double().cpu().numpy())

    def pick(w, r, n, seed, extra=()):
        rng = np.random.default_rng(seed)
        c = w.chunk
        base = {0, c - 1, c, 2 * c - 1, *extra} | set(rng.choice(w.share, size=n, replace=False).tolist())
        return np.array(sorted(i for i in base if 0 <= i < w.share))

    print("[bench] workload: tiny causal MHA", file=sys.stderr, flush=True)
    # tiny causal MHA, fp32, cp = 4: every rank in one launch; the oracle runs the whole unit
    w = inputs.WORKLOADS["tiny_causal_mha_fp32_s256_cp4"]
    q, k, v = inputs.workload_qkv(w)
    qs, ks, vs = zig_shares(q.to(dev), w.rd), zig_shares(k.to(dev), w.rd), zig_shares(v.to(dev), w.rd)
    o = torch.empty_like(qs)
    lse = torch.empty(w.rd, w.H, w.B, w.share, dtype=torch.float32, device=dev)
    d = B.attn_desc(w.S, w.rd, qs, ks, vs, o=o, all_ranks=True)
    fl = 2.0 * w.B * w.H * w.S * w.S * w.D
    entry = {"all_ranks_walk": _rate(_timed(lambda: B.usp_attn_fwd(qs, ks, vs, o, lse, d, -1)), fl),
             "TFLOP": fl / 1e12, "note": "latency-bound, not rated against the roofline"}
    if cpu:
        from oracle import attention as oa
        t0 = time.perf_counter()
        o_ref, l_ref = oa.attention_full(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.scale)
        dt = time.perf_counter() - t0
        err = []
        for r in range(w.rd):
            p = ix.zigzag_share_positions(w.S, w.rd, r)
            err.append(compare(o[r].double().cpu().numpy(), lse[r].double().cpu().numpy(), o_ref[:, p],
                               l_ref[:, :, p]))
        worst = worst_of(err)
        worst["bars"] = {"o_max_abs": 2e-5, "o_mean_abs": 1e-6, "lse_max_abs": 1e-6}
        exact = 4.0 * w.D * w.H * w.B * (w.S * (w.S + 1) // 2)
        entry["cpu_baseline"] = baseline_entry(dt, exact, exact, "the whole unit: one-shot fp64 attention of all "
                                               f"{w.S} tokens (every rank and step), {dt * 1e3:.1f} ms", worst)
    res[w.name] = entry

    print("[bench] workload: 8K causal MHA", file=sys.stderr, flush=True)
    # 8K causal MHA, cp = 4, every rank in one launch
    w = inputs.WORKLOADS["causal_mha_s8k_cp4"]
    q, k, v = inputs.workload_qkv(w)
    qs, ks, vs = zig_shares(q.to(dev), w.rd), zig_shares(k.to(dev), w.rd), zig_shares(v.to(dev), w.rd)
    o = torch.empty_like(qs)
    lse = torch.empty(w.rd, w.H, w.B, w.share, dtype=torch.float32, device=dev)
    d = B.attn_desc(w.S, w.rd, qs, ks, vs, o=o, all_ranks=True)
    fl = 2.0 * w.B * w.H * w.S * w.S * w.D
    t = _rate(_timed(lambda: B.usp_attn_fwd(qs, ks, vs, o, lse, d, -1)), fl)
    entry = {"all_ranks_walk": t, "all_ranks_walk_ms": t["ms"], "TFLOP": fl / 1e12, "TFLOP/s": t["TFLOP/s"]}
    if cpu:
        dt = fls = 0.0
        err = []
        for r in range(w.rd):
            rows = pick(w, r, 24, 60 + r)
            pos = ix.zigzag_share_positions(w.S, w.rd, r)[rows]
            o_ref, l_ref, dtr, flr = oracle_rows(w, q, k, v, pos)
            dt, fls = dt + dtr, fls + flr
            err.append(compare(*gpu_rows(o[r], lse[r], rows), o_ref, l_ref))
        worst = worst_of(err)
        worst["bars"] = err[0]["bars"]
        entry["cpu_baseline"] = baseline_entry(dt, fls, fl, f"about 28 seeded rows (chunk edges included) of every "
                                               f"rank x {w.H} heads vs all {w.S} keys, fp64 numpy", worst)
    res[w.name] = entry

    print("[bench] workload: 32K causal GQA", file=sys.stderr, flush=True)
    # 32K causal GQA, cp = 8: ranks 0 and 7 (walk), rank 0 step by step + merges
    w = inputs.WORKLOADS["causal_gqa_s32k_cp8"]
    q, k, v = inputs.workload_qkv(w)
    qd = q.to(dev)
    qs, ks, vs = zig_shares(qd, w.rd), zig_shares(k.to(dev), w.rd), zig_shares(v.to(dev), w.rd)
    fl_rank = share_walk_flops(w.D, w.H, w.B, w.rd, w.chunk)[0]
    entry = {"TFLOP_per_rank": fl_rank / 1e12}
    qz = torch.empty((w.rd, 1) + tuple(qs.shape[1:]), dtype=q.dtype, device=dev)
    entry["zigzag_extract_all_ranks_q"] = _time_flushed(lambda: B.usp_zigzag_extract(qd, qz, w.rd, 1, -1, -1),
                                                        2 * q.numel() * q.element_size())
    del qz
    for r in (0, w.rd - 1):
        qr = qs[r].contiguous()
        o = torch.empty_like(qr)
        lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
        d = B.attn_desc(w.S, w.rd, qr, ks, vs, o=o)
        t = _rate(_timed(lambda: B.usp_attn_fwd(qr, ks, vs, o, lse, d, r)), fl_rank)
        entry[f"rank{r}_walk"] = t
        entry[f"rank{r}_walk_ms"] = t["ms"]
        entry[f"rank{r}_TFLOP/s"] = t["TFLOP/s"]
        if cpu:
            rows = pick(w, r, 32, 70 + r)
            pos = ix.zigzag_share_positions(w.S, w.rd, r)[rows]
            o_ref, l_ref, dt, fls = oracle_rows(w, q, k, v, pos)
            entry[f"rank{r}_cpu_baseline"] = baseline_entry(
                dt, fls, fl_rank, f"{len(rows)} seeded rows (chunk edges included) of rank {r} x {w.H} heads vs "
                f"all {w.S} keys, fp64 numpy", compare(*gpu_rows(o, lse, rows), o_ref, l_ref))
    qr = qs[0].contiguous()
    acc = torch.zeros(w.H, w.B, w.share, w.D, dtype=torch.float32, device=dev)
    lacc = torch.zeros(w.H, w.B, w.share, dtype=torch.float32, device=dev)
    ost, lst = torch.empty_like(acc), torch.empty_like(lacc)
    d = B.attn_desc(w.S, w.rd, qr, ks, vs)
    steps = [_rate(_timed(lambda t=t: B.usp_ring_attn_step_fwd(qr, ks, vs, ost, lst, d, 0, t)), fl_rank / w.rd)
             for t in range(w.rd)]
    rows = w.H * w.B * w.share
    merge = _time_flushed(lambda: B.usp_lse_merge(acc, lacc, ost, lst), 3 * rows * w.D * 4 + 3 * rows * 4)
    entry["rank0_steps"] = steps
    entry["rank0_whole_ring"] = ring_forms(
        lambda t, o_, l_: B.usp_ring_attn_step_fwd(qr, ks, vs, o_, l_, d, 0, t),
        lambda t, o_, l_: B.usp_ring_attn_step_fwd_merge(qr, ks, vs, o_, l_, d, 0, t),
        lambda: B.usp_lse_merge(acc, lacc, ost, lst), w.rd, acc, lacc, ost, lst, fl_rank)
    entry["rank0_step_ms"] = [x["ms"] for x in steps]
    entry["rank0_step_TFLOP/s"] = [x["TFLOP/s"] for x in steps]
    entry["merge"] = merge
    entry["merge_ms"] = merge["ms"]
    entry["merge_GB/s"] = merge["GB/s"]
    entry["merge_frac_hbm"] = merge["frac_hbm"]
    res[w.name] = entry
    del qs, ks, vs, acc, lacc, ost, lst, qd

    print("[bench] workload: packed variable-length 32K", file=sys.stderr, flush=True)
    # packed variable-length 32K, cp = 4: each rank
    w = inputs.WORKLOADS["packed_varlen_s32k_cp4"]
    q, k, v = inputs.workload_qkv(w)
    cu = inputs.workload_cu_seqlens(w)
    cu_t = torch.from_numpy(cu).to(dev)
    qs, ks, vs = zig_shares(q.to(dev), w.rd), zig_shares(k.to(dev), w.rd), zig_shares(v.to(dev), w.rd)
    entry = {"num_samples": len(cu) - 1}
    c = w.chunk
    cpu_dt = cpu_fl = unit_fl = 0.0
    errs = []
    for r in range(w.rd):
        share_pos = np.concatenate([np.arange(r * c, (r + 1) * c), np.arange((2 * w.rd - 1 - r) * c, (2 * w.rd - r) * c)])
        fl = 4.0 * w.D * w.H * w.B * packed_pairs(cu, share_pos)
        unit_fl += fl
        qr = qs[r].contiguous()
        o = torch.empty_like(qr)
        lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
        d = B.attn_desc(w.S, w.rd, qr, ks, vs, o=o, cu_seqlens=cu_t)
        t = _rate(_timed(lambda: B.usp_attn_fwd(qr, ks, vs, o, lse, d, r)), fl)
        entry[f"rank{r}"] = {"TFLOP": fl / 1e12, **t}
        if cpu:
            edges = [int(i) for b in cu[1:-1] for i in np.nonzero(np.abs(share_pos - b) <= 1)[0]]
            rows = pick(w, r, 16, 80 + r, extra=edges)
            o_ref, l_ref, dt, fls = oracle_rows(w, q, k, v, share_pos[rows], cu=cu)
            cpu_dt, cpu_fl = cpu_dt + dt, cpu_fl + fls
            errs.append(compare(*gpu_rows(o, lse, rows), o_ref, l_ref))
    if cpu:
        worst = worst_of(errs)
        entry["cpu_baseline"] = baseline_entry(cpu_dt, cpu_fl, unit_fl, f"about 22 seeded rows (sample and chunk "
                                               f"edges included) of every rank x {w.H} heads, fp64 numpy", worst)
    res[w.name] = entry
    print("[bench] workload: packed 32K, both splits", file=sys.stderr, flush=True)
    res[w.name + "_split_balance"] = split_balance(w, q.to(dev), k.to(dev), v.to(dev), zig_shares)
    return res


def sample_rows(w, n_rows):
    """The seeded query rows (local rows of a share) of the oracle sample."""
    import numpy as np
    rng = np.random.default_rng(1234)
    return np.sort(rng.choice(w.S // w.rd, size=n_rows, replace=False))


def gpu_sample(share, w, n_rows):
    """The sample rows of the share's outputs after a step, on the host:
    o (B, n, hb, D) from the head-major bf16 output and lse (hb, B, n)."""
    import torch
    rows = torch.from_numpy(sample_rows(w, n_rows)).to(share.oh.device)
    u = share.u
    o = share.oh[u].index_select(2, rows).to(torch.float64).cpu().numpy().transpose(1, 2, 0, 3)
    lse = share.lse[u].index_select(2, rows).to(torch.float64).cpu().numpy()
    return o, lse


def cpu_baseline(w, r, u, n_rows, gpu=None):
    """The oracle as it stands on a bounded sample: n_rows query rows of this
    share (all its heads) against the whole sequence, fp64 on the host.  With
    ``gpu`` (the same rows of a step's GPU output, from gpu_sample), o (bf16)
    and lse are compared with the oracle's: max and mean abs error."""
    import numpy as np
    import torch
    from oracle import attention as oa
    from oracle import index as ix
    from sequence_ring_attention_amd import inputs
    q, k, v = inputs.workload_qkv(w)
    hb = w.H // w.ud
    qn = q[:, :, u * hb:(u + 1) * hb].to(torch.float64).numpy()
    kv_lo, kv_hi = u * (w.Hkv // w.ud), (u + 1) * (w.Hkv // w.ud)
    kn = k[:, :, kv_lo:kv_hi].to(torch.float64).numpy()
    vn = v[:, :, kv_lo:kv_hi].to(torch.float64).numpy()
    pos = ix.zigzag_share_positions(w.S, w.rd, r)
    rows = sample_rows(w, n_rows)
    qp = pos[rows]
    t0 = time.perf_counter()
    o_ref, l_ref = oa.masked_attention(qn[:, qp], kn, vn, w.scale, q_pos=qp)   # (B, n, hb, D), (hb, B, n)
    dt = time.perf_counter() - t0
    errors = None
    if gpu is not None:
        errors = {"rows": int(n_rows), "heads": hb, **compare(gpu[0], gpu[1], o_ref, l_ref)}
    pairs = int((qp + 1).sum())                       # causal: position p sees p + 1 keys
    flops = 4.0 * w.D * hb * w.B * pairs
    share_flops = share_walk_flops(w.D, hb, w.B, w.rd, w.chunk)[0]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "kind": "oracle",
            "extrapolated_unit_seconds": dt * share_flops / flops,
            "sample": f"{n_rows} random query rows of share (r={r}, u={u}) x {hb} heads vs all "
                      f"{w.S} keys, fp64 numpy, {dt:.2f} s, {flops / 1e9:.1f} GFLOP causal-effective",
            "seconds": dt, "host_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "gpu_vs_oracle": errors}


def split_balance(w, q, k, v, zig_shares):
    """The packed workload's samples with lengths rounded down to multiples
    of 2 cp, walked by every rank under both splits of the shares: Algorithm
    2 on the whole packed stream, and on every sample (usp_zigzag_extract_varlen);
    each rank's forward walk and its backward.  A real ring waits for its
    slowest rank each step, so the figure of merit is the slowest rank's time
    against the mean."""
    import numpy as np
    import torch
    from sequence_ring_attention_amd import binding as B
    from sequence_ring_attention_amd import inputs
    dev = q.device
    cu = inputs.workload_cu_seqlens(w, multiple=2 * w.rd)
    c = w.chunk
    ps_pairs = per_sample_pairs(cu, w.rd)   # the same on every rank
    out = {"num_samples": len(cu) - 1, "lengths_multiple_of": 2 * w.rd}
    for split in ("stream", "per_sample"):
        if split == "stream":
            qs, ks, vs = zig_shares(q, w.rd), zig_shares(k, w.rd), zig_shares(v, w.rd)
        else:
            def varlen_shares(x):
                o = torch.empty((w.rd, 1, x.shape[0], x.shape[1] // w.rd) + tuple(x.shape[2:]), dtype=x.dtype,
                                device=dev)
                B.usp_zigzag_extract_varlen(x, o, w.rd, 1, -1, -1, cu)
                return o[:, 0]
            qs, ks, vs = varlen_shares(q), varlen_shares(k), varlen_shares(v)
        ranks = []
        for r in range(w.rd):
            if split == "stream":
                pos = np.concatenate([np.arange(r * c, (r + 1) * c),
                                      np.arange((2 * w.rd - 1 - r) * c, (2 * w.rd - r) * c)])
                pairs = packed_pairs(cu, pos)
            else:
                pairs = ps_pairs
            fl = 4.0 * w.D * w.H * w.B * pairs
            qr = qs[r].contiguous()
            o = torch.empty_like(qr)
            lse = torch.empty(w.H, w.B, w.share, dtype=torch.float32, device=dev)
            d = B.attn_desc(w.S, w.rd, qr, ks, vs, o=o, cu_seqlens=cu, zigzag_per_sample=split == "per_sample")
            tf = _timed(lambda: B.usp_attn_fwd(qr, ks, vs, o, lse, d, r))
            ms = tf["ms"]
            # the rank's backward from this forward (2.5 times its work: S, dP, dV, dK, dQ)
            d_o = inputs.randn(tuple(qr.shape), 99, "bf16").to(dev)
            dq = torch.empty_like(qr)
            dk = torch.zeros(ks.shape, dtype=torch.float32, device=dev)
            dv = torch.zeros(vs.shape, dtype=torch.float32, device=dev)
            stats = torch.empty(2 * lse.numel(), dtype=torch.float32, device=dev)
            tb = _timed(lambda: B.usp_attn_bwd(qr, ks, vs, o, d_o, lse, dq, dk, dv, stats, d, r))
            bms = tb["ms"]
            ranks.append({"TFLOP": fl / 1e12, "ms": ms, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
                          "bwd_ms": bms, "bwd_TFLOP/s": 2.5 * fl / (bms * 1e-3) / 1e12,
                          "calls_per_rep": tf["calls_per_rep"], "bwd_calls_per_rep": tb["calls_per_rep"]})
        times = [x["ms"] for x in ranks]
        btimes = [x["bwd_ms"] for x in ranks]
        out[split] = {"ranks": ranks, "slowest_ms": max(times), "mean_ms": sum(times) / len(times),
                      "slowest_over_mean": max(times) / (sum(times) / len(times)),
                      "bwd_slowest_ms": max(btimes), "bwd_slowest_over_mean": max(btimes) / (sum(btimes) / len(btimes))}
    out["slowest_rank_speedup"] = out["stream"]["slowest_ms"] / out["per_sample"]["slowest_ms"]
    out["bwd_slowest_rank_speedup"] = out["stream"]["bwd_slowest_ms"] / out["per_sample"]["bwd_slowest_ms"]
    return out


def ring_steps(share, flops):
    """The share's walk as cp separate ring steps (usp_ring_attn_step_fwd,
    fp32 partials) and LSE merges, each launch timed alone: the step-wise
    form a real ring runs while the next KV block is in flight."""
    import torch
    from sequence_ring_attention_amd import binding as B
    u, r = share.u, share.r
    q, k, v = share.qh[u], share.kh[u], share.vh[u]
    desc = share.desc(u)
    ost = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    lst = torch.empty(tuple(share.lse[u].shape), dtype=torch.float32, device=q.device)
    acc, lacc = torch.zeros_like(ost), torch.full_like(lst, float("-inf"))
    step_ms = [_time(lambda t=t: B.usp_ring_attn_step_fwd(q, k, v, ost, lst, desc, r, t)) for t in range(share.rd)]
    rows = lst.numel()
    merge = _time_flushed(lambda: B.usp_lse_merge(acc, lacc, ost, lst), 3 * rows * q.shape[-1] * 4 + 3 * rows * 4)
    per_step = flops / share.rd
    ring = ring_forms(lambda t, o_, l_: B.usp_ring_attn_step_fwd(q, k, v, o_, l_, desc, r, t),
                      lambda t, o_, l_: B.usp_ring_attn_step_fwd_merge(q, k, v, o_, l_, desc, r, t),
                      lambda: B.usp_lse_merge(acc, lacc, ost, lst), share.rd, acc, lacc, ost, lst, flops)
    return {"step_ms": step_ms, "step_TFLOP/s": [per_step / (m * 1e-3) / 1e12 for m in step_ms],
            "step_frac_mfma": [per_step / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS for m in step_ms],
            "work_per_step_tflop": per_step / 1e12, "merge": merge, "whole_ring": ring}


def ring_forms(step, step_merge, merge, cp, acc, lacc, ost, lst, flops):
    """A rank's whole ring in its two step-wise forms, each timed as one
    sequence of launches: step 0 into the accumulator, then every later step
    as a partial plus usp_lse_merge, or as usp_ring_attn_step_fwd_merge (the
    merge in the step kernel's epilogue, no partial in HBM)."""
    def two_launch():
        step(0, acc, lacc)
        for t in range(1, cp):
            step(t, ost, lst)
            merge()

    def fused():
        step(0, acc, lacc)
        for t in range(1, cp):
            step_merge(t, acc, lacc)
    a, b = _timed(two_launch), _timed(fused)
    return {"two_launch": {**a, "TFLOP/s": flops / (a["ms"] * 1e-3) / 1e12},
            "merge_fused": {**b, "TFLOP/s": flops / (b["ms"] * 1e-3) / 1e12},
            "launches": {"two_launch": 2 * cp - 1, "merge_fused": cp}}


def backward_walk(share, fwd_flops, reps=20):
    """The ring backward of the same share (usp_attn_bwd: per-row statistics,
    dQ pass, dK/dV pass) after its forward, with a seeded upstream gradient.
    Algorithmic work: five products of the forward's shape (S, dP, dV, dK,
    dQ), 2.5 times the forward's flops; the two passes execute seven."""
    import torch
    from sequence_ring_attention_amd import binding as B
    from sequence_ring_attention_amd import inputs
    u = share.u
    q, k, v, o, lse = share.qh[u], share.kh[u], share.vh[u], share.oh[u], share.lse[u]
    d_o = inputs.randn(tuple(o.shape), 99, "bf16").to(o.device)
    dq = torch.empty_like(q)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=k.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
    stats = torch.empty(2 * lse.numel(), dtype=torch.float32, device=q.device)
    desc = share.desc(u)
    prep_ms = _time(lambda: B.usp_attn_bwd_prep(o, d_o, lse, stats, desc, share.r), reps)
    bwd_ms = _time(lambda: B.usp_attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, stats, desc, share.r), reps)
    flops = 2.5 * fwd_flops
    prep_bytes = 2 * o.numel() * o.element_size() + 3 * lse.numel() * 4
    return {"entry": "usp_attn_bwd", "ms": bwd_ms, "TFLOP/s": flops / (bwd_ms * 1e-3) / 1e12,
            "frac_mfma": flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "work_per_launch_tflop": flops / 1e12, "executed_products": 7, "algorithmic_products": 5,
            "executed_by_pass": {"dQ": "S, dP, dQ", "dK/dV": "S, dP, dV, dK"},
            "prep": {"ms": prep_ms, "bytes": prep_bytes, "GB/s": prep_bytes / (prep_ms * 1e-3) / 1e9}}


def main():
    args = parse()
    _CALLS_PER_REP[0] = max(0, args.calls_per_rep)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share on a single MI355X; --gpus {args.gpus} is not "
              "supported: the library runs one GPU's share and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    import torch
    if args.only_workloads:
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"workloads": extra_workloads(cpu=False)}), flush=True)
        return
    from sequence_ring_attention_amd import inputs
    from sequence_ring_attention_amd.pipeline import OneGpuShare

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = inputs.WORKLOADS[WORKLOAD]
    r, u = args.ring_rank, args.ulysses_rank
    dev = torch.device("cuda:0")
    print(f"[bench] generating {WORKLOAD} inputs", file=sys.stderr, flush=True)
    q, k, v = inputs.workload_qkv(w)
    Q, K, V = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    share = OneGpuShare(Q, K, V, w.rd, w.ud, r, u)
    share.prepare_peers()
    torch.cuda.synchronize()
    print("[bench] peers prepared; warmup", file=sys.stderr, flush=True)

    # algorithmic work per step
    hb = w.H // w.ud
    c = w.chunk
    flops, flops_exact = share_walk_flops(w.D, hb, w.B, w.rd, c)   # half-diagonal convention, exact
    zig_bytes, fwd_bytes, inv_bytes = share.copy_bytes()

    for _ in range(args.warmup):
        share.step()
    torch.cuda.synchronize()

    # timed region: whole steps, with per-phase events on the same stream
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    t_start.record(stream)
    wall0 = time.perf_counter()
    for s in range(args.steps):
        share.step(marks[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    seg = lambda i, j: sum(marks[s][i].elapsed_time(marks[s][j]) for s in range(args.steps)) / args.steps
    zig_ms, fwd_ms, walk_ms, inv_ms = seg(0, 1), seg(1, 2), seg(2, 3), seg(3, 4)

    walk_tflops = flops / (walk_ms * 1e-3) / 1e12
    copy_ref = plain_copy_reference(inv_bytes // 2)
    traffic = measured_traffic()
    result = {
        "metric": "ring-step attention causal TFLOP/s + % bf16 MFMA peak; layout GB/s, 1 GPU",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "seq_len": w.S, "num_q_heads": w.H, "num_kv_heads": w.Hkv,
                   "head_dim": w.D, "batch": w.B, "ring_degree": w.rd, "ulysses_degree": w.ud,
                   "share": {"ring_rank": r, "ulysses_rank": u},
                   "share_tokens": w.S // w.rd, "heads_per_gpu": hb},
        "roofline": {"bound": "mfma", "achieved": walk_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": walk_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": WALK_KERNEL,
                     "work_per_launch_tflop": flops / 1e12,
                     "work_per_launch_tflop_exact_pairs": flops_exact / 1e12,
                     "avg_launch_ms": walk_ms},
        "kernels": {
            "zigzag_extract_qkv": {"ms": zig_ms, "bytes": zig_bytes,
                                   "GB/s": zig_bytes / (zig_ms * 1e-3) / 1e9,
                                   "frac_hbm": zig_bytes / (zig_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "ulysses_layout_fwd_qkv": {"ms": fwd_ms, "bytes": fwd_bytes,
                                       "GB/s": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
                                       "frac_hbm": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "ring_walk_attention": {"ms": walk_ms, "TFLOP/s": walk_tflops,
                                    "frac_mfma": walk_tflops / PEAK_BF16_TFLOPS},
            "ulysses_layout_inv_o": {"ms": inv_ms, "bytes": inv_bytes,
                                     "GB/s": inv_bytes / (inv_ms * 1e-3) / 1e9,
                                     "frac_hbm": inv_bytes / (inv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "plain_device_copy_reference": copy_ref,
        },
        "wall_s_timed": wall,
    }
    sample = None if args.no_cpu_baseline else gpu_sample(share, w, args.cpu_rows)   # outputs of the last step
    walks = sorted(marks[s][2].elapsed_time(marks[s][3]) for s in range(args.steps))
    result["kernels"]["ring_walk_attention"].update(
        {"ms_median": walks[len(walks) // 2], "ms_min": walks[0], "ms_max": walks[-1]})
    print("[bench] clock during the walk", file=sys.stderr, flush=True)
    clk = clock_during(lambda: share._walk(u))
    result["roofline"]["clock"] = clk
    if clk.get("mhz"):
        # the same walk rated against the peak at the clock it ran at (256 CUs x 4096 bf16 FLOP/clk)
        at_clock = 256 * 4096 * clk["mhz"] * 1e6 / 1e12
        result["roofline"]["peak_at_measured_clock"] = at_clock
        result["roofline"]["frac_at_measured_clock"] = walk_tflops / at_clock
    if not args.no_backward:
        print("[bench] backward of the same share", file=sys.stderr, flush=True)
        result["backward"] = backward_walk(share, flops)
    if not args.no_extra:
        print("[bench] ring steps one by one", file=sys.stderr, flush=True)
        result["ring_steps"] = ring_steps(share, flops)
        print("[bench] copy launches, cache flushed", file=sys.stderr, flush=True)
        result["copy_launches"] = copy_launches(share, w)
        r2 = w.rd - 1 if r != w.rd - 1 else 0
        print(f"[bench] walk of share ({r2}, {u})", file=sys.stderr, flush=True)
        result["other_share"] = other_share_walk(Q, K, V, w, r2, u, flops)
        print("[bench] head chunks", file=sys.stderr, flush=True)
        result["head_chunks"] = head_chunk_steps(Q, K, V, w, r, u, flops, ms_step, share.head_major_bytes())
    if not args.no_extra:
        print("[bench] other workloads", file=sys.stderr, flush=True)
        del share, Q, K, V
        torch.cuda.empty_cache()
        result["workloads"] = extra_workloads(cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, r, u, args.cpu_rows, sample)
        result["cpu_baseline"]["index_oracle_copies"] = index_oracle_copies()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
