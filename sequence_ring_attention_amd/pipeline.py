"""One GPU's share of USP-Attention on a virtual (ud x rd) grid.

The share of virtual GPU (ring rank r, Ulysses rank u) is, in the order of
the "USP" paper review's Algorithms 1 and 2 (section 三):

1. zigzag-extract its own Q, K, V shard from the global tensors;
2. Ulysses layout (the all-to-all as a permutation) of Q, K, V to head-major
   (hc/ud, bs, 2c, hd) for its head block u;
3. the ring walk over the cp KV blocks with the fused LSE merge, writing O
   (bf16) and lse;
4. the inverse Ulysses layout of O back to its (bs, 2c/ud, hc, hd) shard.

On a real grid the peers' pieces arrive over the interconnect: the other
Ulysses ranks' shards and outputs (all-to-all) and the other ring ranks' KV
blocks (ring P2P).  Here they are produced once by ``prepare_peers`` with
the same kernels, outside ``step``; ``step`` is exactly the per-GPU work.

With ``head_chunk`` (headwise chunking, [UPipe page] section 2) steps 2-4
run once per chunk of ``head_chunk`` query heads of the head block (and
their KV heads): the head-major tensors then hold one chunk at a time.  With
``overlap_chunks`` as well, consecutive chunks alternate between the current
stream and a second one (default priority), each with its own head-major
query buffer, so one chunk's walk can fill the CUs another leaves idle: two
chunks' query tensors are then held at once.

This module only allocates buffers and sequences C-ABI calls.
"""
import torch

from . import binding as B


class OneGpuShare:
    def __init__(self, Q, K, V, rd, ud, ring_rank, ulysses_rank, causal=True, cu_seqlens=None, per_sample=False,
                 head_chunk=None, overlap_chunks=False, split_walk=False):
        """Q (B, S, H, D), K/V (B, S, Hkv, D): global tensors on the GPU.
        ``cu_seqlens``: packed-sample boundaries; ``per_sample``: the shares
        are the per-sample zigzag split (Algorithm 2 on every sample) instead
        of the split of the whole packed stream.  ``head_chunk``: query heads
        per chunk (dividing H / ud, a multiple or a divisor of H / Hkv), or
        None for the whole head block at once.  ``overlap_chunks``: run
        consecutive chunks on two streams (needs ``head_chunk``).
        ``split_walk``: chunks walk with usp_attn_fwd_split (a chunk's heavy
        query tiles split over two workgroups when the chunk's launch is too
        small to fill the GPU), with one workspace per query buffer."""
        self.Q, self.K, self.V = Q, K, V
        self.rd, self.ud, self.r, self.u = rd, ud, ring_rank, ulysses_rank
        Bn, S, H, D = Q.shape
        Hkv = K.shape[2]
        if H % ud or Hkv % ud or S % (2 * rd * ud):
            raise ValueError("grid does not divide the problem")
        self.Bn, self.S, self.H, self.Hkv, self.D = Bn, S, H, Hkv, D
        self.T, self.L = S // (rd * ud), S // rd
        self.causal, self.per_sample = causal, per_sample
        hb, G = H // ud, H // Hkv
        if head_chunk is not None and head_chunk != hb:
            if head_chunk < 1 or hb % head_chunk or (head_chunk % G and G % head_chunk):
                raise ValueError("head_chunk must divide H / ud and hold whole GQA groups or lie in one")
            self.chunk = int(head_chunk)
        else:
            self.chunk = None
        self.cu = None if cu_seqlens is None else B.host_cu_seqlens(cu_seqlens)
        if per_sample and self.cu is None:
            raise ValueError("the per-sample split needs cu_seqlens")
        dev, dt = Q.device, Q.dtype
        T, L = self.T, self.L
        e = lambda *s: torch.empty(*s, dtype=dt, device=dev)
        # group shards of ring group r (slot u is ours, the others are the peers')
        self.qz, self.kz, self.vz = e(ud, Bn, T, H, D), e(ud, Bn, T, Hkv, D), e(ud, Bn, T, Hkv, D)
        # the ring's KV blocks (block j = ring rank j's share) for every head block
        self.kh = e(ud, rd, Hkv // ud, Bn, L, D)
        self.vh = e(ud, rd, Hkv // ud, Bn, L, D)
        if self.chunk is None:
            # head-major Q and outputs of every Ulysses rank in the group
            self.qh = e(ud, hb, Bn, L, D)
            self.oh = e(ud, hb, Bn, L, D)
        else:
            # one chunk of query heads, head-major (reused by every chunk), and
            # the group's outputs chunk by chunk: [c, u'] = rank u''s heads of chunk c
            # one buffer per stream in use; qc is the first
            self.qcs = [e(self.chunk, Bn, L, D) for _ in range(2 if overlap_chunks else 1)]
            self.qc = self.qcs[0]
            self.ohc = e(hb // self.chunk, ud, self.chunk, Bn, L, D)
        if overlap_chunks and self.chunk is None:
            raise ValueError("overlap_chunks needs head_chunk")
        self.overlap = bool(overlap_chunks)
        self._side = torch.cuda.Stream(device=dev) if self.overlap else None
        self.split_walk = bool(split_walk)
        self._ws = {}
        self.lse = torch.empty(ud, hb, Bn, L, dtype=torch.float32, device=dev)
        self.out = e(Bn, T, H, D)     # this GPU's output shard after the inverse layout
        self._descs = {}

    def desc(self, u):
        if u not in self._descs:
            self._descs[u] = B.attn_desc(self.S, self.rd, self.qh[u], self.kh[u], self.vh[u], o=self.oh[u],
                                         layout="hbsd", causal=self.causal, cu_seqlens=self.cu,
                                         zigzag_per_sample=self.per_sample)
        return self._descs[u]

    # ------------------------------------------------------------ pieces --
    def _extract(self, X, out, r, u):
        if self.per_sample:
            B.usp_zigzag_extract_varlen(X, out, self.rd, self.ud, r, u, self.cu)
        else:
            B.usp_zigzag_extract(X, out, self.rd, self.ud, r, u)

    def _kv_blocks(self, r, u, scratch_k, scratch_v):
        """Ring rank r's K/V head block u, head-major, into the ring slots."""
        self._extract(self.K, scratch_k, r, -1)
        self._extract(self.V, scratch_v, r, -1)
        B.usp_ulysses_a2a_layout(scratch_k, self.kh[u, r], self.ud, u)
        B.usp_ulysses_a2a_layout(scratch_v, self.vh[u, r], self.ud, u)

    def _walk(self, u):
        B.usp_attn_fwd(self.qh[u], self.kh[u], self.vh[u], self.oh[u], self.lse[u], self.desc(u), self.r)

    # ------------------------------------------------------ head chunks --
    def _chunk_heads(self, c):
        """Query heads [h0, h0 + nh) and KV heads [k0, k0 + nk) of chunk c
        (query head h reads KV head h // G; a chunk inside one GQA group
        has that group's KV head)."""
        nh, G = self.chunk, self.H // self.Hkv
        return c * nh, nh, c * nh // G, max(nh // G, 1)

    def _chunk_desc(self):
        if "chunk" not in self._descs:
            _, _, k0, nk = self._chunk_heads(0)
            self._descs["chunk"] = B.attn_desc(self.S, self.rd, self.qc, self.kh[0][:, k0:k0 + nk],
                                               self.vh[0][:, k0:k0 + nk], o=self.ohc[0, 0], layout="hbsd",
                                               causal=self.causal, cu_seqlens=self.cu,
                                               zigzag_per_sample=self.per_sample)
        return self._descs["chunk"]

    def _walk_chunk(self, u, c, qc=None):
        """Ulysses rank u's walk over chunk c's heads, its query heads in qc."""
        h0, nh, k0, nk = self._chunk_heads(c)
        q = self.qc if qc is None else qc
        args = (q, self.kh[u][:, k0:k0 + nk], self.vh[u][:, k0:k0 + nk], self.ohc[c, u], self.lse[u, h0:h0 + nh],
                self._chunk_desc(), self.r)
        if self.split_walk:
            i = 0 if q is self.qcs[0] else 1     # the walks of one query buffer run in order on one stream
            if i not in self._ws:
                n = B.usp_attn_fwd_split_workspace(self._chunk_desc(), self.r)
                self._ws[i] = torch.empty(n, dtype=torch.uint8, device=q.device)
            B.usp_attn_fwd_split(*args, self._ws[i])
        else:
            B.usp_attn_fwd(*args)

    def _chunks(self):
        return range(self.H // self.ud // self.chunk)

    def prepare_peers(self):
        """Everything the peers would send: other ring ranks' KV blocks (all
        head blocks), the group's other shards, and the other Ulysses ranks'
        outputs."""
        sk = torch.empty_like(self.kz)
        sv = torch.empty_like(self.vz)
        for u in range(self.ud):
            for r in range(self.rd):
                self._kv_blocks(r, u, sk, sv)
        self._extract(self.Q, self.qz, self.r, -1)
        self._extract(self.K, self.kz, self.r, -1)
        self._extract(self.V, self.vz, self.r, -1)
        for u in range(self.ud):
            if u == self.u:
                continue
            if self.chunk is None:
                B.usp_ulysses_a2a_layout(self.qz, self.qh[u], self.ud, u)
                self._walk(u)
            else:
                for c in self._chunks():
                    h0, nh, _, _ = self._chunk_heads(c)
                    B.usp_ulysses_a2a_layout_heads(self.qz, self.qc, self.ud, u, h0, nh)
                    self._walk_chunk(u, c)

    def step(self, marks=None):
        """The per-GPU hot path: extract, layout, ring walk, inverse layout.

        ``marks``: optional 5 events recorded on the current stream around
        the four phases (for per-kernel timing).  With head chunks the
        layouts and walks of the chunks interleave: marks 1 and 2 then both
        follow the extract, and marks 3 and 4 both close the step."""
        r, u, rd, ud = self.r, self.u, self.rd, self.ud
        mark = (lambda i: marks[i].record()) if marks is not None else (lambda i: None)
        mark(0)
        if self.per_sample:
            self._extract(self.Q, self.qz[u], r, u)
            self._extract(self.K, self.kz[u], r, u)
            self._extract(self.V, self.vz[u], r, u)
        else:  # Q, K and V in one launch
            B.usp_zigzag_extract_n((self.Q, self.K, self.V), (self.qz[u], self.kz[u], self.vz[u]), rd, ud, r, u)
        mark(1)
        if self.chunk is not None:
            mark(2)
            if self.overlap:
                self._chunks_overlapped(r, u, ud)
            else:
                k_done = -1
                for c in self._chunks():
                    h0, nh, k0, nk = self._chunk_heads(c)
                    B.usp_ulysses_a2a_layout_heads(self.qz, self.qc, ud, u, h0, nh)
                    if k0 != k_done:  # chunks inside one GQA group share its KV head
                        B.usp_ulysses_a2a_layout_heads(self.kz, self.kh[u, r, k0:k0 + nk], ud, u, k0, nk)
                        B.usp_ulysses_a2a_layout_heads(self.vz, self.vh[u, r, k0:k0 + nk], ud, u, k0, nk)
                        k_done = k0
                    self._walk_chunk(u, c)
                    B.usp_ulysses_a2a_layout_heads(self.ohc[c], self.out, ud, u, h0, nh, inverse=True)
            mark(3)
            mark(4)
            return self.out
        B.usp_ulysses_a2a_layout_n((self.qz, self.kz, self.vz), (self.qh[u], self.kh[u, r], self.vh[u, r]), ud, u)
        mark(2)
        self._walk(u)
        mark(3)
        B.usp_ulysses_a2a_layout(self.oh, self.out, ud, u, inverse=True)
        mark(4)
        return self.out

    def _chunks_overlapped(self, r, u, ud):
        """The chunks on two streams: chunk c on stream c % 2 with query
        buffer c % 2.  Work on one stream is ordered, so a buffer is reused
        only after its previous chunk's walk; a GQA group's K/V layout is
        done once, and a chunk on the other stream waits for its event.  The
        side stream starts after the extract and the current stream waits for
        it before the step ends."""
        main = torch.cuda.current_stream()
        streams = (main, self._side)
        self._side.wait_stream(main)
        kv_ready = {}
        for c in self._chunks():
            s = streams[c % 2]
            h0, nh, k0, nk = self._chunk_heads(c)
            with torch.cuda.stream(s):
                qc = self.qcs[c % 2]
                B.usp_ulysses_a2a_layout_heads(self.qz, qc, ud, u, h0, nh)
                if k0 not in kv_ready:
                    B.usp_ulysses_a2a_layout_heads(self.kz, self.kh[u, r, k0:k0 + nk], ud, u, k0, nk)
                    B.usp_ulysses_a2a_layout_heads(self.vz, self.vh[u, r, k0:k0 + nk], ud, u, k0, nk)
                    ev = torch.cuda.Event()
                    ev.record(s)
                    kv_ready[k0] = (ev, c % 2)
                elif kv_ready[k0][1] != c % 2:
                    s.wait_event(kv_ready[k0][0])
                self._walk_chunk(u, c, qc)
                B.usp_ulysses_a2a_layout_heads(self.ohc[c], self.out, ud, u, h0, nh, inverse=True)
        main.wait_stream(self._side)

    # ------------------------------------------------------- accounting --
    def head_major_bytes(self):
        """Bytes of the head-major tensors one chunk's attention works on
        (its query heads, one ring block of their KV heads, its outputs):
        what headwise chunking bounds.  With overlapped chunks two chunks are
        in flight, so twice that."""
        e = self.Q.element_size()
        if self.chunk is None:
            nh, nk = self.H // self.ud, self.Hkv // self.ud
        else:
            _, nh, _, nk = self._chunk_heads(0)
        in_flight = 2 if self.overlap else 1
        return in_flight * (2 * nh + 2 * nk) * self.Bn * self.L * self.D * e

    def copy_bytes(self):
        """Bytes each copy phase of one step reads plus writes (every element
        once): zigzag extract of Q, K, V; forward layout of Q, K, V; inverse
        layout of O.  A shard of Q holds as many elements as one Ulysses head
        block of the 2c-token share."""
        e = self.Q.element_size()
        q = self.T * self.H * self.D * self.Bn * e
        kv = self.T * self.Hkv * self.D * self.Bn * e
        return 2 * (q + 2 * kv), 2 * (q + 2 * kv), 2 * q
