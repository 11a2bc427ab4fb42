/*
 * usp.h -- C ABI of libusp.so: one GPU's share of the USP attention forward
 * pass (Ulysses all-to-all layout + zigzag Ring-Attention) and its backward
 * on AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [USP review]    "USP: 统一序列并行方法用于长上下文生成式AI" (xllm-io paper
 *                   review of Fang & Zhao, USP), section 三: the AllToAll4D
 *                   layout (bs, L/N, hc, hd) -> (hc/N, bs, L, hd), Algorithm 1
 *                   (USP-Attention) and Algorithm 2 (load-balanced split).
 *   [CP vs Ulysses] "Context Parallel 与 Ulysses" (ml-interview blog): the
 *                   ring schedule and the LSE merge (concepts section,
 *                   Figure 1), the causal balance of the 2*cp split (Figure 2).
 *   [YunChang]      the YunChang README translation: the user-facing layout
 *                   [batch, seq_len, num_heads, head_dim] and the attention
 *                   call's options (dropout, window, softcap, ALiBi ...).
 *   [UPipe page]    "Untied Ulysses：基于分头切分的高效上下文并行方案"
 *                   (ai-stack.site summary of UPipe), section 2: headwise
 *                   chunking of the Ulysses head blocks.
 *
 * Conventions shared by every entry point:
 *   - Every buffer is device memory owned by the caller.  The library
 *     allocates nothing, keeps no device state between calls (except the
 *     statistics array of usp_attn_bwd_noalloc, a static device symbol) and
 *     never synchronises: work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and results are valid once that stream has
 *     completed.
 *   - Element strides count elements, not bytes; head_dim is always the
 *     contiguous (stride 1) dimension.
 *   - Validation is synchronous and happens before any launch.  A non-OK
 *     status means nothing was enqueued (except USP_ERR_HIP, which reports a
 *     launch error).  usp_last_error_detail() gives a message for the last
 *     non-OK status of the calling thread.
 *   - Calls are thread-safe; calls that write the same buffers race.
 *   - Positions: S is the global sequence length, rd (= cp) the ring degree,
 *     ud the Ulysses degree, c = S / (2 rd) the zigzag chunk length.  Ring
 *     rank r holds chunks r and 2 rd - 1 - r (in that order), i.e. a "share"
 *     of 2c tokens whose global positions are r*c + i for i < c and
 *     (2 rd - 1 - r)*c + (i - c) for c <= i < 2c.
 */
#ifndef USP_H
#define USP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define USP_ABI_VERSION 7

/* Most packed samples one call takes (their boundaries travel by value). */
#define USP_MAX_SEQS 256

typedef enum {
  USP_OK = 0,
  USP_ERR_INVALID_ARG = 1, /* a null/misaligned pointer, a bad size, rank or step */
  USP_ERR_UNSUPPORTED = 2, /* a valid request this library does not implement */
  USP_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} usp_status;

typedef enum { USP_DTYPE_BF16 = 0, USP_DTYPE_FP32 = 1 } usp_dtype;

/* Element strides of a 4D [batch, seq, head, head_dim] tensor. */
typedef struct {
  int64_t b, s, h;
} usp_strides;

/*
 * Problem description shared by the attention entry points.
 *
 * Q is one ring rank's share (2c rows per batch and head) in `dtype`; K and V
 * are the cp KV blocks as they would arrive over the ring: block j is ring
 * rank j's share and starts `kv_block_stride` elements after block j - 1.
 * With strides, both the sequence-major layout (B, 2c, H, D) and the
 * head-major layout after the Ulysses all-to-all (H, B, 2c, D) are accepted
 * without copies.
 */
typedef struct {
  int64_t batch;          /* B >= 1                                             */
  int64_t seq_len;        /* S, global; must divide by 2 * cp                   */
  int64_t num_q_heads;    /* Hq (the heads this GPU holds)                      */
  int64_t num_kv_heads;   /* Hkv; Hq % Hkv == 0, query head h reads KV head
                             h / (Hq / Hkv) (contiguous groups)                 */
  int64_t head_dim;       /* D: 64 or 128                                       */
  usp_dtype dtype;        /* of Q, K, V and the final O; partials and lse are
                             always fp32                                        */
  float softmax_scale;    /* multiplies Q K^T; usually 1 / sqrt(D)              */
  int32_t causal;         /* 1: key visible iff its global position <= the
                             query's (token itself included); 0: no mask        */
  int32_t cp;             /* ring degree (number of virtual ring ranks) >= 1    */
  usp_strides q, k, v, o; /* element strides; o is used by usp_attn_fwd only    */
  int64_t kv_block_stride;/* elements from KV block j to block j + 1            */
  int64_t q_rank_stride;  /* usp_attn_fwd with ring_rank = -1: elements from
                             rank r's query share to rank r + 1's               */
  int64_t o_rank_stride;  /* same, for the output O                            */
  const int32_t *cu_seqlens; /* HOST memory, read during the call only:
                             num_seqs + 1 strictly increasing global boundaries
                             from 0 to S of packed samples (a key is visible
                             only inside its query's sample; needs causal = 1).
                             NULL = one sequence.                               */
  int32_t num_seqs;       /* 1 .. USP_MAX_SEQS when cu_seqlens is set           */
  int32_t zigzag_per_sample; /* 0: the shares are Algorithm 2's split of the
                             whole packed stream.  1: of every sample on its own
                             (see usp_zigzag_extract_varlen): ring rank r holds
                             chunks r and 2 cp - 1 - r of each sample, in sample
                             order.  Needs cu_seqlens, every sample length a
                             multiple of 2 cp.                                  */
} usp_attn_desc;

/*
 * Zigzag split -- [USP review] section 三, Algorithm 2: cut the sequence into
 * 2 rd chunks, give ring rank r chunks r and 2 rd - 1 - r, and give Ulysses
 * rank u the u-th of ud equal parts of that share.
 *
 * Shapes (dtype elements, all contiguous):
 *   x / out "global":  (B, S, H, D)
 *   shard:             (B, S / (rd ud), H, D)
 * Forward (inverse = 0), x global ->
 *   ring_rank >= 0, ulysses_rank >= 0: out = that rank's shard;
 *   ring_rank >= 0, ulysses_rank = -1: out = (ud, shard) of ring group r;
 *   ring_rank = -1, ulysses_rank = -1: out = (rd, ud, shard) of every rank
 *     (for B = 1 this is the whole sequence in zigzag order).
 * Inverse (inverse = 1) swaps the roles: x holds the shard(s) in the layout
 *   above and out is global; only the positions of the selected rank(s) are
 *   written.
 * Errors: USP_ERR_INVALID_ARG for null or 16-byte-misaligned pointers, x ==
 *   out, sizes < 1, S % (2 rd ud) != 0, ranks out of range or
 *   (ring_rank = -1, ulysses_rank >= 0).
 */
usp_status usp_zigzag_extract(const void *x, void *out, usp_dtype dtype, int64_t batch,
                              int64_t seq_len, int64_t heads, int64_t head_dim, int32_t rd,
                              int32_t ud, int32_t ring_rank, int32_t ulysses_rank,
                              int32_t inverse, void *stream);

/* Most tensors one batched copy call (the _n entry points) moves. */
#define USP_MAX_COPY_BATCH 4

/*
 * Zigzag split of several tensors in one launch -- the same Algorithm 2 map
 * as usp_zigzag_extract, applied to n tensors (Q, K and V of one step) that
 * share dtype, B, S, D and the ranks but may differ in head count: tensor i
 * is x[i] -> out[i] with heads[i] heads, exactly as usp_zigzag_extract would
 * copy it.  x, out and heads are host arrays of n entries, read during the
 * call; the caller owns every buffer.
 * Errors: as usp_zigzag_extract for every tensor, plus USP_ERR_INVALID_ARG
 *   for n outside [1, USP_MAX_COPY_BATCH], a null array, or an output whose
 *   byte extent overlaps any input's or another output's, and
 *   USP_ERR_UNSUPPORTED when the tensors together hold 2^32 or more 8 KiB
 *   copy pieces.
 */
usp_status usp_zigzag_extract_n(int32_t n, const void *const *x, void *const *out, const int64_t *heads,
                                usp_dtype dtype, int64_t batch, int64_t seq_len, int64_t head_dim,
                                int32_t rd, int32_t ud, int32_t ring_rank, int32_t ulysses_rank,
                                int32_t inverse, void *stream);

/*
 * Per-sample zigzag split of packed samples -- [USP review] section 三,
 * Algorithm 2 applied to every sample on its own: sample n (boundaries
 * cu_seqlens[n] .. cu_seqlens[n + 1], length a multiple of 2 rd) is cut into
 * 2 rd chunks, ring rank r takes chunks r and 2 rd - 1 - r of every sample in
 * sample order (a share of S / rd tokens), and Ulysses rank u the u-th of ud
 * equal parts of that share.  Every rank then carries the same causal work
 * ([CP vs Ulysses] Figure 2's pairing, sample by sample).  With one sample it
 * equals usp_zigzag_extract.
 *
 * Shapes, modes and errors as usp_zigzag_extract, plus: cu_seqlens is HOST
 * memory read during the call (num_seqs + 1 boundaries from 0 to seq_len,
 * strictly increasing, 1 <= num_seqs <= USP_MAX_SEQS, every length a
 * multiple of 2 rd), else USP_ERR_INVALID_ARG.
 */
usp_status usp_zigzag_extract_varlen(const void *x, void *out, usp_dtype dtype, int64_t batch,
                                     int64_t seq_len, int64_t heads, int64_t head_dim,
                                     int32_t rd, int32_t ud, int32_t ring_rank,
                                     int32_t ulysses_rank, int32_t inverse,
                                     const int32_t *cu_seqlens, int32_t num_seqs, void *stream);

/*
 * Ulysses AllToAll4D as a single-GPU permutation -- [USP review] section 三:
 * (bs, L/N, hc, hd) -> (hc/N, bs, L, hd) (the page writes "hs" for hc) and
 * Algorithm 1, steps 1-3 (forward) and 5 (inverse).  Rank u takes head block
 * u (hc/N contiguous heads) from every peer u', and peers' sequence pieces
 * are gathered in u' order:
 *     Y_u[h', b, u' (L/N) + t, :] = X_u'[b, t, u (hc/N) + h', :].
 *
 * Forward (inverse = 0): in = the N peers' shards, (N, bs, L/N, hc, hd);
 *   out = (hc/N, bs, L, hd) for ulysses_rank = u >= 0, or
 *   (N, hc/N, bs, L, hd) for every rank when ulysses_rank = -1.
 * Inverse (inverse = 1): in = the N head-major tensors (N, hc/N, bs, L, hd);
 *   out = rank u's (bs, L/N, hc, hd), or (N, bs, L/N, hc, hd) for -1.
 * seq_len is L, the sequence length the Ulysses group holds together.
 * Errors: USP_ERR_INVALID_ARG for null or 16-byte-misaligned pointers,
 *   in == out, sizes < 1, hc % N != 0, L % N != 0, rank out of range.
 */
usp_status usp_ulysses_a2a_layout(const void *in, void *out, usp_dtype dtype, int64_t batch,
                                  int64_t seq_len, int64_t heads, int64_t head_dim,
                                  int32_t ulysses_degree, int32_t ulysses_rank, int32_t inverse,
                                  void *stream);

/*
 * The Ulysses layout of several tensors in one launch -- the same
 * AllToAll4D permutation as usp_ulysses_a2a_layout ([USP review] section
 * 三), applied to n tensors (Q, K and V) that share dtype, bs, L, hd, the
 * degree, the rank and the direction but may differ in head count: tensor i
 * is in[i] -> out[i] with heads[i] heads (hc), exactly as
 * usp_ulysses_a2a_layout would copy it.  in, out and heads are host arrays
 * of n entries, read during the call.
 * Errors: as usp_ulysses_a2a_layout for every tensor, plus
 *   USP_ERR_INVALID_ARG for n outside [1, USP_MAX_COPY_BATCH], a null array,
 *   or an output whose byte extent overlaps any input's or another output's,
 *   and USP_ERR_UNSUPPORTED when the tensors together hold 2^32 or more copy
 *   pieces.
 */
usp_status usp_ulysses_a2a_layout_n(int32_t n, const void *const *in, void *const *out, const int64_t *heads,
                                    usp_dtype dtype, int64_t batch, int64_t seq_len, int64_t head_dim,
                                    int32_t ulysses_degree, int32_t ulysses_rank, int32_t inverse,
                                    void *stream);

/*
 * The Ulysses layout of one chunk of heads -- headwise chunking ([UPipe
 * page] "Untied Ulysses", section 2): the all-to-all moves heads
 * [head_offset, head_offset + num_heads) of every head block at a time, so
 * that the attention's head-major tensors exist for one chunk only.  With
 * head_offset = 0 and num_heads = hc/N it is usp_ulysses_a2a_layout.
 *
 * Forward: in = (N, bs, L/N, hc, hd); out = (num_heads, bs, L, hd) for rank
 *   u, or (N, num_heads, bs, L, hd) for -1:
 *     Y_u[i, b, u' (L/N) + t, :] = X_u'[b, t, u (hc/N) + head_offset + i, :].
 * Inverse: in = the N peers' chunk outputs (N, num_heads, bs, L, hd); out =
 *   rank u's (bs, L/N, hc, hd), or (N, bs, L/N, hc, hd) for -1.  Only heads
 *   u' (hc/N) + head_offset + i of the output are written; the rest of out
 *   is left as it is.
 * Errors: as usp_ulysses_a2a_layout, plus USP_ERR_INVALID_ARG unless
 *   0 <= head_offset and 1 <= num_heads and head_offset + num_heads <= hc/N.
 */
usp_status usp_ulysses_a2a_layout_heads(const void *in, void *out, usp_dtype dtype, int64_t batch,
                                        int64_t seq_len, int64_t heads, int64_t head_dim,
                                        int32_t ulysses_degree, int32_t ulysses_rank, int64_t head_offset,
                                        int64_t num_heads, int32_t inverse, void *stream);

/*
 * One ring step -- [CP vs Ulysses], concepts section and Figure 1: at step t
 * ring rank r holds KV block j = (r - t) mod cp and computes its queries
 * against it.  Output is the step's partial result: o_step = softmax-weighted
 * sum of the visible values of block j, normalised over block j only, and
 * lse_step = natural-log log-sum-exp of the scaled logits over those keys.  A
 * query that sees no key of block j gets o = 0 and lse = -inf.
 *
 *   q:        rank r's share, strides desc->q, 2c rows
 *   k_all, v_all: the cp KV blocks (desc->k, desc->v, desc->kv_block_stride)
 *   o_step:   fp32 (Hq, B, 2c, D), contiguous
 *   lse_step: fp32 (Hq, B, 2c), contiguous
 * Errors: USP_ERR_INVALID_ARG for a bad descriptor (see usp_attn_desc), null
 *   or misaligned pointers, ring_rank or step outside [0, cp);
 *   USP_ERR_UNSUPPORTED for head_dim other than 64/128, cu_seqlens with
 *   causal = 0, or (bf16) a block whose 2c rows of one (batch, head) slice
 *   span 4 GiB or more at the given row stride (the bf16 kernels address a
 *   slice with 32-bit byte offsets; the head-major layout keeps it dense).
 *   The backward entry points apply the same limit to Q's and dO's rows.
 */
usp_status usp_ring_attn_step_fwd(const void *q, const void *k_all, const void *v_all,
                                  float *o_step, float *lse_step, const usp_attn_desc *desc,
                                  int32_t ring_rank, int32_t step, void *stream);
/* (Descriptor errors of every attention entry point also cover cu_seqlens:
 * USP_ERR_INVALID_ARG unless it holds num_seqs + 1 strictly increasing
 * boundaries from 0 to seq_len with 1 <= num_seqs <= USP_MAX_SEQS, and, with
 * zigzag_per_sample, every length a multiple of 2 cp.) */

/*
 * One ring step merged into a running accumulator in the same launch:
 * usp_ring_attn_step_fwd of rank r at step t (block j = (r - t) mod cp)
 * followed by usp_lse_merge, with the merge ([CP vs Ulysses], concepts
 * section) done in the step kernel's epilogue, so the step's partial never
 * reaches HBM.  Results are bitwise those of the two calls on an accumulator
 * whose empty rows hold o = 0.
 *   o_acc (Hq, B, 2c, D), lse_acc (Hq, B, 2c): fp32, contiguous, read and
 *                    written in place.  A row whose lse_acc is -inf takes the
 *                    step's partial as it is and its o_acc is not read, so a
 *                    ring starts from lse_acc = -inf with o_acc left as it is.
 *                    A row with no visible key in the step is left alone.
 * Errors: as usp_ring_attn_step_fwd.
 */
usp_status usp_ring_attn_step_fwd_merge(const void *q, const void *k_all, const void *v_all,
                                        float *o_acc, float *lse_acc, const usp_attn_desc *desc,
                                        int32_t ring_rank, int32_t step, void *stream);

/*
 * LSE merge, in place on the accumulator -- [CP vs Ulysses], concepts
 * section: lse = log(e^lse1 + e^lse2), o = e^(lse1 - lse) o1 + e^(lse2 - lse)
 * o2, evaluated as M + log(e^(lse1-M) + e^(lse2-M)) with M = max(lse1, lse2).
 * A partial with lse = -inf (no visible key) is the identity; two such
 * partials give (0, -inf).
 *   o_acc (rows, head_dim), lse_acc (rows): fp32, updated in place
 *   o_step (rows, head_dim), lse_step (rows): fp32, read only
 * Errors: USP_ERR_INVALID_ARG for null or 16-byte-misaligned pointers, rows <
 *   0, head_dim < 1 or head_dim % 4 != 0.  rows = 0 is a no-op.
 */
usp_status usp_lse_merge(float *o_acc, float *lse_acc, const float *o_step,
                         const float *lse_step, int64_t rows, int64_t head_dim, void *stream);

/*
 * The whole ring for one rank in a single launch -- LoadBalance-RingAttention
 * of [USP review] Algorithm 1 step 4 with the ring of [CP vs Ulysses]: the
 * rank walks KV blocks (r - t) mod cp for t = 0 .. cp-1, which already sit in
 * HBM, and folds each step into a running (max, sum, output) per query row;
 * that running fold is the LSE merge applied step after step.  The epilogue
 * writes the final O in `dtype` (bf16: round to nearest even) with strides
 * desc->o, and lse (fp32, natural log) as (Hq, B, 2c).
 *
 * ring_rank = -1 runs every rank in one launch: rank r's query share starts
 * r * desc->q_rank_stride elements after q, its output r * desc->o_rank_stride
 * after o, and lse becomes (cp, Hq, B, 2c).
 * Errors: as usp_ring_attn_step_fwd, and ring_rank outside [-1, cp).
 */
usp_status usp_attn_fwd(const void *q, const void *k_all, const void *v_all, void *o,
                        float *lse, const usp_attn_desc *desc, int32_t ring_rank, void *stream);

/*
 * usp_attn_fwd for launches too small to fill the GPU once (at most one
 * 256-row query tile per CU: a few query heads of a share, e.g. headwise
 * chunks): a causal query tile whose work is
 * above the launch's mean has its ring steps walked by two workgroups, steps
 * [0, t_mid) and [t_mid, cp), each into an fp32 partial (o, lse) in
 * `workspace`; a finalize kernel merges the two partials by the LSE rule of
 * [CP vs Ulysses], concepts section (the same rule usp_lse_merge applies),
 * rounds o once to `dtype` and writes o and lse exactly where usp_attn_fwd
 * does.  Results equal usp_attn_fwd's to rounding (the merge replaces part of
 * the in-kernel running fold).  Larger launches, packed samples, fp32,
 * cp = 1 and cp > 15 run usp_attn_fwd's walk and leave the workspace
 * untouched.
 *   workspace:       device memory owned by the caller, 256-byte aligned, at
 *                    least usp_attn_fwd_split_workspace(desc, ring_rank)
 *                    bytes; overwritten.  Calls that may overlap on the GPU
 *                    need separate workspaces.
 * Errors: as usp_attn_fwd, plus USP_ERR_INVALID_ARG for a null, misaligned
 *   or too small workspace.
 */
usp_status usp_attn_fwd_split(const void *q, const void *k_all, const void *v_all, void *o,
                              float *lse, const usp_attn_desc *desc, int32_t ring_rank,
                              void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of workspace usp_attn_fwd_split needs for this descriptor and
 * ring_rank: two fp32 partials (head_dim + 1 floats) of every query row the
 * call covers.  Host-only; -1 for a null descriptor or ring_rank out of
 * range. */
int64_t usp_attn_fwd_split_workspace(const usp_attn_desc *desc, int32_t ring_rank);

/*
 * ---------------------------------------------------------------- backward
 * Gradients of the attention above for training (the pages train with the
 * method: [YunChang] runs its tests with a backward flag, [USP review]
 * section 六 trains end to end).  They are the derivative of the forward:
 * with P the softmax probabilities over all cp blocks and dO the gradient of
 * the output,
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  dQ = scale dS K,
 *   dK = scale dS^T Q,  delta = rowsum(dO * O) per query row,
 * and a KV head's dK, dV sum the contributions of its query heads.  On the
 * ring ([CP vs Ulysses], concepts section), P restricted to block j is
 * exp(scale q k^T - lse) with the forward's final lse, so every step's
 * contribution stands alone: a rank's dQ sums its cp steps, and block j's
 * dK, dV sum the steps of every rank against block j.  In a real ring the dK,
 * dV accumulators travel with their KV block; here the blocks sit in HBM and
 * the accumulators are the caller's fp32 buffers.
 *
 * Buffers shared by the backward entry points (device, caller-owned):
 *   d_o:   the output gradient, `dtype`, with O's strides (desc->o) and, for
 *          ring_rank = -1, desc->o_rank_stride between ranks.
 *   stats: fp32 per-row statistics written by usp_attn_bwd_prep and read by
 *          the gradient passes: stats[i] = delta of row i and stats[R + i] =
 *          lse of row i times log2(e) (+inf where lse = -inf), with rows i
 *          ordered (Hq, B, 2c), or (cp, Hq, B, 2c) for ring_rank = -1, and R
 *          the number of rows.  2 R floats.
 *   dk_all, dv_all: fp32 accumulators with K's and V's element strides
 *          (desc->k, desc->v, desc->kv_block_stride): a zeroed buffer shaped
 *          like k_all, in fp32, fits.  The gradient passes add into them.
 * Errors (all backward entry points): as usp_ring_attn_step_fwd, plus
 *   USP_ERR_INVALID_ARG for O or dO strides that do not keep 16-byte
 *   alignment or more than 2^29 statistics rows.
 */

/*
 * Per-row statistics of the backward: delta = rowsum(dO * O) (computed in
 * fp32 from `dtype` O and dO) and lse * log2(e), into `stats` (layout above).
 *   o, d_o: desc->o strides (rank stride desc->o_rank_stride for -1)
 *   lse:    the forward's fp32 lse, (Hq, B, 2c) or (cp, Hq, B, 2c)
 */
usp_status usp_attn_bwd_prep(const void *o, const void *d_o, const float *lse, float *stats,
                             const usp_attn_desc *desc, int32_t ring_rank, void *stream);

/*
 * One ring step of the backward: ring rank r at step t against KV block
 * j = (r - t) mod cp ([CP vs Ulysses], concepts section and Figure 1).
 * Adds the step's contributions:
 *   dq_acc (fp32 (Hq, B, 2c, D), contiguous) += scale dS K_j,
 *   block j of dk_all += scale dS^T Q,  block j of dv_all += P^T dO,
 * where P = exp(scale q k^T - lse) on block j's visible keys.
 * `stats` comes from usp_attn_bwd_prep with the same ring_rank.
 * Errors: as usp_ring_attn_step_fwd.
 */
usp_status usp_ring_attn_step_bwd(const void *q, const void *k_all, const void *v_all,
                                  const void *d_o, const float *stats, float *dq_acc,
                                  float *dk_all, float *dv_all, const usp_attn_desc *desc,
                                  int32_t ring_rank, int32_t step, void *stream);

/*
 * The whole ring backward for one rank (or every rank, ring_rank = -1):
 * usp_attn_bwd_prep into `stats`, then dQ of the rank's queries over all cp
 * steps, written in `dtype` with Q's strides (desc->q, desc->q_rank_stride),
 * and the rank's contributions to every block's dK and dV, added into
 * dk_all, dv_all.  With ring_rank = -1 the blocks receive the sum over all
 * ranks, which is the full gradient of K and V.
 * Errors: as usp_attn_fwd.
 */
usp_status usp_attn_bwd(const void *q, const void *k_all, const void *v_all, const void *o,
                        const void *d_o, const float *lse, void *dq, float *dk_all,
                        float *dv_all, float *stats, const usp_attn_desc *desc,
                        int32_t ring_rank, void *stream);

/*
 * The ring backward without a caller-provided statistics buffer -- for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight training or serving loops, harnesses that forbid hipMalloc).  It is
 * usp_attn_bwd with the same arguments except `stats`: the per-row
 * statistics (delta and lse * log2(e), 2 floats per row) live in a
 * library-owned device array of USP_NOALLOC_MAX_STATS_ROWS rows (16 MiB)
 * that each GPU the library runs on holds until the process ends.  The call
 * allocates nothing.  The array is resolved once per device, on the first
 * call with that device current.  Every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (other streams, other threads) race
 * on it and must be ordered by the caller.  Every row the passes read is
 * written by the call first, so nothing carries over between calls.
 * Outputs are bitwise those of usp_attn_bwd.
 * Errors: as usp_attn_bwd, plus USP_ERR_INVALID_ARG when the call needs more
 *   than USP_NOALLOC_MAX_STATS_ROWS statistics rows ((cp for ring_rank = -1,
 *   else 1) * num_q_heads * batch * seq_len / cp); this is checked before
 *   anything touches the GPU.  USP_ERR_HIP if the array's device address
 *   cannot be obtained.
 */
#define USP_NOALLOC_MAX_STATS_ROWS (1 << 21)

usp_status usp_attn_bwd_noalloc(const void *q, const void *k_all, const void *v_all, const void *o,
                                const void *d_o, const float *lse, void *dq, float *dk_all, float *dv_all,
                                const usp_attn_desc *desc, int32_t ring_rank, void *stream);

/* Name of a status code (static storage). */
const char *usp_status_string(usp_status status);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *usp_last_error_detail(void);

/* USP_ABI_VERSION of the loaded library. */
int32_t usp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* USP_H */
