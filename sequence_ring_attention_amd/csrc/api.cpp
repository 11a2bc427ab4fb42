// C ABI of libusp.so (declared in include/usp.h): argument validation, grid
// planning and dispatch to the HIP kernels.  Every check runs on the host
// before anything is enqueued; no entry point allocates or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/usp.h"
#include "usp_internal.h"

namespace {

thread_local char g_detail[512] = "";

usp_status fail(usp_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}

usp_status ok() {
  g_detail[0] = '\0';
  return USP_OK;
}

usp_status hip_result(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(USP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elem_bytes(usp_dtype dt) { return dt == USP_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(usp_dtype dt) { return dt == USP_DTYPE_BF16 || dt == USP_DTYPE_FP32; }

uint32_t log2_exact(uint64_t v) {
  if (v == 0 || (v & (v - 1))) return 31;
  uint32_t s = 0;
  while ((1ull << s) < v) ++s;
  return s;
}

// Fill the piece fields of a copy plan: pieces of about 8 KiB.  Small pieces
// keep many workgroups' loads in flight: at the 128K-token share, against
// 64 KiB pieces, the inverse layout went from 4.0 to 5.5 TB/s, the batched
// extract from 5.1 to 5.8 and the forward layout from 5.0 to 5.3 (4 KiB
// pieces lost on the forward layout).
void plan_pieces(usp::CopyPlan &p) {
  uint64_t rows = 8192 / p.row_bytes;
  if (rows < 1) rows = 1;
  if (rows > p.rows_per_item) rows = p.rows_per_item;
  p.rows_per_piece = (uint32_t)rows;
  p.pieces_per_item = (uint32_t)((p.rows_per_item + rows - 1) / rows);
  p.row_vecs = (uint32_t)(p.row_bytes / 16);
  p.row_vecs_shift = log2_exact(p.row_vecs);
  if (p.src_row_bytes == 0) {  // rows of equal size on both sides
    p.src_row_bytes = p.row_bytes;
    p.grp_shift = 31;
  }
  if (p.dst_unit_bytes == 0) p.dst_unit_bytes = p.row_bytes;
}

constexpr int64_t kMaxIndex = (int64_t)1 << 31;
static_assert(usp::kMaxCopyBatch == USP_MAX_COPY_BATCH, "batched copy limit");

// Packed-sample boundaries from host memory into the kernels' by-value copy.
// `split` > 0: the per-sample zigzag over `split` ring ranks, which needs
// every length to divide by 2 split.
usp_status read_samples(const int32_t *cu, int32_t nseq, int64_t seq_len, int32_t split, usp::Samples &out,
                        const char *who) {
  out = usp::Samples{};
  if (!cu) {
    if (split > 0) return fail(USP_ERR_INVALID_ARG, "%s: the per-sample split needs cu_seqlens", who);
    return USP_OK;
  }
  if (nseq < 1 || nseq > USP_MAX_SEQS)
    return fail(USP_ERR_INVALID_ARG, "%s: num_seqs %d outside 1..%d", who, (int)nseq, (int)USP_MAX_SEQS);
  if (cu[0] != 0 || (int64_t)cu[nseq] != seq_len)
    return fail(USP_ERR_INVALID_ARG, "%s: cu_seqlens must run from 0 to seq_len", who);
  for (int32_t n = 0; n < nseq; ++n) {
    if (cu[n + 1] <= cu[n]) return fail(USP_ERR_INVALID_ARG, "%s: cu_seqlens must increase strictly", who);
    if (split > 0 && (cu[n + 1] - cu[n]) % (2 * split) != 0)
      return fail(USP_ERR_INVALID_ARG, "%s: sample %d of length %d does not divide into 2*%d chunks", who, (int)n,
                  (int)(cu[n + 1] - cu[n]), (int)split);
  }
  out.nseq = nseq;
  out.per_sample = split > 0;
  for (int32_t n = 0; n <= nseq; ++n) out.cu[n] = cu[n];
  return USP_OK;
}

}  // namespace

extern "C" {

const char *usp_status_string(usp_status s) {
  switch (s) {
    case USP_OK: return "USP_OK";
    case USP_ERR_INVALID_ARG: return "USP_ERR_INVALID_ARG";
    case USP_ERR_UNSUPPORTED: return "USP_ERR_UNSUPPORTED";
    case USP_ERR_HIP: return "USP_ERR_HIP";
  }
  return "USP_ERR_UNKNOWN";
}

const char *usp_last_error_detail(void) { return g_detail; }

int32_t usp_abi_version(void) { return USP_ABI_VERSION; }

namespace {

// Validate one zigzag extract and fill its copy plan; `in_bytes` and
// `out_bytes` are the byte extents the copy reads and writes.
usp_status zigzag_plan(const char *who, const void *x, void *out, usp_dtype dtype, int64_t batch, int64_t seq_len,
                       int64_t heads, int64_t head_dim, int32_t rd, int32_t ud, int32_t ring_rank,
                       int32_t ulysses_rank, int32_t inverse, usp::CopyPlan &p, int64_t &in_bytes,
                       int64_t &out_bytes) {
  if (!x || !out) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(x) || !aligned16(out))
    return fail(USP_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  if (x == out) return fail(USP_ERR_INVALID_ARG, "%s: x and out must differ", who);
  if (!dtype_ok(dtype)) return fail(USP_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dtype);
  if (batch < 1 || seq_len < 1 || heads < 1 || head_dim < 1 || rd < 1 || ud < 1)
    return fail(USP_ERR_INVALID_ARG, "%s: sizes and degrees must be >= 1", who);
  if (inverse != 0 && inverse != 1) return fail(USP_ERR_INVALID_ARG, "%s: inverse must be 0 or 1", who);
  if (seq_len % (2 * (int64_t)rd * ud) != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: seq_len %lld not divisible by 2*rd*ud = %lld", who,
                (long long)seq_len, (long long)(2 * (int64_t)rd * ud));
  if (ring_rank < -1 || ring_rank >= rd || ulysses_rank < -1 || ulysses_rank >= ud)
    return fail(USP_ERR_INVALID_ARG, "%s: rank out of range", who);
  if (ring_rank == -1 && ulysses_rank != -1)
    return fail(USP_ERR_INVALID_ARG, "%s: ring_rank = -1 needs ulysses_rank = -1", who);
  const int64_t row_bytes = heads * head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0)
    return fail(USP_ERR_UNSUPPORTED, "%s: heads*head_dim*element size must be a multiple of 16 bytes", who);
  if (batch * seq_len >= kMaxIndex) return fail(USP_ERR_UNSUPPORTED, "%s: too many rows", who);

  p = usp::CopyPlan{};
  p.src = static_cast<const char *>(x);
  p.dst = static_cast<char *>(out);
  p.kind = inverse ? usp::kZigzagInv : usp::kZigzagFwd;
  const int64_t groups = ring_rank < 0 ? (int64_t)rd * ud : (ulysses_rank < 0 ? ud : 1);
  p.n_items = (uint32_t)(groups * batch);
  p.rows_per_item = (uint32_t)(seq_len / ((int64_t)rd * ud));
  p.row_bytes = (uint64_t)row_bytes;
  p.p[0] = batch;
  p.p[1] = seq_len;
  p.p[2] = seq_len / (2 * (int64_t)rd);
  p.p[3] = rd;
  p.p[4] = ud;
  p.p[5] = p.rows_per_item;
  p.p[6] = ring_rank;
  p.p[7] = ulysses_rank;
  plan_pieces(p);
  const int64_t global = batch * seq_len * row_bytes, shards = (int64_t)p.n_items * p.rows_per_item * row_bytes;
  in_bytes = inverse ? shards : global;
  out_bytes = inverse ? global : shards;
  return USP_OK;
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// A batch of n copies must not write where any of them reads or another
// writes, and its pieces are counted in 32 bits on the device.
usp_status batch_disjoint(const char *who, int32_t n, const usp::CopyPlan *p, const int64_t *in_bytes,
                          const int64_t *out_bytes) {
  uint64_t pieces = 0;
  for (int32_t i = 0; i < n; ++i) pieces += (uint64_t)p[i].n_items * p[i].pieces_per_item;
  if (pieces > 0xffffffffull) return fail(USP_ERR_UNSUPPORTED, "%s: too many pieces for one launch", who);
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < n; ++j) {
      if (overlap(p[i].dst, out_bytes[i], p[j].src, in_bytes[j]))
        return fail(USP_ERR_INVALID_ARG, "%s: output %d overlaps input %d", who, (int)i, (int)j);
      if (i != j && overlap(p[i].dst, out_bytes[i], p[j].dst, out_bytes[j]))
        return fail(USP_ERR_INVALID_ARG, "%s: outputs %d and %d overlap", who, (int)i, (int)j);
    }
  return USP_OK;
}

}  // namespace

usp_status usp_zigzag_extract(const void *x, void *out, usp_dtype dtype, int64_t batch,
                              int64_t seq_len, int64_t heads, int64_t head_dim, int32_t rd,
                              int32_t ud, int32_t ring_rank, int32_t ulysses_rank,
                              int32_t inverse, void *stream) {
  usp::CopyPlan p;
  int64_t nin, nout;
  const usp_status st = zigzag_plan("zigzag_extract", x, out, dtype, batch, seq_len, heads, head_dim, rd, ud,
                                    ring_rank, ulysses_rank, inverse, p, nin, nout);
  if (st != USP_OK) return st;
  return hip_result(usp::launch_copy(p, static_cast<hipStream_t>(stream)), "zigzag_extract launch");
}

usp_status usp_zigzag_extract_n(int32_t n, const void *const *x, void *const *out, const int64_t *heads,
                                usp_dtype dtype, int64_t batch, int64_t seq_len, int64_t head_dim, int32_t rd,
                                int32_t ud, int32_t ring_rank, int32_t ulysses_rank, int32_t inverse,
                                void *stream) {
  if (n < 1 || n > usp::kMaxCopyBatch)
    return fail(USP_ERR_INVALID_ARG, "zigzag_extract_n: n = %d outside [1, %d]", (int)n, usp::kMaxCopyBatch);
  if (!x || !out || !heads) return fail(USP_ERR_INVALID_ARG, "zigzag_extract_n: null array");
  usp::CopyPlan p[usp::kMaxCopyBatch];
  int64_t nin[usp::kMaxCopyBatch], nout[usp::kMaxCopyBatch];
  for (int32_t i = 0; i < n; ++i) {
    const usp_status st = zigzag_plan("zigzag_extract_n", x[i], out[i], dtype, batch, seq_len, heads[i], head_dim,
                                      rd, ud, ring_rank, ulysses_rank, inverse, p[i], nin[i], nout[i]);
    if (st != USP_OK) return st;
  }
  const usp_status st = batch_disjoint("zigzag_extract_n", n, p, nin, nout);
  if (st != USP_OK) return st;
  return hip_result(usp::launch_copy_n(p, n, static_cast<hipStream_t>(stream)), "zigzag_extract_n launch");
}

usp_status usp_zigzag_extract_varlen(const void *x, void *out, usp_dtype dtype, int64_t batch,
                                     int64_t seq_len, int64_t heads, int64_t head_dim,
                                     int32_t rd, int32_t ud, int32_t ring_rank,
                                     int32_t ulysses_rank, int32_t inverse,
                                     const int32_t *cu_seqlens, int32_t num_seqs, void *stream) {
  const char *who = "zigzag_extract_varlen";
  if (!x || !out) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(x) || !aligned16(out)) return fail(USP_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  if (x == out) return fail(USP_ERR_INVALID_ARG, "%s: x and out must differ", who);
  if (!dtype_ok(dtype)) return fail(USP_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dtype);
  if (batch < 1 || seq_len < 1 || heads < 1 || head_dim < 1 || rd < 1 || ud < 1)
    return fail(USP_ERR_INVALID_ARG, "%s: sizes and degrees must be >= 1", who);
  if (inverse != 0 && inverse != 1) return fail(USP_ERR_INVALID_ARG, "%s: inverse must be 0 or 1", who);
  if (seq_len % (2 * (int64_t)rd * ud) != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: seq_len %lld not divisible by 2*rd*ud", who, (long long)seq_len);
  if (ring_rank < -1 || ring_rank >= rd || ulysses_rank < -1 || ulysses_rank >= ud)
    return fail(USP_ERR_INVALID_ARG, "%s: rank out of range", who);
  if (ring_rank == -1 && ulysses_rank != -1)
    return fail(USP_ERR_INVALID_ARG, "%s: ring_rank = -1 needs ulysses_rank = -1", who);
  const int64_t row_bytes = heads * head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0)
    return fail(USP_ERR_UNSUPPORTED, "%s: heads*head_dim*element size must be a multiple of 16 bytes", who);
  if (batch * seq_len >= kMaxIndex) return fail(USP_ERR_UNSUPPORTED, "%s: too many rows", who);
  if (!cu_seqlens) return fail(USP_ERR_INVALID_ARG, "%s: null cu_seqlens", who);
  usp::ZigzagVarlenArgs a{};
  usp_status s = read_samples(cu_seqlens, num_seqs, seq_len, rd, a.sm, who);
  if (s != USP_OK) return s;
  a.src = static_cast<const char *>(x);
  a.dst = static_cast<char *>(out);
  a.row_bytes = row_bytes;
  a.B = (int32_t)batch;
  a.S = (int32_t)seq_len;
  a.rd = rd;
  a.ud = ud;
  a.T = (int32_t)(seq_len / ((int64_t)rd * ud));
  a.ring_rank = ring_rank;
  a.ulysses_rank = ulysses_rank;
  a.inverse = inverse;
  return hip_result(usp::launch_zigzag_varlen(a, static_cast<hipStream_t>(stream)), "zigzag_extract_varlen launch");
}

namespace {

// The Ulysses layout of heads [h0, h0 + nh) of every head block (the whole
// block when h0 = 0, nh = heads / degree).
usp_status ulysses_plan(const char *who, const void *in, void *out, usp_dtype dtype, int64_t batch,
                        int64_t seq_len, int64_t heads, int64_t head_dim, int32_t ulysses_degree,
                        int32_t ulysses_rank, int64_t h0, int64_t nh, int32_t inverse, usp::CopyPlan &p,
                        int64_t &in_bytes, int64_t &out_bytes) {
  if (!in || !out) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(in) || !aligned16(out))
    return fail(USP_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  if (in == out) return fail(USP_ERR_INVALID_ARG, "%s: in and out must differ", who);
  if (!dtype_ok(dtype)) return fail(USP_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dtype);
  if (batch < 1 || seq_len < 1 || heads < 1 || head_dim < 1 || ulysses_degree < 1)
    return fail(USP_ERR_INVALID_ARG, "%s: sizes and degree must be >= 1", who);
  if (inverse != 0 && inverse != 1) return fail(USP_ERR_INVALID_ARG, "%s: inverse must be 0 or 1", who);
  const int64_t N = ulysses_degree;
  if (heads % N != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: heads %lld not divisible by degree %lld", who, (long long)heads,
                (long long)N);
  if (seq_len % N != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: seq_len %lld not divisible by degree %lld", who, (long long)seq_len,
                (long long)N);
  if (ulysses_rank < -1 || ulysses_rank >= ulysses_degree)
    return fail(USP_ERR_INVALID_ARG, "%s: rank out of range", who);
  const int64_t hb = heads / N, Ls = seq_len / N;
  if (h0 < 0 || nh < 1 || h0 + nh > hb)
    return fail(USP_ERR_INVALID_ARG, "%s: head range [%lld, %lld) outside the head block of %lld", who,
                (long long)h0, (long long)(h0 + nh), (long long)hb);
  const int64_t row_bytes = head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0)
    return fail(USP_ERR_UNSUPPORTED, "%s: head_dim*element size must be a multiple of 16 bytes", who);
  if (N * batch * seq_len * heads >= kMaxIndex) return fail(USP_ERR_UNSUPPORTED, "%s: too many rows", who);

  const int64_t G = ulysses_rank < 0 ? N : 1;
  p = usp::CopyPlan{};
  p.src = static_cast<const char *>(in);
  p.dst = static_cast<char *>(out);
  p.kind = inverse ? usp::kUlyssesInv : usp::kUlyssesFwd;
  p.n_items = (uint32_t)(G * nh * batch * N);
  p.rows_per_item = (uint32_t)Ls;
  p.row_bytes = (uint64_t)row_bytes;
  int64_t peers_per_item = 1;
  const uint32_t head_shift = log2_exact((uint64_t)row_bytes / 16);
  if (!inverse && head_shift < 31) {
    // source-major forward: a row is one token's heads of the chunk,
    // contiguous in the source, scattered to the chunk's head planes
    p.kind = usp::kUlyssesFwdRows;
    p.n_items = (uint32_t)(G * batch * N);
    p.row_bytes = (uint64_t)(nh * row_bytes);
    p.dst_unit_bytes = (uint64_t)row_bytes;
    p.src_row_bytes = (uint64_t)row_bytes;
    p.grp_shift = head_shift;
  }
  if (inverse && head_shift < 31) {
    // output-major inverse: a row is one token's heads of the chunk (all of
    // its heads when the chunk is the whole block), contiguous in the
    // output and gathered from the head planes
    const bool whole = nh == hb;
    peers_per_item = whole ? 1 : N;
    p.kind = usp::kUlyssesInvRows;
    p.n_items = (uint32_t)(G * batch * peers_per_item);
    p.row_bytes = (uint64_t)((whole ? heads : nh) * row_bytes);
    p.dst_unit_bytes = (uint64_t)row_bytes;
    p.src_row_bytes = (uint64_t)row_bytes;
    p.grp_shift = head_shift;
  }
  p.p[0] = batch;
  p.p[1] = seq_len;
  p.p[2] = heads;
  p.p[3] = N;
  p.p[4] = hb;
  p.p[5] = Ls;
  p.p[6] = ulysses_rank;
  p.p[7] = h0;
  p.p[8] = nh;
  p.p[9] = peers_per_item;
  plan_pieces(p);
  // extents: one rank's sequence-major shard holds every head, its
  // head-major tensor the chunk's; N of them are read, G written
  const int64_t eb = elem_bytes(dtype);
  const int64_t shard = batch * Ls * heads * head_dim * eb;
  const int64_t planes = nh * batch * seq_len * head_dim * eb;
  in_bytes = N * (inverse ? planes : shard);
  out_bytes = G * (inverse ? shard : planes);
  return USP_OK;
}

usp_status ulysses_layout(const char *who, const void *in, void *out, usp_dtype dtype, int64_t batch,
                          int64_t seq_len, int64_t heads, int64_t head_dim, int32_t ulysses_degree,
                          int32_t ulysses_rank, int64_t h0, int64_t nh, int32_t inverse, void *stream) {
  usp::CopyPlan p;
  int64_t nin, nout;
  const usp_status st = ulysses_plan(who, in, out, dtype, batch, seq_len, heads, head_dim, ulysses_degree,
                                     ulysses_rank, h0, nh, inverse, p, nin, nout);
  if (st != USP_OK) return st;
  return hip_result(usp::launch_copy(p, static_cast<hipStream_t>(stream)), "ulysses layout launch");
}

}  // namespace

usp_status usp_ulysses_a2a_layout(const void *in, void *out, usp_dtype dtype, int64_t batch,
                                  int64_t seq_len, int64_t heads, int64_t head_dim,
                                  int32_t ulysses_degree, int32_t ulysses_rank, int32_t inverse,
                                  void *stream) {
  const int64_t hb = ulysses_degree >= 1 && heads >= 1 ? heads / ulysses_degree : 1;
  return ulysses_layout("ulysses_a2a_layout", in, out, dtype, batch, seq_len, heads, head_dim, ulysses_degree,
                        ulysses_rank, 0, hb < 1 ? 1 : hb, inverse, stream);
}

usp_status usp_ulysses_a2a_layout_n(int32_t n, const void *const *in, void *const *out, const int64_t *heads,
                                    usp_dtype dtype, int64_t batch, int64_t seq_len, int64_t head_dim,
                                    int32_t ulysses_degree, int32_t ulysses_rank, int32_t inverse, void *stream) {
  if (n < 1 || n > usp::kMaxCopyBatch)
    return fail(USP_ERR_INVALID_ARG, "ulysses_a2a_layout_n: n = %d outside [1, %d]", (int)n, usp::kMaxCopyBatch);
  if (!in || !out || !heads) return fail(USP_ERR_INVALID_ARG, "ulysses_a2a_layout_n: null array");
  usp::CopyPlan p[usp::kMaxCopyBatch];
  int64_t nin[usp::kMaxCopyBatch], nout[usp::kMaxCopyBatch];
  for (int32_t i = 0; i < n; ++i) {
    const int64_t hb = ulysses_degree >= 1 && heads[i] >= 1 ? heads[i] / ulysses_degree : 1;
    const usp_status st = ulysses_plan("ulysses_a2a_layout_n", in[i], out[i], dtype, batch, seq_len, heads[i],
                                       head_dim, ulysses_degree, ulysses_rank, 0, hb < 1 ? 1 : hb, inverse, p[i],
                                       nin[i], nout[i]);
    if (st != USP_OK) return st;
  }
  const usp_status st = batch_disjoint("ulysses_a2a_layout_n", n, p, nin, nout);
  if (st != USP_OK) return st;
  return hip_result(usp::launch_copy_n(p, n, static_cast<hipStream_t>(stream)), "ulysses_a2a_layout_n launch");
}

usp_status usp_ulysses_a2a_layout_heads(const void *in, void *out, usp_dtype dtype, int64_t batch,
                                        int64_t seq_len, int64_t heads, int64_t head_dim,
                                        int32_t ulysses_degree, int32_t ulysses_rank, int64_t head_offset,
                                        int64_t num_heads, int32_t inverse, void *stream) {
  return ulysses_layout("ulysses_a2a_layout_heads", in, out, dtype, batch, seq_len, heads, head_dim, ulysses_degree,
                        ulysses_rank, head_offset, num_heads, inverse, stream);
}

usp_status usp_lse_merge(float *o_acc, float *lse_acc, const float *o_step, const float *lse_step,
                         int64_t rows, int64_t head_dim, void *stream) {
  if (rows < 0) return fail(USP_ERR_INVALID_ARG, "lse_merge: rows < 0");
  if (head_dim < 1 || head_dim % 4 != 0)
    return fail(USP_ERR_INVALID_ARG, "lse_merge: head_dim must be a positive multiple of 4");
  if (rows == 0) return ok();
  if (!o_acc || !lse_acc || !o_step || !lse_step) return fail(USP_ERR_INVALID_ARG, "lse_merge: null pointer");
  if (!aligned16(o_acc) || !aligned16(o_step))
    return fail(USP_ERR_INVALID_ARG, "lse_merge: o buffers must be 16-byte aligned");
  return hip_result(usp::launch_lse_merge(o_acc, lse_acc, o_step, lse_step, rows, head_dim,
                                          static_cast<hipStream_t>(stream)),
                    "lse_merge launch");
}

}  // extern "C"

namespace {

// Shared checks of the attention descriptor; fills the kernel arguments.
// The bf16 kernels stage one (batch, head) slice of a share through a buffer
// descriptor and 32-bit byte offsets, which must cover its L rows.
bool rows_span_32bit(int64_t L, int64_t row_stride, int64_t e, int64_t head_dim) {
  return (L - 1) * row_stride * e + head_dim * e <= (int64_t)0xffffffff;
}

usp_status attn_prepare(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const usp_attn_desc *d, int32_t ring_rank, bool all_ranks_ok,
                        usp::AttnArgs &a, const char *who) {
  if (!d) return fail(USP_ERR_INVALID_ARG, "%s: null descriptor", who);
  if (!q || !k || !v || !o || !lse) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(USP_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", who);
  if (!dtype_ok(d->dtype)) return fail(USP_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)d->dtype);
  if (d->batch < 1 || d->seq_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->cp < 1)
    return fail(USP_ERR_INVALID_ARG, "%s: sizes and cp must be >= 1", who);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: num_q_heads must be a multiple of num_kv_heads", who);
  if (d->seq_len % (2 * (int64_t)d->cp) != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: seq_len %lld not divisible by 2*cp = %lld", who,
                (long long)d->seq_len, (long long)(2 * (int64_t)d->cp));
  if (!(d->softmax_scale > 0.0f) || !std::isfinite(d->softmax_scale))
    return fail(USP_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", who);
  if (d->causal != 0 && d->causal != 1) return fail(USP_ERR_INVALID_ARG, "%s: causal must be 0 or 1", who);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(USP_ERR_UNSUPPORTED, "%s: head_dim %lld (supported: 64, 128)", who, (long long)d->head_dim);
  if (d->cu_seqlens && !d->causal)
    return fail(USP_ERR_UNSUPPORTED, "%s: packed samples (cu_seqlens) need causal = 1", who);
  if (d->zigzag_per_sample != 0 && d->zigzag_per_sample != 1)
    return fail(USP_ERR_INVALID_ARG, "%s: zigzag_per_sample must be 0 or 1", who);
  if (ring_rank < (all_ranks_ok ? -1 : 0) || ring_rank >= d->cp)
    return fail(USP_ERR_INVALID_ARG, "%s: ring_rank %d out of range", who, (int)ring_rank);
  const int64_t L = d->seq_len / d->cp;
  if (d->seq_len >= kMaxIndex || d->batch * d->num_q_heads * L * d->cp >= kMaxIndex)
    return fail(USP_ERR_UNSUPPORTED, "%s: problem too large for 32-bit row indices", who);
  // every stride the kernels use must keep 16-byte alignment of a head row
  const int64_t e = elem_bytes(d->dtype);
  const int64_t strides[] = {d->q.b, d->q.s, d->q.h, d->k.b, d->k.s, d->k.h, d->v.b, d->v.s,
                             d->v.h, d->kv_block_stride};
  for (int64_t s : strides)
    if (s < 0 || (s * e) % 16 != 0)
      return fail(USP_ERR_INVALID_ARG, "%s: strides must be >= 0 and keep 16-byte alignment", who);
  if (d->dtype == USP_DTYPE_BF16 &&
      (!rows_span_32bit(L, d->k.s, e, d->head_dim) || !rows_span_32bit(L, d->v.s, e, d->head_dim)))
    return fail(USP_ERR_UNSUPPORTED, "%s: the %lld rows of a K/V block slice span 4 GiB or more at row stride "
                "%lld (the head-major layout keeps them dense)", who, (long long)L,
                (long long)(d->k.s > d->v.s ? d->k.s : d->v.s));

  a = usp::AttnArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = const_cast<void *>(o);
  a.lse = const_cast<float *>(lse);
  a.B = (int32_t)d->batch;
  a.Hq = (int32_t)d->num_q_heads;
  a.Hkv = (int32_t)d->num_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.L = (int32_t)L;
  a.c = (int32_t)(L / 2);
  a.cp = d->cp;
  a.causal = d->causal;
  a.q_sb = d->q.b; a.q_ss = d->q.s; a.q_sh = d->q.h;
  a.k_sb = d->k.b; a.k_ss = d->k.s; a.k_sh = d->k.h;
  a.v_sb = d->v.b; a.v_ss = d->v.s; a.v_sh = d->v.h;
  a.o_sb = d->o.b; a.o_ss = d->o.s; a.o_sh = d->o.h;
  a.kv_blk = d->kv_block_stride;
  a.q_rank = d->q_rank_stride;
  a.o_rank = d->o_rank_stride;
  a.scale = d->softmax_scale;
  a.scale_log2 = (float)((double)d->softmax_scale * 1.4426950408889634074);
  a.ring_rank = ring_rank;
  a.n_ranks = ring_rank < 0 ? d->cp : 1;
  a.n_qtiles = (int32_t)((L + 127) / 128);
  const int64_t groups = (int64_t)a.n_ranks * a.n_qtiles * a.B * a.Hkv;
  a.xcd_remap = groups % 8 == 0;
  return read_samples(d->cu_seqlens, d->num_seqs, d->seq_len, d->zigzag_per_sample ? d->cp : 0, a.sm, who);
}

usp_status attn_launch(const usp::AttnArgs &a, const usp_attn_desc *d, void *stream, const char *who) {
  hipError_t e = d->dtype == USP_DTYPE_BF16
                     ? usp::launch_attn_bf16(a, (int)d->head_dim, static_cast<hipStream_t>(stream))
                     : usp::launch_attn_fp32(a, (int)d->head_dim, static_cast<hipStream_t>(stream));
  return hip_result(e, who);
}

// ---------------------------------------------------------------- backward

constexpr int64_t kMaxStatsRows = (int64_t)1 << 29;

// O and dO are read with 16-byte vector loads and 16-byte direct tile loads.
usp_status o_strides_check(const usp_attn_desc *d, int32_t ring_rank, const char *who) {
  const int64_t e = elem_bytes(d->dtype);
  const int64_t st[] = {d->o.b, d->o.s, d->o.h, ring_rank < 0 ? d->o_rank_stride : 0,
                        ring_rank < 0 ? d->q_rank_stride : 0};
  for (int64_t s : st)
    if (s < 0 || (s * e) % 16 != 0)
      return fail(USP_ERR_INVALID_ARG, "%s: O/dO strides and rank strides must be >= 0 and keep 16-byte alignment",
                  who);
  return USP_OK;
}

int64_t stats_rows(const usp_attn_desc *d, int32_t ring_rank) {
  return (ring_rank < 0 ? (int64_t)d->cp : 1) * d->num_q_heads * d->batch * (d->seq_len / d->cp);
}

usp_status bwd_prepare(const void *q, const void *k, const void *v, const void *d_o, const float *stats,
                       const usp_attn_desc *d, int32_t ring_rank, bool all_ranks_ok, usp::BwdArgs &b,
                       const char *who) {
  usp::AttnArgs a;
  usp_status s = attn_prepare(q, k, v, d_o, stats, d, ring_rank, all_ranks_ok, a, who);
  if (s != USP_OK) return s;
  if ((s = o_strides_check(d, ring_rank, who)) != USP_OK) return s;
  const int64_t rows = stats_rows(d, ring_rank);
  if (rows >= kMaxStatsRows)
    return fail(USP_ERR_INVALID_ARG, "%s: %lld statistics rows (limit 2^29)", who, (long long)rows);
  if (d->dtype == USP_DTYPE_BF16 && (!rows_span_32bit(a.L, d->q.s, 2, d->head_dim) ||
                                     !rows_span_32bit(a.L, d->o.s, 2, d->head_dim)))
    return fail(USP_ERR_UNSUPPORTED, "%s: the %lld rows of a Q/dO slice span 4 GiB or more (the head-major "
                "layout keeps them dense)", who, (long long)a.L);
  b = usp::BwdArgs{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.dout = d_o;
  b.stats = stats;
  b.rows = rows;
  b.B = a.B; b.Hq = a.Hq; b.Hkv = a.Hkv; b.G = a.G;
  b.L = a.L; b.c = a.c; b.cp = a.cp; b.causal = a.causal;
  b.q_sb = a.q_sb; b.q_ss = a.q_ss; b.q_sh = a.q_sh;
  b.k_sb = a.k_sb; b.k_ss = a.k_ss; b.k_sh = a.k_sh;
  b.v_sb = a.v_sb; b.v_ss = a.v_ss; b.v_sh = a.v_sh;
  b.do_sb = d->o.b; b.do_ss = d->o.s; b.do_sh = d->o.h;
  b.kv_blk = a.kv_blk;
  b.q_rank = a.q_rank;
  b.do_rank = a.o_rank;
  b.scale = a.scale;
  b.scale_log2 = a.scale_log2;
  b.sm = a.sm;
  b.ring_rank = ring_rank;
  b.n_ranks = a.n_ranks;
  return USP_OK;
}

usp_status grads_check(const void *dq, const float *dk, const float *dv, const void *q, const void *k,
                       const void *v, const char *who) {
  if (!dq || !dk || !dv) return fail(USP_ERR_INVALID_ARG, "%s: null gradient pointer", who);
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(USP_ERR_INVALID_ARG, "%s: gradient buffers must be 16-byte aligned", who);
  if (dq == q || (const void *)dk == k || (const void *)dv == v || (const void *)dk == v ||
      (const void *)dv == k || (const void *)dk == (const void *)dv || dq == (const void *)dk ||
      dq == (const void *)dv)
    return fail(USP_ERR_INVALID_ARG, "%s: gradient buffers must not alias each other or the inputs", who);
  return USP_OK;
}

usp_status prep_launch(const void *o, const void *d_o, const float *lse, float *stats, const usp_attn_desc *d,
                       int32_t ring_rank, void *stream, const char *who) {
  usp::PrepArgs p{};
  p.o = o;
  p.dout = d_o;
  p.lse = lse;
  p.stats = stats;
  p.rows = stats_rows(d, ring_rank);
  p.B = (int32_t)d->batch;
  p.Hq = (int32_t)d->num_q_heads;
  p.L = (int32_t)(d->seq_len / d->cp);
  p.o_sb = p.do_sb = d->o.b;
  p.o_ss = p.do_ss = d->o.s;
  p.o_sh = p.do_sh = d->o.h;
  p.o_rank = p.do_rank = ring_rank < 0 ? d->o_rank_stride : 0;
  return hip_result(usp::launch_bwd_prep(p, (int)d->head_dim, d->dtype == USP_DTYPE_BF16,
                                         static_cast<hipStream_t>(stream)), who);
}

usp_status bwd_launch(const usp::BwdArgs &b, const usp_attn_desc *d, void *stream, const char *who) {
  hipError_t e = d->dtype == USP_DTYPE_BF16
                     ? usp::launch_attn_bwd_bf16(b, (int)d->head_dim, static_cast<hipStream_t>(stream))
                     : usp::launch_attn_bwd_fp32(b, (int)d->head_dim, static_cast<hipStream_t>(stream));
  return hip_result(e, who);
}

}  // namespace

extern "C" {

usp_status usp_ring_attn_step_fwd(const void *q, const void *k_all, const void *v_all, float *o_step,
                                  float *lse_step, const usp_attn_desc *desc, int32_t ring_rank,
                                  int32_t step, void *stream) {
  usp::AttnArgs a;
  usp_status s = attn_prepare(q, k_all, v_all, o_step, lse_step, desc, ring_rank, false, a,
                              "ring_attn_step_fwd");
  if (s != USP_OK) return s;
  if (!aligned16(o_step)) return fail(USP_ERR_INVALID_ARG, "ring_attn_step_fwd: o_step must be 16-byte aligned");
  if (step < 0 || step >= desc->cp)
    return fail(USP_ERR_INVALID_ARG, "ring_attn_step_fwd: step %d out of range", (int)step);
  a.t_lo = step;
  a.t_hi = step + 1;
  a.partial = 1;
  return attn_launch(a, desc, stream, "ring_attn_step_fwd launch");
}

usp_status usp_ring_attn_step_fwd_merge(const void *q, const void *k_all, const void *v_all, float *o_acc,
                                        float *lse_acc, const usp_attn_desc *desc, int32_t ring_rank,
                                        int32_t step, void *stream) {
  const char *who = "ring_attn_step_fwd_merge";
  usp::AttnArgs a;
  usp_status s = attn_prepare(q, k_all, v_all, o_acc, lse_acc, desc, ring_rank, false, a, who);
  if (s != USP_OK) return s;
  if (step < 0 || step >= desc->cp) return fail(USP_ERR_INVALID_ARG, "%s: step %d out of range", who, (int)step);
  a.t_lo = step;
  a.t_hi = step + 1;
  a.partial = 1;
  a.merge = 1;
  return attn_launch(a, desc, stream, "ring_attn_step_fwd_merge launch");
}

usp_status usp_attn_fwd(const void *q, const void *k_all, const void *v_all, void *o, float *lse,
                        const usp_attn_desc *desc, int32_t ring_rank, void *stream) {
  usp::AttnArgs a;
  usp_status s = attn_prepare(q, k_all, v_all, o, lse, desc, ring_rank, true, a, "attn_fwd");
  if (s != USP_OK) return s;
  const int64_t e = elem_bytes(desc->dtype);
  const int64_t ostr[] = {desc->o.b, desc->o.s, desc->o.h, desc->q_rank_stride, desc->o_rank_stride};
  for (int64_t st : ostr)
    if (st < 0 || (st * e) % 8 != 0)
      return fail(USP_ERR_INVALID_ARG, "attn_fwd: o and rank strides must be >= 0 and keep 8-byte alignment");
  if (ring_rank < 0 && (desc->q_rank_stride * e) % 16 != 0)
    return fail(USP_ERR_INVALID_ARG, "attn_fwd: q_rank_stride must keep 16-byte alignment");
  a.t_lo = 0;
  a.t_hi = desc->cp;
  a.partial = 0;
  return attn_launch(a, desc, stream, "attn_fwd launch");
}

int64_t usp_attn_fwd_split_workspace(const usp_attn_desc *desc, int32_t ring_rank) {
  if (!desc || desc->cp < 1 || desc->seq_len < 1 || desc->batch < 1 || desc->num_q_heads < 1 || desc->head_dim < 1 ||
      ring_rank < -1 || ring_rank >= desc->cp)
    return -1;
  const int64_t rows = stats_rows(desc, ring_rank);
  return 2 * rows * (desc->head_dim + 1) * 4;
}

usp_status usp_attn_fwd_split(const void *q, const void *k_all, const void *v_all, void *o, float *lse,
                              const usp_attn_desc *desc, int32_t ring_rank, void *workspace,
                              int64_t workspace_bytes, void *stream) {
  const char *who = "attn_fwd_split";
  usp::AttnArgs a;
  usp_status s = attn_prepare(q, k_all, v_all, o, lse, desc, ring_rank, true, a, who);
  if (s != USP_OK) return s;
  const int64_t e = elem_bytes(desc->dtype);
  const int64_t ostr[] = {desc->o.b, desc->o.s, desc->o.h, desc->q_rank_stride, desc->o_rank_stride};
  for (int64_t st : ostr)
    if (st < 0 || (st * e) % 8 != 0)
      return fail(USP_ERR_INVALID_ARG, "%s: o and rank strides must be >= 0 and keep 8-byte alignment", who);
  if (ring_rank < 0 && (desc->q_rank_stride * e) % 16 != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: q_rank_stride must keep 16-byte alignment", who);
  const int64_t need = usp_attn_fwd_split_workspace(desc, ring_rank);
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(USP_ERR_INVALID_ARG, "%s: workspace must be non-null and 256-byte aligned", who);
  if (workspace_bytes < need)
    return fail(USP_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", who, (long long)workspace_bytes,
                (long long)need);
  a.t_lo = 0;
  a.t_hi = desc->cp;
  a.partial = 0;
  if (desc->dtype != USP_DTYPE_BF16) return attn_launch(a, desc, stream, "attn_fwd_split launch");
  const int64_t rows = stats_rows(desc, ring_rank);
  usp::SplitPlan plan{};
  plan.po = static_cast<float *>(workspace);
  plan.slot_o = rows * desc->head_dim;
  plan.pl = plan.po + 2 * plan.slot_o;
  plan.slot_lse = rows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = hip_result(usp::launch_attn_bf16_split(a, (int)desc->head_dim, plan, st), "attn_fwd_split walk")) !=
      USP_OK)
    return s;
  if (!plan.split) return USP_OK;
  usp::FinalizeArgs f{};
  f.po = plan.po;
  f.pl = plan.pl;
  f.slot_o = plan.slot_o;
  f.slot_lse = plan.slot_lse;
  f.o = o;
  f.lse = lse;
  f.o_sb = desc->o.b;
  f.o_ss = desc->o.s;
  f.o_sh = desc->o.h;
  f.o_rank = ring_rank < 0 ? desc->o_rank_stride : 0;
  f.rows = rows;
  f.B = a.B;
  f.Hq = a.Hq;
  f.L = a.L;
  f.d4 = (int32_t)(desc->head_dim / 4);
  f.ring_rank = ring_rank;
  f.bm = plan.bm;
  f.n_qtiles = plan.n_qtiles;
  for (int i = 0; i < usp::kMaxTileOrder / 32; ++i) f.mask[i] = plan.mask[i];
  return hip_result(usp::launch_split_finalize(f, st), "attn_fwd_split finalize");
}

usp_status usp_attn_bwd_prep(const void *o, const void *d_o, const float *lse, float *stats,
                             const usp_attn_desc *desc, int32_t ring_rank, void *stream) {
  const char *who = "attn_bwd_prep";
  if (!desc) return fail(USP_ERR_INVALID_ARG, "%s: null descriptor", who);
  if (!o || !d_o || !lse || !stats) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(o) || !aligned16(d_o))
    return fail(USP_ERR_INVALID_ARG, "%s: o and d_o must be 16-byte aligned", who);
  if (o == d_o) return fail(USP_ERR_INVALID_ARG, "%s: o and d_o must be distinct buffers", who);
  // the descriptor checks of the attention entry points, with O standing in
  // for the inputs it does not use here
  usp::AttnArgs a;
  usp_status s = attn_prepare(o, o, o, d_o, stats, desc, ring_rank, true, a, who);
  if (s != USP_OK) return s;
  if ((s = o_strides_check(desc, ring_rank, who)) != USP_OK) return s;
  const int64_t rows = stats_rows(desc, ring_rank);
  if (rows >= kMaxStatsRows)
    return fail(USP_ERR_INVALID_ARG, "%s: %lld statistics rows (limit 2^29)", who, (long long)rows);
  return prep_launch(o, d_o, lse, stats, desc, ring_rank, stream, "attn_bwd_prep launch");
}

usp_status usp_ring_attn_step_bwd(const void *q, const void *k_all, const void *v_all, const void *d_o,
                                  const float *stats, float *dq_acc, float *dk_all, float *dv_all,
                                  const usp_attn_desc *desc, int32_t ring_rank, int32_t step, void *stream) {
  const char *who = "ring_attn_step_bwd";
  usp::BwdArgs b;
  usp_status s = bwd_prepare(q, k_all, v_all, d_o, stats, desc, ring_rank, false, b, who);
  if (s != USP_OK) return s;
  if ((s = grads_check(dq_acc, dk_all, dv_all, q, k_all, v_all, who)) != USP_OK) return s;
  if (step < 0 || step >= desc->cp) return fail(USP_ERR_INVALID_ARG, "%s: step %d out of range", who, (int)step);
  b.dq = dq_acc;
  b.dk = dk_all;
  b.dv = dv_all;
  b.t_lo = step;
  b.t_hi = step + 1;
  b.dq_acc = 1;
  return bwd_launch(b, desc, stream, "ring_attn_step_bwd launch");
}

usp_status usp_attn_bwd(const void *q, const void *k_all, const void *v_all, const void *o, const void *d_o,
                        const float *lse, void *dq, float *dk_all, float *dv_all, float *stats,
                        const usp_attn_desc *desc, int32_t ring_rank, void *stream) {
  return usp::attn_bwd_with_stats(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all, stats, desc, ring_rank, stream,
                                  "attn_bwd");
}

}  // extern "C"

namespace usp {

usp_status report(usp_status s, const char *msg) { return s == USP_OK ? ok() : fail(s, "%s", msg); }

int64_t bwd_stats_rows(const usp_attn_desc *d, int32_t ring_rank) { return stats_rows(d, ring_rank); }

usp_status attn_bwd_with_stats(const void *q, const void *k_all, const void *v_all, const void *o, const void *d_o,
                               const float *lse, void *dq, float *dk_all, float *dv_all, float *stats,
                               const usp_attn_desc *desc, int32_t ring_rank, void *stream, const char *who) {
  usp::BwdArgs b;
  usp_status s = bwd_prepare(q, k_all, v_all, d_o, stats, desc, ring_rank, true, b, who);
  if (s != USP_OK) return s;
  if ((s = grads_check(dq, dk_all, dv_all, q, k_all, v_all, who)) != USP_OK) return s;
  if (!o || !lse) return fail(USP_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(o)) return fail(USP_ERR_INVALID_ARG, "%s: o must be 16-byte aligned", who);
  if (o == d_o || dq == o || dq == d_o)
    return fail(USP_ERR_INVALID_ARG, "%s: o, d_o and dq must be distinct buffers", who);
  if ((s = prep_launch(o, d_o, lse, stats, desc, ring_rank, stream, "attn_bwd prep launch")) != USP_OK) return s;
  b.dq = dq;
  b.dk = dk_all;
  b.dv = dv_all;
  b.t_lo = 0;
  b.t_hi = desc->cp;
  b.dq_acc = 0;
  return bwd_launch(b, desc, stream, "attn_bwd launch");
}

}  // namespace usp
