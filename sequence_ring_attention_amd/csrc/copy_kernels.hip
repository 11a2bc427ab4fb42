// Zigzag split and Ulysses all-to-all layout as batched 2D row copies.
//
// Both are pure data movement, bound by HBM bandwidth.  Every shape reduces
// to "items": runs of rows that are contiguous (or evenly strided) on both
// sides, so each workgroup copies whole 16-byte vectors with one scalar
// index decode per piece instead of per element.
//
// Zigzag ("USP" paper review, section 三, Algorithm 2): the share of ring
// rank r is chunk r followed by chunk 2rd-1-r; the u-th of ud equal parts of
// it belongs to Ulysses rank u.  In (B, S, H, D) a token's H*D elements are
// one contiguous row, so a shard is at most two contiguous runs of rows.
//
// Ulysses (same section, the AllToAll4D box (bs, L/N, hc, hd) ->
// (hc/N, bs, L, hd)): for fixed (head h', batch b, source peer u') the
// Ls = L/N rows of D elements are strided by hc*D on the sequence-major side
// and contiguous on the head-major side.  The forward copies such head rows
// (strided reads, contiguous writes).  The inverse writes whole output rows
// instead: a token's hc heads are contiguous in the output, and head
// u' hc/N + h' is plane u' hc/N + h' of the head-major input, so a row is
// gathered from the hc planes; writes then stream and only reads gather, as
// in the forward.
#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
// workgroups of a row-copy launch (each loops over its pieces); 8192 held
// the whole-Q extract of the 128K-token share at 5.9 TB/s, 65536 gives 6.1
constexpr uint32_t kMaxCopyGrid = 65536;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct RowMap {
  int64_t src_base, src_stride, dst_base, dst_stride;  // in rows
  int64_t split, src_jump, dst_jump;                   // rows t >= split add the jumps
  int64_t src_grp;                                     // source rows between the pieces of a gathered row
  int64_t dst_grp;                                     // destination rows between the pieces of a scattered row
};

__device__ inline RowMap decode(const CopyPlan &P, uint32_t item) {
  RowMap m;
  m.split = INT64_MAX;
  m.src_jump = m.dst_jump = 0;
  m.src_grp = 0;
  m.dst_grp = 0;
  if (P.kind == kZigzagFwd || P.kind == kZigzagInv) {
    const int64_t B = P.p[0], S = P.p[1], c = P.p[2], rd = P.p[3], ud = P.p[4], T = P.p[5];
    const int64_t r_fix = P.p[6], u_fix = P.p[7];
    const int64_t b = item % B, g = item / B;
    int64_t r, u;
    if (r_fix < 0) {
      r = g / ud;
      u = g % ud;
    } else if (u_fix < 0) {
      r = r_fix;
      u = g;
    } else {
      r = r_fix;
      u = u_fix;
    }
    // local index l = u*T + t; position r*c + l for l < c, (2rd-1-r)*c + l - c after.
    const int64_t global_base = b * S + r * c + u * T;
    const int64_t split = c - u * T;
    const int64_t jump = (2 * rd - 1 - r) * c - c - r * c;
    const int64_t shard_base = (int64_t)item * T;
    if (P.kind == kZigzagFwd) {
      m.src_base = global_base;
      m.dst_base = shard_base;
      m.src_jump = jump;
    } else {
      m.src_base = shard_base;
      m.dst_base = global_base;
      m.dst_jump = jump;
    }
    m.src_stride = m.dst_stride = 1;
    m.split = split;
  } else if (P.kind == kUlyssesFwd) {
    const int64_t bs = P.p[0], L = P.p[1], hc = P.p[2], N = P.p[3], hb = P.p[4], Ls = P.p[5];
    const int64_t u_fix = P.p[6], h0 = P.p[7], nh = P.p[8];
    int64_t rest = item;
    const int64_t up = rest % N;
    rest /= N;
    const int64_t b = rest % bs;
    rest /= bs;
    const int64_t hp = rest % nh;
    const int64_t g = rest / nh;
    const int64_t u = u_fix < 0 ? g : u_fix;
    m.dst_base = ((g * nh + hp) * bs + b) * L + up * Ls;
    m.dst_stride = 1;
    m.src_base = ((up * bs + b) * Ls) * hc + u * hb + h0 + hp;
    m.src_stride = hc;
  } else if (P.kind == kUlyssesFwdRows) {
    // item (g, b, peer u'); row t = token t of shard u': its heads
    // u hb + h0 .. + nh, contiguous in the source (head rows count the
    // offsets); head i of the row goes to output plane g nh + i (dst_grp
    // rows apart), row b L + u' Ls + t
    const int64_t bs = P.p[0], L = P.p[1], hc = P.p[2], N = P.p[3], hb = P.p[4], Ls = P.p[5];
    const int64_t u_fix = P.p[6], h0 = P.p[7], nh = P.p[8];
    int64_t rest = item;
    const int64_t up = rest % N;
    rest /= N;
    const int64_t b = rest % bs, g = rest / bs;
    const int64_t u = u_fix < 0 ? g : u_fix;
    m.src_base = ((up * bs + b) * Ls) * hc + u * hb + h0;
    m.src_stride = hc;
    m.dst_base = (g * nh * bs + b) * L + up * Ls;
    m.dst_stride = 1;
    m.dst_grp = bs * L;
  } else if (P.kind == kUlyssesInvRows) {
    // item (g, b, peer group); row t = token t of output shard g: heads
    // u' hb + h0 .. + nh of one peer u' (np = N), or all hc heads when the
    // chunk is the whole block (np = 1, u' = 0: head hh is plane hh); head i
    // of the row comes from input plane u' nh + i (src_grp rows apart), and
    // destination offsets count head rows
    const int64_t bs = P.p[0], L = P.p[1], hc = P.p[2], hb = P.p[4], Ls = P.p[5];
    const int64_t u_fix = P.p[6], h0 = P.p[7], nh = P.p[8], np = P.p[9];
    int64_t rest = item;
    const int64_t up = rest % np;
    rest /= np;
    const int64_t b = rest % bs, g = rest / bs;
    const int64_t u = u_fix < 0 ? g : u_fix;
    m.src_base = (up * nh * bs + b) * L + u * Ls;
    m.src_stride = 1;
    m.src_grp = bs * L;
    m.dst_base = (g * bs + b) * Ls * hc + up * hb + h0;
    m.dst_stride = hc;
  } else {  // kUlyssesInv: one head row per row
    const int64_t bs = P.p[0], L = P.p[1], hc = P.p[2], N = P.p[3], hb = P.p[4], Ls = P.p[5];
    const int64_t u_fix = P.p[6], h0 = P.p[7], nh = P.p[8];
    int64_t rest = item;
    const int64_t hp = rest % nh;
    rest /= nh;
    const int64_t up = rest % N;
    rest /= N;
    const int64_t b = rest % bs;
    const int64_t g = rest / bs;
    const int64_t u = u_fix < 0 ? g : u_fix;
    m.src_base = ((up * nh + hp) * bs + b) * L + u * Ls;
    m.src_stride = 1;
    m.dst_base = ((g * bs + b) * Ls) * hc + up * hb + h0 + hp;
    m.dst_stride = hc;
  }
  return m;
}

// One piece (a run of rows of one item) of plan P, by the whole workgroup.
__device__ inline void copy_piece(const CopyPlan &P, uint32_t piece) {
  const uint32_t item = piece / P.pieces_per_item;
  const uint32_t row0 = (piece - item * P.pieces_per_item) * P.rows_per_piece;
  const uint32_t nrows = min(P.rows_per_piece, P.rows_per_item - row0);
  const RowMap m = decode(P, item);
  const uint32_t nvec = nrows * P.row_vecs;
  for (uint32_t v0 = threadIdx.x; v0 < nvec; v0 += kThreads * kUnroll) {
    u32x4 buf[kUnroll];
    int64_t doff[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const uint32_t idx = v0 + k * kThreads;
      doff[k] = -1;
      if (idx < nvec) {
        uint32_t row, col;
        if (P.row_vecs_shift < 31) {
          row = idx >> P.row_vecs_shift;
          col = idx & (P.row_vecs - 1);
        } else {
          row = idx / P.row_vecs;
          col = idx - row * P.row_vecs;
        }
        const int64_t t = (int64_t)row0 + row;
        const bool second = t >= m.split;
        // head row of a gathered or scattered row (0 unless grp_shift < 31)
        // and the vector within it; a gathered row reads head rows from
        // several source planes, a scattered one writes them to several
        // destination planes
        const uint32_t grp = P.grp_shift < 31 ? col >> P.grp_shift : 0;
        const uint32_t gcol = col - (grp << (P.grp_shift & 31));
        const bool scatter = P.kind == kUlyssesFwdRows;
        const int64_t srow = m.src_base + t * m.src_stride + grp * m.src_grp + (second ? m.src_jump : 0);
        const int64_t drow = m.dst_base + t * m.dst_stride + grp * m.dst_grp + (second ? m.dst_jump : 0);
        buf[k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(P.src + srow * (int64_t)P.src_row_bytes) + (scatter ? col : gcol));
        doff[k] = drow * (int64_t)P.dst_unit_bytes + (int64_t)(scatter ? gcol : col) * 16;
      }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      if (doff[k] >= 0) __builtin_nontemporal_store(buf[k], reinterpret_cast<u32x4 *>(P.dst + doff[k]));
    }
  }
}

__global__ __launch_bounds__(kThreads) void copy_rows_kernel(CopyPlan P) {
  const uint32_t total = P.n_items * P.pieces_per_item;
  for (uint32_t piece = blockIdx.x; piece < total; piece += gridDim.x) copy_piece(P, piece);
}

// Several plans in one launch: the pieces of plan i are global pieces
// [first[i], first[i + 1]), dealt to the workgroups like those of one plan.
__global__ __launch_bounds__(kThreads) void copy_rows_n_kernel(CopyBatch C) {
  const uint32_t total = C.first[C.n];
  for (uint32_t piece = blockIdx.x; piece < total; piece += gridDim.x) {
    int i = 0;
#pragma unroll
    for (int k = 1; k < kMaxCopyBatch; ++k) i += (k < C.n) & (piece >= C.first[k]);
    copy_piece(C.plan[i], piece - C.first[i]);
  }
}

// Per-sample zigzag extract ([USP review] section 三, Algorithm 2 applied to
// every packed sample): row t of the shard of (ring rank r, Ulysses rank u)
// is row u T + t of rank r's share, whose global position the share map
// gives.  One thread per 16-byte vector; the shard buffer is rank-major
// (ranks in use, Ulysses ranks in use, B, T, row).
__global__ __launch_bounds__(kThreads) void zigzag_varlen_kernel(ZigzagVarlenArgs a) {
  const int64_t vecs = a.row_bytes / 16;
  const int n_u = a.ulysses_rank >= 0 ? 1 : a.ud;
  const int n_r = a.ring_rank >= 0 ? 1 : a.rd;
  const int64_t total = (int64_t)n_r * n_u * a.B * a.T * vecs;
  const ShareMap sm(0, a.rd, a.S / a.rd, a.sm);
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t vec = idx % vecs;
    const int64_t srow = idx / vecs;  // row of the shard buffer
    int64_t rest = srow;
    const int t = (int)(rest % a.T);
    rest /= a.T;
    const int b = (int)(rest % a.B);
    rest /= a.B;
    const int ui = (int)(rest % n_u);
    const int ri = (int)(rest / n_u);
    const int r = a.ring_rank >= 0 ? a.ring_rank : ri;
    const int u = a.ulysses_rank >= 0 ? a.ulysses_rank : ui;
    const int64_t grow = (int64_t)b * a.S + sm.pos(r, u * a.T + t);  // row of (B, S, H, D)
    const int64_t from = (a.inverse ? srow : grow) * a.row_bytes + vec * 16;
    const int64_t to = (a.inverse ? grow : srow) * a.row_bytes + vec * 16;
    __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.src + from)),
                                reinterpret_cast<u32x4 *>(a.dst + to));
  }
}

}  // namespace

hipError_t launch_zigzag_varlen(const ZigzagVarlenArgs &a, hipStream_t stream) {
  const int64_t n_u = a.ulysses_rank >= 0 ? 1 : a.ud, n_r = a.ring_rank >= 0 ? 1 : a.rd;
  const int64_t total = n_r * n_u * a.B * a.T * (a.row_bytes / 16);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(zigzag_varlen_kernel, dim3((uint32_t)(blocks < 8192 ? blocks : 8192)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_n(const CopyPlan *plans, int n, hipStream_t stream) {
  CopyBatch C{};
  C.n = n;
  C.first[0] = 0;
  for (int i = 0; i < n; ++i) {
    C.plan[i] = plans[i];
    C.first[i + 1] = C.first[i] + plans[i].n_items * plans[i].pieces_per_item;
  }
  const uint32_t total = C.first[n];
  if (total == 0) return hipSuccess;
  const uint32_t grid = total < kMaxCopyGrid ? total : kMaxCopyGrid;
  hipLaunchKernelGGL(copy_rows_n_kernel, dim3(grid), dim3(kThreads), 0, stream, C);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyPlan &plan, hipStream_t stream) {
  const uint64_t total = (uint64_t)plan.n_items * plan.pieces_per_item;
  if (total == 0) return hipSuccess;
  const uint32_t grid = (uint32_t)(total < kMaxCopyGrid ? total : kMaxCopyGrid);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(grid), dim3(kThreads), 0, stream, plan);
  return hipGetLastError();
}

}  // namespace usp
