// Ring-step / ring-walk attention for fp32 inputs (small problems).
//
// One workgroup of four wavefronts per (rank, query head, batch, query row):
// the wavefronts take turns over the row's visible keys in groups of 16 and
// each keeps its own running max, sum and output, merged at the end by the
// LSE rule; the 64 lanes of a wavefront split head_dim.  Logits, the running
// max/sum and the output accumulator are kept in double: a product of two
// floats is exact in double, so the only rounding that reaches the fp32
// outputs is the final one.
//
// Semantics as the bf16 kernel (positions from the share map of either
// split): ring rank r at step t reads KV block
// (r - t) mod cp ("Context Parallel 与 Ulysses", concepts section and
// Figure 1); a key is visible iff its global position is <= the query's
// (causal) and, for packed samples, inside the query's sample.  The fold over
// steps is the online form of the LSE merge of the same page.
#include "lse_rule.h"
#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;
constexpr int KB = 16;  // keys per group

// Lane i's value of x, in every lane.
__device__ inline double read_lane(double x, int i) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, i);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), i);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fp32_kernel(AttnArgs a) {
  constexpr int PER = D / 64;  // elements per lane (1 or 2)
  constexpr int NWV = kThreads / 64;
  // the four wavefronts of a workgroup share one query row: wavefront w
  // takes key groups w, w + 4, ... of the row's walk, and wavefront 0 merges
  // the four partial results by the LSE rule
  __shared__ double part_m[NWV], part_l[NWV], part_acc[NWV][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int64_t rest = blockIdx.x;
  const int qrow = (int)(rest % a.L);
  rest /= a.L;
  const int b = (int)(rest % a.B);
  rest /= a.B;
  const int hq = (int)(rest % a.Hq);
  const int rank = a.ring_rank >= 0 ? a.ring_rank : (int)(rest / a.Hq);
  const int kvh = hq / a.G;
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  const int qpos = sm.pos(rank, qrow);
  const int sst = sm.packed() ? sm.seg_start(qpos) : 0;

  const float *qp = static_cast<const float *>(a.q) + (a.ring_rank < 0 ? rank * a.q_rank : 0) +
                    b * a.q_sb + (int64_t)qrow * a.q_ss + hq * a.q_sh;
  double qv[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qv[e] = (double)qp[lane + 64 * e];
    acc[e] = 0.0;
  }
  const double scale = (double)a.scale;
  double m = -INFINITY, l = 0.0;
  int grp = 0;  // key groups of the row's walk so far
  for (int t = a.t_lo; t < a.t_hi; ++t) {
    int j = (rank - t) % a.cp;
    if (j < 0) j += a.cp;
    const float *kb = static_cast<const float *>(a.k) + j * a.kv_blk + b * a.k_sb + kvh * a.k_sh;
    const float *vb = static_cast<const float *>(a.v) + j * a.kv_blk + b * a.v_sb + kvh * a.v_sh;
    // positions grow with the local row, so the keys of block j this row
    // sees are the local rows [lo, hi): at or before the query (causal) and
    // not before its sample's start (sst = 0 for one sequence)
    const int hi = __builtin_amdgcn_readfirstlane(a.causal ? sm.count_le(j, qpos) : a.L);
    const int lo = __builtin_amdgcn_readfirstlane(sst > 0 ? sm.count_le(j, sst - 1) : 0);
    // KB keys at a time: their partial dot products are summed across the
    // wavefront in one pass of independent shuffles, and the running max,
    // sum and output are rescaled once per group
    for (int k0 = lo; k0 < hi; k0 += KB, ++grp) {
      if (grp % NWV != wv) continue;
      const int n = hi - k0 < KB ? hi - k0 : KB;
      // the group's K and V elements are requested together: one memory
      // latency per group
      double part[KB];
      float vv[KB][PER];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        part[i] = 0.0;
#pragma unroll
        for (int e = 0; e < PER; ++e) vv[i][e] = i < n ? vb[(int64_t)(k0 + i) * a.v_ss + lane + 64 * e] : 0.0f;
        if (i < n) {
#pragma unroll
          for (int e = 0; e < PER; ++e) part[i] += qv[e] * (double)kb[(int64_t)(k0 + i) * a.k_ss + lane + 64 * e];
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
        for (int i = 0; i < KB; ++i) part[i] += __shfl_xor(part[i], off);
      }
      double m_new = m;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        part[i] *= scale;
        if (i < n) m_new = part[i] > m_new ? part[i] : m_new;
      }
      const double alpha = exp(m - m_new);  // m = -inf before the first key: alpha = 0
      l *= alpha;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] *= alpha;
      // lane i < n takes key k0 + i's probability (one exp per lane instead
      // of every lane evaluating all of them), read back lane by lane
      double mine = part[0];
#pragma unroll
      for (int i = 1; i < KB; ++i) mine = lane == i ? part[i] : mine;
      const double pl = lane < n ? exp(mine - m_new) : 0.0;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (i < n) {
          const double p = read_lane(pl, i);
          l += p;
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += p * (double)vv[i][e];
        }
      }
      m = m_new;
    }
  }
  // the four partials -> wavefront 0
  if (lane == 0) {
    part_m[wv] = m;
    part_l[wv] = l;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) part_acc[wv][lane + 64 * e] = acc[e];
  __syncthreads();
  if (wv != 0) return;
  {
    double mm = part_m[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) mm = part_m[i] > mm ? part_m[i] : mm;
    l = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0;
    if (mm != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NWV; ++i) {
        const double f = exp(part_m[i] - mm);  // 0 for a wavefront that saw no key
        l += part_l[i] * f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += part_acc[i][lane + 64 * e] * f;
      }
    }
    m = mm;
  }
  const bool empty = l == 0.0;
  const double inv = empty ? 0.0 : 1.0 / l;
  const float lse = empty ? -INFINITY : (float)(m + log(l));
  if (a.partial && a.merge) {
    // the step's partial folded into the accumulator by the LSE rule (see the
    // bf16 kernel); every lane reads the row's lse before lane 0 stores it
    const int64_t prow = ((int64_t)hq * a.B + b) * a.L + qrow;
    float *o = static_cast<float *>(a.o) + prow * D;
    const float la = a.lse[prow];
    double w1, w2, lm;
    merge_weights((double)la, (double)lse, w1, w2, lm);
    const bool take = la == -INFINITY, keep = !take && empty;
    if (!keep) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float y = (float)(acc[e] * inv);
        o[lane + 64 * e] = take ? y : blend1(w1, o[lane + 64 * e], w2, y);
      }
      if (lane == 0) a.lse[prow] = take ? lse : (float)lm;
    }
    return;
  }
  if (a.partial) {
    float *o = static_cast<float *>(a.o) + (((int64_t)hq * a.B + b) * a.L + qrow) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (float)(acc[e] * inv);
  } else {
    float *o = static_cast<float *>(a.o) + (a.ring_rank < 0 ? rank * a.o_rank : 0) + b * a.o_sb +
               (int64_t)qrow * a.o_ss + hq * a.o_sh;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (float)(acc[e] * inv);
  }
  if (lane == 0) {
    const int64_t li = (((a.ring_rank < 0 ? (int64_t)rank * a.Hq : 0) + hq) * a.B + b) * a.L + qrow;
    a.lse[li] = lse;
  }
}

}  // namespace

hipError_t launch_attn_fp32(const AttnArgs &a, int head_dim, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.Hq * a.B * a.L * a.n_ranks;  // one workgroup per query row
  if (blocks == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_fp32_kernel<64>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fp32_kernel<128>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace usp
