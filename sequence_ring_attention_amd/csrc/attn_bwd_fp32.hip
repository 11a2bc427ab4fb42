// Ring-step / ring-walk attention backward for fp32 inputs (small problems).
//
// The gradients are the derivative of the forward: with the forward's final
// lse, P = exp(scale q k^T - lse) on the visible pairs of each KV block ("Context
// Parallel 与 Ulysses", concepts section: the step results of one row share
// that row's softmax over all blocks), dP = dO V^T, dS = P (dP - delta),
// dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, with delta = rowsum(dO O)
// and lse2 = lse log2(e) taken from the statistics buffer.
//
// Two passes, each owning its outputs so that no two lanes write one value:
//   * dQ: one workgroup per (rank, query head, batch, query row) walks the
//     steps' KV blocks, like the forward;
//   * dK, dV: one workgroup per (KV block, KV head, batch, key row) walks the
//     query rows of every rank that reaches the block, over the query heads
//     that read the KV head, and adds its sums into the fp32 accumulators.
// Each wavefront is one of four that share the row, taking its groups of 16
// keys (queries) in turn; a group's dot products are summed across the
// wavefront in one pass of independent shuffles, and the four wavefronts'
// sums are added in a fixed order at the end.  The 64 lanes split head_dim;
// dot products and sums are in double (fp32 products are exact there), so
// the outputs see one final rounding.
#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;
constexpr int NWV = kThreads / 64;  // wavefronts sharing one row
constexpr int KB = 16;              // keys (queries) per group
constexpr double kLog2e = 1.4426950408889634074;

// Sums x[0 .. N) across the wavefront, every lane getting every sum: one
// pass of N independent shuffles per step.
template <int N>
__device__ inline void wave_sums(double *x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], off);
  }
}

// Lane i's value of x, in every lane.
__device__ inline double read_lane(double x, int i) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, i);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), i);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// x[i] for i = lane (lanes 0 .. N - 1), by selects (no dynamic indexing).
template <int N>
__device__ inline double pick_lane(const double *x, int lane) {
  double r = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = lane == i ? x[i] : r;
  return r;
}

__device__ inline int mod_cp(int x, int cp) {
  x %= cp;
  return x < 0 ? x + cp : x;
}

template <int D>
__global__ __launch_bounds__(kThreads) void dq_fp32_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  __shared__ double part[NWV][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int64_t rest = blockIdx.x;
  const int qrow = (int)(rest % a.L);
  rest /= a.L;
  const int b = (int)(rest % a.B);
  rest /= a.B;
  const int hq = (int)(rest % a.Hq);
  const int rank = a.ring_rank >= 0 ? a.ring_rank : (int)(rest / a.Hq);
  const int rs = a.ring_rank >= 0 ? 0 : rank;
  const int kvh = hq / a.G;
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  const int qpos = sm.pos(rank, qrow);
  const int sst = sm.packed() ? sm.seg_start(qpos) : 0;
  const int64_t srow = (((int64_t)rs * a.Hq + hq) * a.B + b) * a.L + qrow;
  const double delta = (double)a.stats[srow];
  const double lse2 = (double)a.stats[a.rows + srow];

  const float *qp = static_cast<const float *>(a.q) + (a.ring_rank < 0 ? rank * a.q_rank : 0) + b * a.q_sb +
                    (int64_t)qrow * a.q_ss + hq * a.q_sh;
  const float *dp = static_cast<const float *>(a.dout) + (a.ring_rank < 0 ? rank * a.do_rank : 0) +
                    b * a.do_sb + (int64_t)qrow * a.do_ss + hq * a.do_sh;
  double qv[PER], dov[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qv[e] = (double)qp[lane + 64 * e];
    dov[e] = (double)dp[lane + 64 * e];
    acc[e] = 0.0;
  }
  const double sl2 = (double)a.scale * kLog2e;
  int grp = 0;  // key groups of the row's walk so far
  for (int t = a.t_lo; t < a.t_hi; ++t) {
    const int j = mod_cp(rank - t, a.cp);
    const float *kb = static_cast<const float *>(a.k) + j * a.kv_blk + b * a.k_sb + kvh * a.k_sh;
    const float *vb = static_cast<const float *>(a.v) + j * a.kv_blk + b * a.v_sb + kvh * a.v_sh;
    // positions grow with the local row: the keys this row sees are the
    // local rows [lo, hi) of block j (sst = 0 for one sequence)
    const int hi = __builtin_amdgcn_readfirstlane(a.causal ? sm.count_le(j, qpos) : a.L);
    const int lo = __builtin_amdgcn_readfirstlane(sst > 0 ? sm.count_le(j, sst - 1) : 0);
    for (int k0 = lo; k0 < hi; k0 += KB, ++grp) {
      if (grp % NWV != wv) continue;
      const int n = hi - k0 < KB ? hi - k0 : KB;
      double sg[2 * KB];  // logits, then dO . V
      float kk[KB][PER];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        sg[i] = 0.0;
        sg[KB + i] = 0.0;
#pragma unroll
        for (int e = 0; e < PER; ++e) kk[i][e] = 0.0f;
        if (i < n) {
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            kk[i][e] = kb[(int64_t)(k0 + i) * a.k_ss + lane + 64 * e];
            sg[i] += qv[e] * (double)kk[i][e];
            sg[KB + i] += dov[e] * (double)vb[(int64_t)(k0 + i) * a.v_ss + lane + 64 * e];
          }
        }
      }
      wave_sums<2 * KB>(sg);
      // lane i < n evaluates key k0 + i's dS
      const double si = pick_lane<KB>(sg, lane), gi = pick_lane<KB>(sg + KB, lane);
      const double dsl = lane < n ? exp2(si * sl2 - lse2) * (gi - delta) : 0.0;  // lse2 = +inf: p = 0
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (i < n) {
          const double ds = read_lane(dsl, i);
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += ds * (double)kk[i][e];
        }
      }
    }
  }
  // the four wavefronts' sums, added in a fixed order by wavefront 0
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wv][lane + 64 * e] = acc[e];
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    acc[e] = part[0][lane + 64 * e];
#pragma unroll
    for (int i = 1; i < NWV; ++i) acc[e] += part[i][lane + 64 * e];
  }
  const double scale = (double)a.scale;
  if (a.dq_acc) {
    float *o = static_cast<float *>(a.dq) + (((int64_t)hq * a.B + b) * a.L + qrow) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (float)((double)o[lane + 64 * e] + acc[e] * scale);
  } else {
    float *o = static_cast<float *>(a.dq) + (a.ring_rank < 0 ? rank * a.q_rank : 0) + b * a.q_sb +
               (int64_t)qrow * a.q_ss + hq * a.q_sh;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (float)(acc[e] * scale);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void dkdv_fp32_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  __shared__ double part[NWV][2][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int64_t rest = blockIdx.x;
  const int krow = (int)(rest % a.L);
  rest /= a.L;
  const int b = (int)(rest % a.B);
  rest /= a.B;
  const int g = (int)(rest % a.Hkv);
  const int slot = (int)(rest / a.Hkv);
  // block j and the ranks whose queries reach it in this launch
  const int j = a.ring_rank >= 0 ? mod_cp(a.ring_rank - (a.t_lo + slot), a.cp) : slot;
  const int r_first = a.ring_rank >= 0 ? a.ring_rank : 0;
  const int r_last = a.ring_rank >= 0 ? a.ring_rank : a.cp - 1;
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  const int kpos = sm.pos(j, krow);
  const int kend = sm.packed() ? sm.seg_end(kpos) : 0x7fffffff;

  const int64_t kvo = j * a.kv_blk;
  const float *kp = static_cast<const float *>(a.k) + kvo + b * a.k_sb + (int64_t)krow * a.k_ss + g * a.k_sh;
  const float *vp = static_cast<const float *>(a.v) + kvo + b * a.v_sb + (int64_t)krow * a.v_ss + g * a.v_sh;
  double kv[PER], vv[PER], dk[PER], dv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kv[e] = (double)kp[lane + 64 * e];
    vv[e] = (double)vp[lane + 64 * e];
    dk[e] = 0.0;
    dv[e] = 0.0;
  }
  const double sl2 = (double)a.scale * kLog2e;
  int grp = 0;  // query groups so far
  for (int r = r_first; r <= r_last; ++r) {
    const int rs = a.ring_rank >= 0 ? 0 : r;
    // the query rows of rank r that see this key: [lo, hi) (causal: at or
    // after the key; packed: before the end of its sample)
    const int lo = __builtin_amdgcn_readfirstlane(a.causal ? sm.count_le(r, kpos - 1) : 0);
    const int hi = __builtin_amdgcn_readfirstlane(sm.packed() ? sm.count_le(r, kend - 1) : a.L);
    for (int hq = g * a.G; hq < (g + 1) * a.G; ++hq) {
      const float *qb = static_cast<const float *>(a.q) + (a.ring_rank < 0 ? r * a.q_rank : 0) + b * a.q_sb +
                        hq * a.q_sh;
      const float *db = static_cast<const float *>(a.dout) + (a.ring_rank < 0 ? r * a.do_rank : 0) +
                        b * a.do_sb + hq * a.do_sh;
      const int64_t srow0 = (((int64_t)rs * a.Hq + hq) * a.B + b) * a.L;
      for (int i0 = lo; i0 < hi; i0 += KB, ++grp) {
        if (grp % NWV != wv) continue;
        const int n = hi - i0 < KB ? hi - i0 : KB;
        double sg[2 * KB];  // logits, then dO . V
        float qe[KB][PER], de[KB][PER];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          sg[i] = 0.0;
          sg[KB + i] = 0.0;
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            qe[i][e] = 0.0f;
            de[i][e] = 0.0f;
          }
          if (i < n) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
              qe[i][e] = qb[(int64_t)(i0 + i) * a.q_ss + lane + 64 * e];
              de[i][e] = db[(int64_t)(i0 + i) * a.do_ss + lane + 64 * e];
              sg[i] += (double)qe[i][e] * kv[e];
              sg[KB + i] += (double)de[i][e] * vv[e];
            }
          }
        }
        wave_sums<2 * KB>(sg);
        // lane i < n evaluates query i0 + i's P and dS
        const double si = pick_lane<KB>(sg, lane), gi = pick_lane<KB>(sg + KB, lane);
        double pl = 0.0, dsl = 0.0;
        if (lane < n) {
          pl = exp2(si * sl2 - (double)a.stats[a.rows + srow0 + i0 + lane]);
          dsl = pl * (gi - (double)a.stats[srow0 + i0 + lane]);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          if (i < n) {
            const double p = read_lane(pl, i), ds = read_lane(dsl, i);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
              dv[e] += p * (double)de[i][e];
              dk[e] += ds * (double)qe[i][e];
            }
          }
        }
      }
    }
  }
  // the four wavefronts' sums, added in a fixed order by wavefront 0
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    part[wv][0][lane + 64 * e] = dk[e];
    part[wv][1][lane + 64 * e] = dv[e];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    dk[e] = part[0][0][lane + 64 * e];
    dv[e] = part[0][1][lane + 64 * e];
#pragma unroll
    for (int i = 1; i < NWV; ++i) {
      dk[e] += part[i][0][lane + 64 * e];
      dv[e] += part[i][1][lane + 64 * e];
    }
  }
  float *dkp = a.dk + kvo + b * a.k_sb + (int64_t)krow * a.k_ss + g * a.k_sh;
  float *dvp = a.dv + kvo + b * a.v_sb + (int64_t)krow * a.v_ss + g * a.v_sh;
  const double scale = (double)a.scale;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    dkp[lane + 64 * e] = (float)((double)dkp[lane + 64 * e] + dk[e] * scale);
    dvp[lane + 64 * e] = (float)((double)dvp[lane + 64 * e] + dv[e]);
  }
}

template <int D>
hipError_t launch_d(const BwdArgs &a, hipStream_t stream) {
  const int64_t q_rows = (int64_t)a.Hq * a.B * a.L * a.n_ranks;  // one workgroup each
  if (q_rows > 0) hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3((uint32_t)q_rows), dim3(kThreads), 0, stream, a);
  const int n_slots = a.ring_rank >= 0 ? a.t_hi - a.t_lo : a.cp;
  const int64_t k_rows = (int64_t)n_slots * a.Hkv * a.B * a.L;  // one workgroup each
  if (k_rows > 0) hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3((uint32_t)k_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_fp32(const BwdArgs &a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace usp
