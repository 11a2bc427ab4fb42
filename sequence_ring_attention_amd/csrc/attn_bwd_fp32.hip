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
//   * dQ: one wavefront per (rank, query head, batch, query row) walks the
//     steps' KV blocks, like the forward;
//   * dK, dV: one wavefront per (KV block, KV head, batch, key row) walks the
//     query rows of every rank that reaches the block, over the query heads
//     that read the KV head, and adds its sums into the fp32 accumulators.
// The 64 lanes split head_dim; dot products and sums are in double (fp32
// products are exact there), so the outputs see one final rounding.
#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;
constexpr double kLog2e = 1.4426950408889634074;

__device__ inline double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline int mod_cp(int x, int cp) {
  x %= cp;
  return x < 0 ? x + cp : x;
}

template <int D>
__global__ __launch_bounds__(kThreads) void dq_fp32_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t rows_per_rank = (int64_t)a.Hq * a.B * a.L;
  if (w >= rows_per_rank * a.n_ranks) return;  // whole wavefront exits together
  int64_t rest = w;
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
  for (int t = a.t_lo; t < a.t_hi; ++t) {
    const int j = mod_cp(rank - t, a.cp);
    const float *kb = static_cast<const float *>(a.k) + j * a.kv_blk + b * a.k_sb + kvh * a.k_sh;
    const float *vb = static_cast<const float *>(a.v) + j * a.kv_blk + b * a.v_sb + kvh * a.v_sh;
    for (int kk = 0; kk < a.L; ++kk) {
      const int kpos = sm.pos(j, kk);
      if (a.causal && kpos > qpos) continue;
      if (kpos < sst) continue;  // another packed sample (sst = 0 for one sequence)
      double s = 0.0, g = 0.0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        s += qv[e] * (double)kb[(int64_t)kk * a.k_ss + lane + 64 * e];
        g += dov[e] * (double)vb[(int64_t)kk * a.v_ss + lane + 64 * e];
      }
      s = wave_sum(s);
      g = wave_sum(g);
      const double p = exp2(s * sl2 - lse2);  // lse2 = +inf for a row with no key: p = 0
      const double ds = p * (g - delta);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += ds * (double)kb[(int64_t)kk * a.k_ss + lane + 64 * e];
    }
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
  const int lane = threadIdx.x & 63;
  const int64_t w = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int n_slots = a.ring_rank >= 0 ? a.t_hi - a.t_lo : a.cp;
  if (w >= (int64_t)n_slots * a.Hkv * a.B * a.L) return;  // whole wavefront exits together
  int64_t rest = w;
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
  for (int r = r_first; r <= r_last; ++r) {
    const int rs = a.ring_rank >= 0 ? 0 : r;
    for (int hq = g * a.G; hq < (g + 1) * a.G; ++hq) {
      const float *qb = static_cast<const float *>(a.q) + (a.ring_rank < 0 ? r * a.q_rank : 0) + b * a.q_sb +
                        hq * a.q_sh;
      const float *db = static_cast<const float *>(a.dout) + (a.ring_rank < 0 ? r * a.do_rank : 0) +
                        b * a.do_sb + hq * a.do_sh;
      const int64_t srow0 = (((int64_t)rs * a.Hq + hq) * a.B + b) * a.L;
      for (int i = 0; i < a.L; ++i) {
        const int qpos = sm.pos(r, i);
        if (a.causal && qpos < kpos) continue;
        if (qpos >= kend) continue;  // another packed sample
        double s = 0.0, gd = 0.0;
        double qe[PER], de[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          qe[e] = (double)qb[(int64_t)i * a.q_ss + lane + 64 * e];
          de[e] = (double)db[(int64_t)i * a.do_ss + lane + 64 * e];
          s += qe[e] * kv[e];
          gd += de[e] * vv[e];
        }
        s = wave_sum(s);
        gd = wave_sum(gd);
        const double p = exp2(s * sl2 - (double)a.stats[a.rows + srow0 + i]);
        const double ds = p * (gd - (double)a.stats[srow0 + i]);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          dv[e] += p * de[e];
          dk[e] += ds * qe[e];
        }
      }
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
  const int64_t q_waves = (int64_t)a.Hq * a.B * a.L * a.n_ranks;
  if (q_waves > 0)
    hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3((uint32_t)((q_waves + 3) / 4)), dim3(kThreads), 0, stream, a);
  const int n_slots = a.ring_rank >= 0 ? a.t_hi - a.t_lo : a.cp;
  const int64_t k_waves = (int64_t)n_slots * a.Hkv * a.B * a.L;
  if (k_waves > 0)
    hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3((uint32_t)((k_waves + 3) / 4)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_fp32(const BwdArgs &a, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace usp
