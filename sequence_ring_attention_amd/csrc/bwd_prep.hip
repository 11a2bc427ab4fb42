// Per-row statistics of the attention backward.
//
// For every query row: delta = rowsum(dO * O), the row term of the softmax
// Jacobian (dS = P (dP - delta); rowsum(P * dP) equals rowsum(dO * O) because
// O = P V), and the forward's lse in base 2, lse * log2(e), with -inf turned
// into +inf so that exp2(s * scale * log2(e) - lse2) is 0 for every s of a
// row that saw no key.  The gradient kernels read both from one buffer:
// stats[i] = delta_i, stats[rows + i] = lse2_i.
//
// HBM-bound: each row reads D elements of O and of dO (16-byte vector loads,
// D / 8 lanes per bf16 row, D / 4 per fp32 row), and writes two floats.
// bf16 products are exact in fp32, and fp32 products exact in double, so the
// only roundings are those of the running sum.
#include <type_traits>

#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(PrepArgs p) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / VEC;         // lanes per row: 8 or 16 (bf16), 16 or 32 (fp32)
  constexpr int RPB = kThreads / LPR;  // rows per workgroup
  typedef typename std::conditional<kBf16, float, double>::type Acc;
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  Acc acc = 0;
  if (row < p.rows) {
    int64_t rest = row;
    const int i = (int)(rest % p.L);
    rest /= p.L;
    const int b = (int)(rest % p.B);
    rest /= p.B;
    const int h = (int)(rest % p.Hq);
    const int64_t rank = rest / p.Hq;
    const T *o = static_cast<const T *>(p.o) + rank * p.o_rank + b * p.o_sb + (int64_t)i * p.o_ss + h * p.o_sh;
    const T *d = static_cast<const T *>(p.dout) + rank * p.do_rank + b * p.do_sb + (int64_t)i * p.do_ss +
                 h * p.do_sh;
    typedef T vec_t __attribute__((ext_vector_type(VEC)));
    const vec_t ov = *reinterpret_cast<const vec_t *>(o + sub * VEC);
    const vec_t dv = *reinterpret_cast<const vec_t *>(d + sub * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += (Acc)ov[e] * (Acc)dv[e];
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (sub == 0 && row < p.rows) {
    p.stats[row] = (float)acc;
    const float lse = p.lse[row];
    p.stats[p.rows + row] = lse == -INFINITY ? INFINITY : (float)((double)lse * 1.4426950408889634074);
  }
}

template <typename T, int D>
hipError_t launch_prep_t(const PrepArgs &p, hipStream_t stream) {
  constexpr int RPB = kThreads / (D / (16 / (int)sizeof(T)));
  const int64_t blocks = (p.rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((uint32_t)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const PrepArgs &p, int head_dim, bool bf16, hipStream_t stream) {
  if (bf16) return head_dim == 128 ? launch_prep_t<__bf16, 128>(p, stream) : launch_prep_t<__bf16, 64>(p, stream);
  return head_dim == 128 ? launch_prep_t<float, 128>(p, stream) : launch_prep_t<float, 64>(p, stream);
}

}  // namespace usp
