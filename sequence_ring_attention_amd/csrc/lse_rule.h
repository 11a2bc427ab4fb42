// The LSE rule of two attention partials of one row, shared by the merge
// kernel, the split walk's finalize and the ring step's fused merge.
//
// "Context Parallel 与 Ulysses" (ml-interview blog), concepts section: two
// partials combine as lse = log(e^lse1 + e^lse2) and
// o = e^(lse1 - lse) o1 + e^(lse2 - lse) o2.  Evaluated in the shifted form
// lse = M + log1p(e^(m - M)) with M the larger and m the smaller input, in
// double precision, so the fp32 result is rounded once.  A partial with
// lse = -inf (no visible key) is the identity; two of them give (0, -inf).
#pragma once

#include <hip/hip_runtime.h>

namespace usp {

// The weights of the two partials and the merged lse of one row.
__device__ inline void merge_weights(double l1, double l2, double &a1, double &a2, double &lse) {
  const bool e1 = l1 == -INFINITY, e2 = l2 == -INFINITY;
  if (e1 && e2) {
    a1 = 0.0;
    a2 = 0.0;
    lse = -INFINITY;
  } else if (e2) {
    a1 = 1.0;
    a2 = 0.0;
    lse = l1;
  } else if (e1) {
    a1 = 0.0;
    a2 = 1.0;
    lse = l2;
  } else {
    const double M = l1 > l2 ? l1 : l2;
    const double w = exp((l1 > l2 ? l2 : l1) - M);  // in (0, 1]
    lse = M + log1p(w);
    const double big = 1.0 / (1.0 + w), small = w / (1.0 + w);
    a1 = l1 > l2 ? big : small;
    a2 = l1 > l2 ? small : big;
  }
}

__device__ inline float4 blend(double a1, float4 x, double a2, float4 y) {
  float4 r;
  r.x = (float)(a1 * (double)x.x + a2 * (double)y.x);
  r.y = (float)(a1 * (double)x.y + a2 * (double)y.y);
  r.z = (float)(a1 * (double)x.z + a2 * (double)y.z);
  r.w = (float)(a1 * (double)x.w + a2 * (double)y.w);
  return r;
}

__device__ inline float blend1(double a1, float x, double a2, float y) {
  return (float)(a1 * (double)x + a2 * (double)y);
}

}  // namespace usp
