// LSE merge of a step's partial result into an accumulator, in place, by the
// rule of lse_rule.h ("Context Parallel 与 Ulysses", concepts section).
//
// All lanes that touch one row live in the same wavefront, so every lane has
// read lse_acc[row] before the row's writer lane stores the new value.
#include "lse_rule.h"
#include "usp_internal.h"

namespace usp {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // vector loads per lane in flight (64-row path): 4 measured faster than 8

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ inline float4 as_float4(f32x4 v) { return make_float4(v.x, v.y, v.z, v.w); }
__device__ inline f32x4 as_f32x4(float4 v) { return f32x4{v.x, v.y, v.z, v.w}; }

// Rows of 2^d4_shift float4 (at most 64): a workgroup of four wavefronts
// takes 64 rows.  Every wavefront computes the weights of the 64 rows (lane i
// those of row i) and streams its quarter of the rows' vectors (64
// consecutive per load, kUnroll loads in flight), taking each vector's row
// weights from the lane that computed them.  All four waves read the rows'
// lse before the barrier; after it, wave 0 writes the merged lse.  Four waves
// per 64 rows keep four times as many loads in flight as one wave would at
// sizes that give each CU only a few 64-row groups, and each wave requests
// its first vectors before the weights' double-precision exp and log1p.
// Measured with the cache flushed, against one wave per 64 rows: 5.29
// against 4.87 TB/s for 131072 rows of 128 (one step of a 4096-token GQA
// share), 6.01 against 5.63 TB/s for 524288 rows; 128- and 512-thread
// workgroups were slower.
__global__ __launch_bounds__(kThreads) void lse_merge_rows64_kernel(float *o_acc, float *lse_acc,
                                                                    const float *o_step, const float *lse_step,
                                                                    int64_t rows, int32_t d4_shift) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int d4 = 1 << d4_shift;
  constexpr int kWaves = kThreads / 64;
  const int per_wave = d4 * 64 / kWaves;  // vectors of one wave: its share of 64 rows x d4
  for (int64_t row0 = (int64_t)blockIdx.x * 64; row0 < rows; row0 += (int64_t)gridDim.x * 64) {
    const int64_t my_row = row0 + lane;
    const bool live = my_row < rows;
    float4 *acc = reinterpret_cast<float4 *>(o_acc) + row0 * d4;
    const float4 *stp = reinterpret_cast<const float4 *>(o_step) + row0 * d4;
    const int64_t nvec = (rows - row0 < 64 ? rows - row0 : 64) * d4;  // vectors of the rows in range
    const int v0 = wave * per_wave;
    // the first kUnroll vectors of both partials are requested before the
    // weights are computed, so their latency overlaps the double-precision
    // exp and log1p
    float4 x[kUnroll], y[kUnroll];
    auto load = [&](int it0) {
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int v = v0 + it0 + k * 64 + lane;
        if (it0 + k * 64 + lane < per_wave && v < nvec) {
          x[k] = as_float4(__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(acc + v)));
          y[k] = as_float4(__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(stp + v)));
        }
      }
    };
    load(0);
    double a1 = 0.0, a2 = 0.0, lse = -INFINITY;
    merge_weights(live ? (double)lse_acc[my_row] : -INFINITY, live ? (double)lse_step[my_row] : -INFINITY, a1,
                  a2, lse);
    for (int it0 = 0; it0 < per_wave; it0 += kUnroll * 64) {
      if (it0 > 0) load(it0);
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int v = v0 + it0 + k * 64 + lane;
        const int src = (v >> d4_shift) & 63;  // the vector's row within the 64
        const double b1 = __shfl(a1, src), b2 = __shfl(a2, src);
        if (it0 + k * 64 + lane < per_wave && v < nvec)
          __builtin_nontemporal_store(as_f32x4(blend(b1, x[k], b2, y[k])), reinterpret_cast<f32x4 *>(acc + v));
      }
    }
    __syncthreads();  // every wave has read lse_acc of these rows
    if (wave == 0 && live) lse_acc[my_row] = (float)lse;
  }
}

__global__ __launch_bounds__(kThreads) void lse_merge_kernel(float *o_acc, float *lse_acc,
                                                             const float *o_step,
                                                             const float *lse_step, int64_t rows,
                                                             int32_t d4, int32_t rows_per_wave,
                                                             int32_t lanes_per_row) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int sub = lane / lanes_per_row;  // row within the wave's group
  const int col0 = lane - sub * lanes_per_row;
  const bool active_lane = sub < rows_per_wave;
  for (int64_t group = wave; group * rows_per_wave < rows; group += nwaves) {
    const int64_t row = group * rows_per_wave + sub;
    const bool live = active_lane && row < rows;
    double l1 = -INFINITY, l2 = -INFINITY;
    if (live) {
      l1 = (double)lse_acc[row];
      l2 = (double)lse_step[row];
    }
    double a1, a2, lse;
    merge_weights(l1, l2, a1, a2, lse);
    if (live) {
      float4 *acc = reinterpret_cast<float4 *>(o_acc + row * (int64_t)d4 * 4);
      const float4 *stp = reinterpret_cast<const float4 *>(o_step + row * (int64_t)d4 * 4);
      for (int col = col0; col < d4; col += lanes_per_row) acc[col] = blend(a1, acc[col], a2, stp[col]);
    }
    // every lane of this row read lse_acc[row] above (same wavefront, program order)
    if (live && col0 == 0) lse_acc[row] = (float)lse;
  }
}

// The split walk's finalize: per row, slot 0's partial alone, or merged with
// slot 1's when the row's tile was split; rounded once to bf16 (nearest even)
// into the caller's layout, with the merged lse.  One thread per four
// elements of a row; every thread of a split row evaluates the row's weights.
__global__ __launch_bounds__(kThreads) void split_finalize_kernel(FinalizeArgs f) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid / f.d4;
  const int c4 = (int)(gid - row * f.d4);
  if (row >= f.rows) return;
  const int qrow = (int)(row % f.L);
  int64_t rest = row / f.L;
  const int b = (int)(rest % f.B);
  rest /= f.B;
  const int hq = (int)(rest % f.Hq);
  const int rank = (int)(rest / f.Hq);
  const int tile = rank * f.n_qtiles + qrow / f.bm;
  const bool split = (f.mask[tile >> 5] >> (tile & 31)) & 1u;
  const float4 x = reinterpret_cast<const float4 *>(f.po)[row * f.d4 + c4];
  float4 r = x;
  float lse = f.pl[row];
  if (split) {
    const float4 y = reinterpret_cast<const float4 *>(f.po + f.slot_o)[row * f.d4 + c4];
    double a1, a2, l;
    merge_weights((double)lse, (double)f.pl[f.slot_lse + row], a1, a2, l);
    r = blend(a1, x, a2, y);
    lse = (float)l;
  }
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = (__bf16)r.x;
  v[1] = (__bf16)r.y;
  v[2] = (__bf16)r.z;
  v[3] = (__bf16)r.w;
  __bf16 *o = static_cast<__bf16 *>(f.o) + (f.ring_rank < 0 ? rank * f.o_rank : 0) + b * f.o_sb + qrow * f.o_ss +
              hq * f.o_sh + 4 * c4;
  *reinterpret_cast<bf16x4 *>(o) = v;
  if (c4 == 0) f.lse[row] = lse;
}

}  // namespace

hipError_t launch_split_finalize(const FinalizeArgs &f, hipStream_t stream) {
  const int64_t threads = f.rows * f.d4;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(split_finalize_kernel, dim3((uint32_t)((threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, f);
  return hipGetLastError();
}

hipError_t launch_lse_merge(float *o_acc, float *lse_acc, const float *o_step,
                            const float *lse_step, int64_t rows, int64_t head_dim,
                            hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int32_t d4 = (int32_t)(head_dim / 4);
  if (d4 <= 64 && (d4 & (d4 - 1)) == 0) {
    int32_t shift = 0;
    while ((1 << shift) < d4) ++shift;
    int64_t blocks = (rows + 63) / 64;  // one 64-row group per block (4 waves)
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(lse_merge_rows64_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, o_acc, lse_acc,
                       o_step, lse_step, rows, shift);
    return hipGetLastError();
  }
  int32_t rows_per_wave = 1, lanes_per_row = 64;
  if (d4 <= 64 && 64 % d4 == 0) {
    rows_per_wave = 64 / d4;
    lanes_per_row = d4;
  }
  const int64_t groups = (rows + rows_per_wave - 1) / rows_per_wave;
  int64_t blocks = (groups + 3) / 4;  // 4 waves per block
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, o_acc,
                     lse_acc, o_step, lse_step, rows, d4, rows_per_wave, lanes_per_row);
  return hipGetLastError();
}

}  // namespace usp
