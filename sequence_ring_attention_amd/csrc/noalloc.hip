// usp_attn_bwd_noalloc: the ring backward with its per-row statistics in a
// library-owned device array instead of a caller buffer, for callers that
// cannot allocate device memory.  The array is a file-scope __device__
// symbol; each device's copy is found once with hipGetSymbolAddress, with
// that device current, and only that address is handed to the kernels.
#include <mutex>

#include "usp_internal.h"

namespace {

constexpr int64_t kMaxRows = USP_NOALLOC_MAX_STATS_ROWS;

// [delta (rows) | lse * log2(e) (rows)] of the current call, 16 MiB.
__device__ __align__(256) float scratch[2 * kMaxRows];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_scratch[kMaxDevices];  // device address of `scratch` per device, once resolved

// The address of the current device's array.
usp_status scratch_address(float **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return usp::report(USP_ERR_HIP, "attn_bwd_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return usp::report(USP_ERR_UNSUPPORTED, "attn_bwd_noalloc: device index >= 64");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return usp::report(USP_ERR_HIP, "attn_bwd_noalloc: hipGetSymbolAddress of the statistics array failed");
    g_scratch[dev] = static_cast<float *>(p);
  }
  *out = g_scratch[dev];
  return USP_OK;
}

}  // namespace

extern "C" usp_status usp_attn_bwd_noalloc(const void *q, const void *k_all, const void *v_all, const void *o,
                                           const void *d_o, const float *lse, void *dq, float *dk_all,
                                           float *dv_all, const usp_attn_desc *desc, int32_t ring_rank,
                                           void *stream) {
  if (!desc) return usp::report(USP_ERR_INVALID_ARG, "attn_bwd_noalloc: null descriptor");
  // the size limit first, before anything touches the GPU; other descriptor
  // errors are reported by the shared checks below
  if (desc->batch >= 1 && desc->num_q_heads >= 1 && desc->cp >= 1 && desc->seq_len >= 1 && ring_rank >= -1 &&
      usp::bwd_stats_rows(desc, ring_rank) > kMaxRows)
    return usp::report(USP_ERR_INVALID_ARG,
                       "attn_bwd_noalloc: the call needs more statistics rows than the 2^21 of the library's array");
  float *stats = nullptr;
  const usp_status s = scratch_address(&stats);
  if (s != USP_OK) return s;
  return usp::attn_bwd_with_stats(q, k_all, v_all, o, d_o, lse, dq, dk_all, dv_all, stats, desc, ring_rank, stream,
                                  "attn_bwd_noalloc");
}
