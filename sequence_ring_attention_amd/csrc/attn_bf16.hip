// Ring-step / ring-walk causal attention, bf16 inputs, MFMA on gfx950.
//
// What is computed ("Context Parallel 与 Ulysses", ml-interview blog):
// ring rank r keeps its queries; at step t it holds KV block j = (r - t) mod
// cp (concepts section, Figure 1) and computes softmax attention of its
// queries against that block, giving (o_j, lse_j); the steps are merged with
// the LSE rule of the same section.  Here the walk over the cp blocks runs
// inside one kernel and the merge is its online form: a running row max m,
// row sum l and unnormalised output O are rescaled whenever m grows, which
// equals merging the per-block (o_j, lse_j) one after another.  The causal
// mask is block-granular (Figure 2: cells above the diagonal are skipped,
// diagonal cells are half computed): key tiles wholly above a query tile are
// never visited, tiles wholly below it run unmasked, and only tiles that
// straddle the diagonal evaluate the elementwise mask.
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows of one
// query head, one batch, one rank):
//   * each wavefront owns 32 query rows;
//   * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16, K tile rows
//     (keys) as the M operand from LDS and the wave's Q rows (N operand) kept
//     in registers, fp32 accumulation.  With S^T, one lane holds one query
//     and 16 of its keys per 32-key block, so the row max needs a single
//     exchange with the partner lane (lane ^ 32), and the rescale of O is a
//     per-lane scalar;
//   * O^T += V^T P^T with V^T from LDS (transposed while staging) and P (the
//     probabilities rounded to bf16) straight from the S^T registers as the
//     N operand: the K-row order of the first product is permuted so that
//     each lane's eight bf16 probabilities are eight consecutive keys.
//   * K and V tiles of 64 keys are staged global -> registers -> LDS; the
//     next tile's global loads are issued before the current tile's math.
//
// Grid order: heaviest query tiles first (the last rows of a share see the
// most keys), and the Hq / Hkv query heads that read one KV head run back to
// back on one XCD (workgroups are dealt to the 8 XCDs round-robin) so that
// their K/V tiles are shared through that XCD's L2.
#include "usp_internal.h"

namespace usp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NT = 256;  // threads per workgroup

template <int D>
struct Lds {
  static constexpr int K_ROW = D * 2 + 16;   // bytes per key row, padded against bank conflicts
  static constexpr int V_ROW = BN * 2 + 16;  // bytes per head-dim row of V^T, padded
  static constexpr int K_BYTES = BN * K_ROW;
  static constexpr int V_BYTES = D * V_ROW;
  static constexpr int BYTES = K_BYTES + V_BYTES;
};

// Global position of local index i of ring rank `rank`'s share.
__device__ inline int share_pos(int rank, int i, int c, int cp) {
  return i < c ? rank * c + i : (2 * cp - 1 - rank) * c + (i - c);
}

// Number of local indices of block j whose position is <= p (positions of a
// share increase with the local index, so this is a prefix length).
__device__ inline int count_le(int j, int p, int c, int cp) {
  const int a = min(max(p - j * c + 1, 0), c);
  const int b = min(max(p - (2 * cp - 1 - j) * c + 1, 0), c);
  return a + b;
}

__device__ inline int seg_start(const int32_t *cu, int nseq, int pos) {
  int lo = 0, hi = nseq;  // cu[lo] <= pos < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= pos) lo = mid; else hi = mid;
  }
  return cu[lo];
}

__device__ inline uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ inline uint32_t hi16(uint32_t w) { return w >> 16; }

// The key range of block j one query tile can see, in 64-key tiles.
struct StepRange {
  int j, kt, ke;
};

template <int D, bool PARTIAL>
__global__ __launch_bounds__(NT, 2) void attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[Lds<D>::BYTES];
  char *const sK = smem;
  char *const sV = smem + Lds<D>::K_BYTES;

  // ---------------------------------------------------------- work item --
  const int bid = blockIdx.x;
  int gi, g;
  if (a.xcd_remap) {
    const int x = bid & 7, i = bid >> 3;
    gi = (i / a.G) * 8 + x;
    g = i % a.G;
  } else {
    gi = bid / a.G;
    g = bid % a.G;
  }
  const int kvh = gi % a.Hkv;
  int rest = gi / a.Hkv;
  const int b = rest % a.B;
  const int order = rest / a.B;
  int rank, lt;
  if (a.ring_rank >= 0) {
    rank = a.ring_rank;
    lt = a.n_qtiles - 1 - order;
  } else {
    rank = order % a.cp;
    lt = a.n_qtiles - 1 - order / a.cp;
  }
  const int hq = kvh * a.G + g;
  const int c = a.c, cp = a.cp, L = a.L;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int q0 = lt * BM;
  const int qrow = q0 + wave * 32 + n;
  const bool qvalid = qrow < L;
  const int qlast = min(q0 + BM, L) - 1;
  const int qpos_min = share_pos(rank, q0, c, cp);
  const int qpos_max = share_pos(rank, qlast, c, cp);
  const int my_qpos = qvalid ? share_pos(rank, qrow, c, cp) : -1;
  int sst_min = 0, sst_max = 0, my_sst = 0;
  if (a.cu) {
    sst_min = seg_start(a.cu, a.nseq, qpos_min);
    sst_max = seg_start(a.cu, a.nseq, qpos_max);
    my_sst = qvalid ? seg_start(a.cu, a.nseq, my_qpos) : 0x7fffffff;
  }

  // ------------------------------------------------------- Q fragments --
  const __bf16 *qbase = static_cast<const __bf16 *>(a.q) + (a.ring_rank < 0 ? rank * a.q_rank : 0) +
                        b * a.q_sb + hq * a.q_sh;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (qvalid)
      qf[ks] = *reinterpret_cast<const bf16x8 *>(qbase + (int64_t)qrow * a.q_ss + 16 * ks + 8 * hh);
    else
      qf[ks] = bf16x8{};
  }

  // ------------------------------------------------------ tile schedule --
  auto step_range = [&](int t) {
    StepRange r;
    r.j = (rank - t) % cp;
    if (r.j < 0) r.j += cp;
    const int hi = a.causal ? count_le(r.j, qpos_max, c, cp) : L;
    const int lo = a.cu ? count_le(r.j, sst_min - 1, c, cp) : 0;
    if (hi <= lo) {
      r.kt = r.ke = 0;
    } else {
      r.kt = lo / BN;
      r.ke = (hi + BN - 1) / BN;
    }
    return r;
  };
  int t = a.t_lo;
  StepRange cur = step_range(t);
  while (cur.kt >= cur.ke && ++t < a.t_hi) cur = step_range(t);

  // ------------------------------------------------------- staging regs --
  constexpr int KCH = D / 8;                  // 16-byte chunks per key row
  constexpr int KROWS = NT / KCH;             // key rows per pass
  constexpr int KPASS = BN / KROWS;           // passes per tile
  constexpr int VITEMS = (BN / 4) * KCH;      // (4 keys x 8 dims) items of V
  uint4 kreg[KPASS];
  uint4 vreg[4];

  auto load_tile = [&](int j, int k0) {
    const __bf16 *kb = static_cast<const __bf16 *>(a.k) + j * a.kv_blk + b * a.k_sb + kvh * a.k_sh;
    const __bf16 *vb = static_cast<const __bf16 *>(a.v) + j * a.kv_blk + b * a.v_sb + kvh * a.v_sh;
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int key = k0 + p * KROWS + tid / KCH;
      kreg[p] = key < L ? *reinterpret_cast<const uint4 *>(kb + (int64_t)key * a.k_ss + (tid % KCH) * 8)
                        : uint4{0, 0, 0, 0};
    }
    if (tid < VITEMS) {
      const int kg = tid % (BN / 4), ch = tid / (BN / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 4 * kg + i;
        vreg[i] = key < L ? *reinterpret_cast<const uint4 *>(vb + (int64_t)key * a.v_ss + ch * 8)
                          : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int key = p * KROWS + tid / KCH;
      *reinterpret_cast<uint4 *>(sK + key * Lds<D>::K_ROW + (tid % KCH) * 16) = kreg[p];
    }
    if (tid < VITEMS) {
      const int kg = tid % (BN / 4), ch = tid / (BN / 4);
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // dims 2m (low halves) and 2m+1 (high halves) of keys 4kg .. 4kg+3
        uint2 even, odd;
        even.x = lo16(w0[m]) | (lo16(w1[m]) << 16);
        even.y = lo16(w2[m]) | (lo16(w3[m]) << 16);
        odd.x = hi16(w0[m]) | (hi16(w1[m]) << 16);
        odd.y = hi16(w2[m]) | (hi16(w3[m]) << 16);
        *reinterpret_cast<uint2 *>(sV + (ch * 8 + 2 * m) * Lds<D>::V_ROW + kg * 8) = even;
        *reinterpret_cast<uint2 *>(sV + (ch * 8 + 2 * m + 1) * Lds<D>::V_ROW + kg * 8) = odd;
      }
    }
  };

  // --------------------------------------------------------- main loop --
  f32x16 O[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) O[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = a.scale_log2;
  // M-row -> key permutation of the K operand (swap bits 2 and 3), so that
  // accumulator register r of lane half hh holds key 16*(r/8) + 8*hh + r%8.
  const int sig = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

  if (t < a.t_hi) load_tile(cur.j, cur.kt * BN);
  while (t < a.t_hi) {
    // the next tile of the walk (wave-uniform)
    int nt = t;
    StepRange nxt = cur;
    ++nxt.kt;
    while (nxt.kt >= nxt.ke && ++nt < a.t_hi) nxt = step_range(nt);

    store_tile();
    __syncthreads();
    if (nt < a.t_hi) load_tile(nxt.j, nxt.kt * BN);

    const int j = cur.j;
    const int k0 = cur.kt * BN;
    // tile class: every (query, key) pair of the workgroup visible?
    const int klast = min(k0 + BN, L) - 1;
    const int kpos_min = share_pos(j, k0, c, cp);
    const int kpos_max = share_pos(j, klast, c, cp);
    bool full = (k0 + BN <= L);
    if (a.causal) full = full && kpos_max <= qpos_min;
    if (a.cu) full = full && kpos_min >= sst_max;

    // S^T = K Q^T for two 32-key blocks
    f32x16 S0 = f32x16{}, S1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(sK + sig * Lds<D>::K_ROW + (16 * ks + 8 * hh) * 2);
      const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(sK + (32 + sig) * Lds<D>::K_ROW + (16 * ks + 8 * hh) * 2);
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[ks], S1, 0, 0, 0);
    }

    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 16 * (r / 8) + 8 * hh + (r % 8);
        const int kk0 = k0 + kl, kk1 = k0 + 32 + kl;
        const int p0 = share_pos(j, kk0, c, cp), p1 = share_pos(j, kk1, c, cp);
        bool v0 = kk0 < L, v1 = kk1 < L;
        if (a.causal) {
          v0 = v0 && p0 <= my_qpos;
          v1 = v1 && p1 <= my_qpos;
        }
        if (a.cu) {
          v0 = v0 && p0 >= my_sst;
          v1 = v1 && p1 >= my_sst;
        }
        if (!v0) S0[r] = -INFINITY;
        if (!v1) S1[r] = -INFINITY;
      }
    }

    // online softmax (base 2, scale folded in)
    float mx = S0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S1[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
    bf16x8 pf[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S0[r], sl2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S1[r], sl2, -m_use));
      psum += p0 + p1;
      pf[r / 8][r % 8] = (__bf16)p0;
      pf[2 + r / 8][r % 8] = (__bf16)p1;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) O[mb] *= alpha;

    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(sV + (32 * mb + n) * Lds<D>::V_ROW + (16 * p + 8 * hh) * 2);
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[p], O[mb], 0, 0, 0);
      }
    }
    __syncthreads();
    t = nt;
    cur = nxt;
  }

  // ---------------------------------------------------------- epilogue --
  const float l = l_run + __shfl_xor(l_run, 32);
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l;
  const float lse = empty ? -INFINITY : (m_run + __log2f(l)) * 0.69314718055994530942f;
  if (!qvalid) return;
  if (PARTIAL) {
    float *o = static_cast<float *>(a.o) + (((int64_t)hq * a.B + b) * L + qrow) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 val;
        val.x = O[mb][4 * r4 + 0] * inv;
        val.y = O[mb][4 * r4 + 1] * inv;
        val.z = O[mb][4 * r4 + 2] * inv;
        val.w = O[mb][4 * r4 + 3] * inv;
        *reinterpret_cast<float4 *>(o + 32 * mb + 8 * r4 + 4 * hh) = val;
      }
    }
  } else {
    __bf16 *o = static_cast<__bf16 *>(a.o) + (a.ring_rank < 0 ? rank * a.o_rank : 0) + b * a.o_sb +
                (int64_t)qrow * a.o_ss + hq * a.o_sh;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 val;
        val[0] = (__bf16)(O[mb][4 * r4 + 0] * inv);
        val[1] = (__bf16)(O[mb][4 * r4 + 1] * inv);
        val[2] = (__bf16)(O[mb][4 * r4 + 2] * inv);
        val[3] = (__bf16)(O[mb][4 * r4 + 3] * inv);
        *reinterpret_cast<bf16x4 *>(o + 32 * mb + 8 * r4 + 4 * hh) = val;
      }
    }
  }
  if (hh == 0) {
    const int64_t li = (((a.ring_rank < 0 ? (int64_t)rank * a.Hq : 0) + hq) * a.B + b) * L + qrow;
    a.lse[li] = lse;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.n_ranks * a.n_qtiles * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((uint32_t)blocks), block(NT);
  if (head_dim == 128) {
    if (a.partial)
      hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (a.partial)
      hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace usp
