// Ring-step / ring-walk attention backward, bf16 inputs, MFMA on gfx950.
//
// What is computed: the derivative of the forward.  With the forward's final
// lse, P = exp(scale q k^T - lse) on the visible pairs of every KV block
// ("Context Parallel 与 Ulysses", concepts section: each step's partial of a
// row is that row's softmax over all blocks, restricted to one block), so
// each step's gradient contribution stands alone:
//   dP = dO V^T,  dS = P (dP - delta),  dQ += scale dS K,
//   dK += scale dS^T Q,  dV += P^T dO,
// with delta = rowsum(dO O) and lse2 = lse log2(e) read from the statistics
// buffer.  The causal mask is block-granular as in the forward (Figure 2):
// tiles above the diagonal are never visited and only tiles that straddle it
// evaluate the elementwise mask.
//
// Two passes, each the single owner of what it writes (no atomics, results
// independent of scheduling):
//   * dQ pass -- a workgroup of 4 wavefronts owns 128 query rows of one
//     (rank, query head, batch), walks the steps' 64-key tiles like the
//     forward and keeps dQ^T in registers.  S^T = K Q^T and dP^T = V dO^T
//     take K and V rows from LDS as the M operand (K-row order permuted so
//     that a lane's probabilities are eight consecutive keys), with the
//     wave's Q and dO rows in registers; dQ^T += K^T dS^T reads K transposed
//     from the same row-major LDS tile (ds_read_b64_tr_b16) and takes dS^T
//     straight from the registers.
//   * dK/dV pass -- a workgroup of 8 wavefronts owns 256 keys of one (KV
//     block, KV head, batch); each wavefront holds its 32 keys' K rows and
//     both accumulators, dV^T and dK^T, in registers, and its V rows in a
//     private LDS area.  For every rank that reaches the block and every
//     query head reading the KV head, the visible 64-row query tiles of Q and
//     dO stream through LDS (double buffered, buffer loads straight to LDS,
//     the forward's swizzle) with the tile's delta and lse2.  S = Q K^T and
//     dP = dO V^T take Q and dO rows as the M operand; dV^T += dO^T P and
//     dK^T += Q^T dS read dO and Q transposed.  S is computed once for both
//     gradients: four products per tile.
// Both passes deal their workgroups heaviest first (a host-side count of the
// tiles each one visits), and on a masked tile a wavefront that sees nothing
// of it skips the tile's products.
// The scale is applied once, to the final dQ and dK.
#include <algorithm>

#include "attn_tiles.h"
#include "usp_internal.h"

namespace usp {
namespace {

using namespace tiles;

constexpr int NW = 4;          // wavefronts per workgroup
constexpr int BM = 32 * NW;    // query rows per dQ workgroup
constexpr int KW = 8;          // wavefronts per dK/dV workgroup (32 keys each)
constexpr int STATS = 512;     // bytes of one tile's delta[64] and lse2[64]

__device__ inline int mod_cp(int x, int cp) {
  x %= cp;
  return x < 0 ? x + cp : x;
}

// Rows of a bf16 matrix as the N operand of v_mfma_f32_32x32x16_bf16: lane
// (n, hh) holds row n, dims 16 ks + 8 hh .. + 7.
template <int D>
__device__ inline void load_row_frags(bf16x8 *f, const __bf16 *row, bool valid, int hh) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    f[ks] = valid ? *reinterpret_cast<const bf16x8 *>(row + 16 * ks + 8 * hh) : bf16x8{};
}

// Per-lane LDS offsets of the operand reads on a 64-row tile (shared by both
// passes): row reads as the M operand (rows sig and 32 + sig, chunk 2 ks + hh)
// and transposed reads (4 rows x 4 dims per 4-lane group).
template <int D>
struct TileOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ inline TileOffsets(int lane) {
    const int n = lane & 31, hh = lane >> 5;
    const int sig = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = sig * Lds<D>::ROW + swz<D>(sig, 2 * ks + hh) * 16;
    const int tg = lane >> 4, trr = (lane >> 2) & 3, tq = lane & 3;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 8 * (tg >> 1) + 4 * e + trr;
        tr[mb][e] = r * Lds<D>::ROW + swz<D>(r, 4 * mb + 2 * (tg & 1) + (tq >> 1)) * 16 + (tq & 1) * 8;
      }
    }
  }
};

// M operand of 32 d-rows x 16 tile rows, read transposed from a row-major
// tile: tile rows 16 p .. 16 p + 15, dims 32 mb .. 32 mb + 31.
template <int D>
__device__ inline bf16x8 read_tr(const char *tile, const TileOffsets<D> &o, int mb, int p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<char *>(tile) + o.tr[mb][0] +
                                                                         p * 16 * Lds<D>::ROW));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<char *>(tile) + o.tr[mb][1] +
                                                                         p * 16 * Lds<D>::ROW));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-lane byte offsets of the direct tile loads of a W-wavefront workgroup
// (see issue_tile_lds).
template <int D, int W>
__device__ inline void tile_load_offsets(uint32_t *voff, int64_t rowbytes, int wave, int lane) {
  constexpr int CH = Lds<D>::CH;
#pragma unroll
  for (int i = 0; i < Lds<D>::KIB_PER_TILE / W; ++i) {
    const int row = (wave + W * i) * Lds<D>::KEYS_PER_KIB + lane / CH;
    voff[i] = (uint32_t)(row * rowbytes + swz<D>(row, lane % CH) * 16);
  }
}

// Schedule of N products that each take one operand row from LDS: AHEAD
// reads first, then two reads per two products.  Without it the compiler
// issues each read right before the product that consumes it and waits for
// it there; the operands are read ahead in the source as well.
template <int N, int AHEAD>
__device__ inline void schedule_products() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < (N - AHEAD) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}


// ================================================================ dQ pass ==

// PS: built for the per-sample split (the other build serves the split of the
// whole stream and holds no per-sample state)
template <int D, bool ACC, bool PS>
__global__ __launch_bounds__(64 * NW, 2) void dq_bf16_kernel(BwdArgs a) {
  // one array per stage, as in the forward: reads of one stage are then
  // provably disjoint from the direct loads filling the other
  __shared__ __attribute__((aligned(1024))) char smem0[Lds<D>::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[Lds<D>::STAGE];

  // work item: as the forward (heaviest query tiles first, the query heads
  // of one KV head back to back on one XCD)
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
  if (a.n_order > 0) {
    const int item = a.order[order];
    rank = a.ring_rank >= 0 ? a.ring_rank : item / a.n_tiles;
    lt = item % a.n_tiles;
  } else if (a.ring_rank >= 0) {
    rank = a.ring_rank;
    lt = a.n_tiles - 1 - order;
  } else {
    rank = order % a.cp;
    lt = a.n_tiles - 1 - order / a.cp;
  }
  const int hq = kvh * a.G + g;
  const int cp = a.cp, L = a.L;
  const ShareMap sm(a.c, a.cp, a.L, a.sm, PS);
  const bool causal = a.causal != 0, packed = sm.packed();

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  // rows [q0, qend); per-sample shares take tiles cut at their pieces
  int q0, qend;
  if (PS) {
    piece_tile(a.sm, a.ps_tiles, a.cp, BM, lt, q0, qend);
  } else {
    q0 = lt * BM;
    qend = min(q0 + BM, L);
  }
  const int qrow = q0 + wave * 32 + n;
  const bool qvalid = qrow < qend;
  const int qlast = qend - 1;
  const int qpos_min = sm.pos(rank, q0);
  const int qpos_max = sm.pos(rank, qlast);
  const int my_qpos = qvalid ? sm.pos(rank, qrow) : -1;
  int sst_min = 0, sst_max = 0, my_sst = 0, my_send = 0;
  if (packed) {
    sst_min = sm.seg_start(qpos_min);
    sst_max = sm.seg_start(qpos_max);
    my_sst = qvalid ? sm.seg_start(my_qpos) : 0x7fffffff;
    if (PS) my_send = qvalid ? sm.seg_end(my_qpos) : 0x7fffffff;
  }
  const int rs = a.ring_rank >= 0 ? 0 : rank;
  const int64_t srow = (((int64_t)rs * a.Hq + hq) * a.B + b) * L + qrow;
  const float delta = qvalid ? a.stats[srow] : 0.0f;
  const float lse2 = qvalid ? a.stats[a.rows + srow] : INFINITY;

  bf16x8 qf[D / 16], dof[D / 16];
  load_row_frags<D>(qf, static_cast<const __bf16 *>(a.q) + (a.ring_rank < 0 ? rank * a.q_rank : 0) + b * a.q_sb +
                            hq * a.q_sh + (int64_t)qrow * a.q_ss, qvalid, hh);
  load_row_frags<D>(dof, static_cast<const __bf16 *>(a.dout) + (a.ring_rank < 0 ? rank * a.do_rank : 0) +
                             b * a.do_sb + hq * a.do_sh + (int64_t)qrow * a.do_ss, qvalid, hh);

  // tile schedule: the key range of each step's block this query tile sees
  auto step_range = [&](int t) {
    StepRange r;
    r.j = mod_cp(rank - t, cp);
    const int hi = causal ? sm.count_le(r.j, qpos_max) : L;
    const int lo = packed ? sm.count_le(r.j, sst_min - 1) : 0;
    // the step's tiles start at lo (key row kt * BN + shift): in a packed
    // stream the first tile then holds no key of an earlier sample
    r.shift = lo % BN;
    if (hi <= lo) {
      r.kt = r.ke = 0;
    } else {
      r.kt = lo / BN;
      r.ke = r.kt + (hi - lo + BN - 1) / BN;
    }
    // key row i of block j is at or before position p iff i < count_le(j, p)
    r.fhi = causal ? sm.count_le(r.j, qpos_min) : L;
    r.flo = packed ? sm.count_le(r.j, sst_max - 1) : 0;
    return r;
  };
  int t = a.t_lo;
  StepRange cur = step_range(t);
  while (cur.kt >= cur.ke && ++t < a.t_hi) cur = step_range(t);

  const int64_t kbytes = a.k_ss * 2, vbytes = a.v_ss * 2;
  const char *const kbase = static_cast<const char *>(a.k) + 2 * (b * a.k_sb + kvh * a.k_sh);
  const char *const vbase = static_cast<const char *>(a.v) + 2 * (b * a.v_sb + kvh * a.v_sh);
  const uint32_t k_extent = (uint32_t)((L - 1) * kbytes + 2 * D);
  const uint32_t v_extent = (uint32_t)((L - 1) * vbytes + 2 * D);
  auto issue_tile = [&](int j, int k0, int stg) {
    char *const st = stg == 0 ? smem0 : smem1;
    uint32_t voff[Lds<D>::KIB_PER_TILE / NW];  // recomputed per tile: a few VALU ops, registers are short
    tile_load_offsets<D, NW>(voff, kbytes, wave, lane);
    issue_tile_lds<D, NW>(st, kbase + 2 * j * a.kv_blk, k_extent, kbytes, k0, L, wave, lane, voff);
    tile_load_offsets<D, NW>(voff, vbytes, wave, lane);
    issue_tile_lds<D, NW>(st + Lds<D>::TILE, vbase + 2 * j * a.kv_blk, v_extent, vbytes, k0, L, wave, lane, voff);
  };
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  const TileOffsets<D> off(lane);

  f32x16 dQ[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dQ[mb] = f32x16{};
  const float sl2 = a.scale_log2;

  auto advance = [&](int &tx, StepRange &x) {
    ++x.kt;
    while (x.kt >= x.ke && ++tx < a.t_hi) x = step_range(tx);
  };

  auto body = [&](auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    int t_nxt = t;
    StepRange nxt = cur;
    advance(t_nxt, nxt);
    if (t_nxt < a.t_hi) issue_tile(nxt.j, nxt.kt * BN + nxt.shift, STG ^ 1);

    const char *const sK = STG == 0 ? smem0 : smem1;
    const char *const sV = sK + Lds<D>::TILE;
    const int k0 = cur.kt * BN + cur.shift;
    const bool full = __builtin_amdgcn_readfirstlane((k0 >= cur.flo) & (k0 + BN <= cur.fhi));
    // positions grow with the local index, so the keys of block j this lane's
    // query sees are one local range; as offsets from the lane's first key
    // row in the tile, [vlo, vhi)
    int vlo = 0, vhi = BN;
    bool seen = true;
    if (!full) {
      const int hi = qvalid ? (causal ? sm.count_le_in(cur.j, my_qpos, my_sst, my_send) : L) : 0;
      const int lo = packed ? sm.count_le_in(cur.j, my_sst - 1, my_sst, my_send) : 0;
      vlo = lo - k0 - 8 * hh;
      vhi = hi - k0 - 8 * hh;
      // a wavefront none of whose queries sees this tile's keys skips its
      // products, leaving the matrix core to the other wavefronts of its SIMD
      seen = __builtin_amdgcn_ballot_w64((lo < hi) & (lo < k0 + BN) & (hi > k0)) != 0;
    }

    // per 32-key half: S^T = K Q^T and dP^T = V dO^T, then that half's
    // dS^T = P^T (dP^T - delta), rounded to bf16 as the N operand of the dQ
    // product.  One half's accumulators at a time leave the registers to
    // read a half's K and V rows ahead of its products.
    bf16x8 dsf[4];
#pragma unroll
    for (int half = 0; half < 2 * seen; ++half) {
      f32x16 S = f32x16{}, P = f32x16{};
      // K and V rows of two k-steps in registers; the next two are read while
      // this pair's four products run
      bf16x8 kr[2][2], vr[2][2];
      auto read_pair = [&](int slot, int ks0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          kr[slot][j] = *reinterpret_cast<const bf16x8 *>(sK + off.row[ks0 + j] + half * 32 * Lds<D>::ROW);
          vr[slot][j] = *reinterpret_cast<const bf16x8 *>(sV + off.row[ks0 + j] + half * 32 * Lds<D>::ROW);
        }
      };
      __builtin_amdgcn_s_setprio(1);
      read_pair(0, 0);
#pragma unroll
      for (int g = 0; g < D / 32; ++g) {
        if (g + 1 < D / 32) read_pair((g + 1) & 1, 2 * (g + 1));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[g & 1][j], qf[2 * g + j], S, 0, 0, 0);
          P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[g & 1][j], dof[2 * g + j], P, 0, 0, 0);
        }
      }
      schedule_products<D / 8, 4>();
      __builtin_amdgcn_s_setprio(0);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = 32 * half + 16 * (r / 8) + (r % 8);
          S[r] = ((kc >= vlo) & (kc < vhi)) ? S[r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], sl2, -lse2));
        dsf[2 * half + r / 8][r % 8] = (__bf16)(p * (P[r] - delta));
      }
    }
    // dQ^T += K^T dS^T, 16 keys per product; K^T read transposed
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mb = 0; mb < D / 32 * seen; ++mb) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        dQ[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(sK, off, mb, p), dsf[p], dQ[mb], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    wait_tiles();
    __syncthreads();
    t = t_nxt;
    cur = nxt;
  };

  if (t < a.t_hi) issue_tile(cur.j, cur.kt * BN + cur.shift, 0);
  wait_tiles();
  __syncthreads();
  while (t < a.t_hi) {
    body(StageTag<0>{});
    if (t >= a.t_hi) break;
    body(StageTag<1>{});
  }

  if (!qvalid) return;
  const float scale = a.scale;
  if (ACC) {
    float *o = static_cast<float *>(a.dq) + (((int64_t)hq * a.B + b) * L + qrow) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 *dst = reinterpret_cast<float4 *>(o + 32 * mb + 8 * r4 + 4 * hh);
        float4 val = *dst;
        val.x += dQ[mb][4 * r4 + 0] * scale;
        val.y += dQ[mb][4 * r4 + 1] * scale;
        val.z += dQ[mb][4 * r4 + 2] * scale;
        val.w += dQ[mb][4 * r4 + 3] * scale;
        *dst = val;
      }
    }
  } else {
    __bf16 *o = static_cast<__bf16 *>(a.dq) + (a.ring_rank < 0 ? rank * a.q_rank : 0) + b * a.q_sb +
                (int64_t)qrow * a.q_ss + hq * a.q_sh;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 val;
        val[0] = (__bf16)(dQ[mb][4 * r4 + 0] * scale);
        val[1] = (__bf16)(dQ[mb][4 * r4 + 1] * scale);
        val[2] = (__bf16)(dQ[mb][4 * r4 + 2] * scale);
        val[3] = (__bf16)(dQ[mb][4 * r4 + 3] * scale);
        *reinterpret_cast<bf16x4 *>(o + 32 * mb + 8 * r4 + 4 * hh) = val;
      }
    }
  }
}

// =========================================================== dK/dV pass ==

// Query tiles (64 rows) of rank r's share that can see a key tile whose
// positions span [kpos_min, kpos_max]: causal -- queries at or after
// kpos_min; packed -- queries before the end of kpos_max's sample.
// Query tiles [qt, qe) of one rank that see some key of the tile, and the
// tiles whose every query sees every key (first row >= flo, one past the last
// row <= fhi).
struct QRange {
  int qt, qe;
  int shift;  // the tiles start at query row qt * BN + shift
  int flo, fhi;
};

// Both key-side gradients in one pass: S = Q K^T and dP = dO V^T once per
// query tile, then dV^T += dO^T P and dK^T += Q^T dS.  Each wavefront holds
// its 32 keys' K rows and both accumulators in registers (160 of them) and
// keeps its V rows in a private LDS area (written once, read back as the dP
// operand), so that the pass fits two wavefronts per SIMD; the V rows in
// registers as well would spill.  Query tiles stream through a two-stage
// ring (the V areas take the LDS a third stage would need).  Measured on the
// 128K-token share's backward against separate dV and dK passes (which
// computed S twice): 60.1 against 69.7 ms for the whole backward.
template <int D, bool PS>
__global__ __launch_bounds__(64 * KW, 2) void dkdv_bf16_kernel(BwdArgs a) {
  constexpr int BK = 32 * KW;
  constexpr int TILE = Lds<D>::TILE;
  constexpr int STAGE = 2 * TILE;
  constexpr int NBLK = Lds<D>::KIB_PER_TILE / KW;
  constexpr int OPS = 2 * NBLK;
  constexpr int VROWS = 32 * Lds<D>::ROW;  // one wavefront's V rows
  __shared__ __attribute__((aligned(1024))) char ring0[STAGE + STATS];
  __shared__ __attribute__((aligned(1024))) char ring1[STAGE + STATS];
  __shared__ __attribute__((aligned(1024))) char vrows[KW * VROWS];

  const int n_slots = a.ring_rank >= 0 ? a.t_hi - a.t_lo : a.cp;
  int rest = blockIdx.x;
  const int g = rest % a.Hkv;
  rest /= a.Hkv;
  const int b = rest % a.B;
  rest /= a.B;
  const int sub = rest % a.order_sub;
  rest /= a.order_sub;
  if (a.n_order > 0) rest = a.order[rest];
  const int slot = rest % n_slots;
  const int kt = (rest / n_slots) * a.order_sub + sub;
  if (kt >= a.n_tiles) return;  // the last group's missing tiles (uniform)
  const int j = a.ring_rank >= 0 ? mod_cp(a.ring_rank - (a.t_lo + slot), a.cp) : slot;
  const int r_first = a.ring_rank >= 0 ? a.ring_rank : 0;
  const int r_last = a.ring_rank >= 0 ? a.ring_rank : a.cp - 1;
  const int L = a.L;
  const ShareMap sm(a.c, a.cp, a.L, a.sm, PS);
  const bool causal = a.causal != 0, packed = sm.packed();

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int k0 = kt * BK;
  const int krow = k0 + 32 * wave + n;
  const bool kvalid = krow < L;
  const int klast = min(k0 + BK, L) - 1;
  const int kpos_min = sm.pos(j, k0);
  const int kpos_max = sm.pos(j, klast);
  const int my_kpos = kvalid ? sm.pos(j, krow) : 0x7fffffff;
  int kend_min = 0x7fffffff, kend_max = 0x7fffffff, my_kend = 0x7fffffff;
  if (packed) {
    kend_min = sm.seg_end(kpos_min);
    kend_max = sm.seg_end(kpos_max);
    my_kend = kvalid ? sm.seg_end(my_kpos) : 0;
  }

  auto q_range = [&](int r) {
    QRange x;
    const int lo = causal ? sm.count_le(r, kpos_min - 1) : 0;
    const int hi = packed ? sm.count_le(r, kend_max - 1) : L;
    // the tiles start at lo: the first one holds no query before the
    // key tile's first position (or, packed, of an earlier sample)
    x.shift = lo % BN;
    if (hi <= lo) {
      x.qt = x.qe = 0;
    } else {
      x.qt = lo / BN;
      x.qe = x.qt + (hi - lo + BN - 1) / BN;
    }
    x.flo = causal ? sm.count_le(r, kpos_max - 1) : 0;
    x.fhi = packed ? sm.count_le(r, kend_min - 1) : L;
    return x;
  };
  struct It {
    int r, h;
    QRange x;
  };
  auto normalise = [&](It &it) {
    while (it.x.qt >= it.x.qe && it.r <= r_last) {
      if (++it.h == a.G) {
        it.h = 0;
        if (++it.r > r_last) break;
      }
      it.x = q_range(it.r);
    }
  };
  auto advance = [&](It &it) {
    ++it.x.qt;
    normalise(it);
  };
  It cur{r_first, 0, q_range(r_first)};
  normalise(cur);
  int lane_r = -1, lane_lo = 0, lane_hi = 0;
  if (cur.r > r_last) return;  // no query sees these keys (uniform)

  const TileOffsets<D> off(lane);
  bf16x8 kf[D / 16];
  const int64_t kvo = j * a.kv_blk;
  load_row_frags<D>(kf, static_cast<const __bf16 *>(a.k) + kvo + b * a.k_sb + g * a.k_sh + (int64_t)krow * a.k_ss,
                    kvalid, hh);
  // this wavefront's V rows, key n stored at row sig(n) of its area so that
  // the tile-row offsets read them back as the N operand
  char *const myv = vrows + wave * VROWS;
  {
    bf16x8 vf[D / 16];
    load_row_frags<D>(vf, static_cast<const __bf16 *>(a.v) + kvo + b * a.v_sb + g * a.v_sh + (int64_t)krow * a.v_ss,
                      kvalid, hh);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) *reinterpret_cast<bf16x8 *>(myv + off.row[ks]) = vf[ks];
  }

  const int64_t qbytes = a.q_ss * 2, dbytes = a.do_ss * 2;
  const uint32_t q_extent = (uint32_t)((L - 1) * qbytes + 2 * D);
  const uint32_t d_extent = (uint32_t)((L - 1) * dbytes + 2 * D);
  const __amdgpu_buffer_rsrc_t delta_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.stats), 0, (uint32_t)(a.rows * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t lse2_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.stats + a.rows), 0, (uint32_t)(a.rows * 4), RSRC_WORD3);
  auto issue = [&](const It &it, int stg) {
    const int hq = g * a.G + it.h;
    const char *qb = static_cast<const char *>(a.q) +
                     2 * ((a.ring_rank < 0 ? it.r * a.q_rank : 0) + b * a.q_sb + hq * a.q_sh);
    const char *db = static_cast<const char *>(a.dout) +
                     2 * ((a.ring_rank < 0 ? it.r * a.do_rank : 0) + b * a.do_sb + hq * a.do_sh);
    char *const st = stg == 0 ? ring0 : ring1;
    // the per-lane load offsets are recomputed here (a few integer ops): kept
    // across the loop they would be spilled
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint32_t qvoff[NBLK], dvoff[NBLK];
    tile_load_offsets<D, KW>(qvoff, qbytes, wave, ln);
    tile_load_offsets<D, KW>(dvoff, dbytes, wave, ln);
    issue_tile_lds<D, KW>(st, qb, q_extent, qbytes, it.x.qt * BN + it.x.shift, L, wave, ln, qvoff);
    issue_tile_lds<D, KW>(st + TILE, db, d_extent, dbytes, it.x.qt * BN + it.x.shift, L, wave, ln, dvoff);
    if (wave < 2) {
      const int rs = a.ring_rank >= 0 ? 0 : it.r;
      const int64_t srow = (((int64_t)rs * a.Hq + hq) * a.B + b) * L + it.x.qt * BN + it.x.shift;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave == 0 ? delta_rsrc : lse2_rsrc,
                                               (lds_void *)(st + STAGE + wave * (STATS / 2)), 4,
                                               (uint32_t)((srow + lane) * 4), 0, 0, 0);
    }
  };
  auto wait_tile = [&](int after) {
    if (wave < 2) {
      if (after >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS + 1) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (after >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  f32x16 accv[D / 32], acck[D / 32];  // dV^T and dK^T
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    accv[mb] = f32x16{};
    acck[mb] = f32x16{};
  }
  const float sl2 = a.scale_log2;

  It ld = cur;
  int pending = 0;
  issue(ld, 0);
  ++pending;
  advance(ld);

  auto body = [&](auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    wait_tile(pending - 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (ld.r <= r_last) {
      issue(ld, STG ^ 1);
      ++pending;
      advance(ld);
    }
    const char *const sQ = STG == 0 ? ring0 : ring1;
    const char *const sD = sQ + TILE;
    const float *const sst = reinterpret_cast<const float *>(sQ + STAGE);
    const int r = cur.r;
    const int q0 = cur.x.qt * BN + cur.x.shift;
    const bool full =
        __builtin_amdgcn_readfirstlane((k0 + BK <= L) & (q0 >= cur.x.flo) & (q0 + BN <= cur.x.fhi));
    int vlo = 0, vhi = BN;
    bool seen = true;
    if (!full) {
      if (r != lane_r) {
        lane_r = r;
        lane_lo = causal ? sm.count_le(r, my_kpos - 1) : 0;
        lane_hi = kvalid ? (packed ? sm.count_le(r, my_kend - 1) : L) : 0;
      }
      vlo = lane_lo - q0 - 8 * hh;
      vhi = lane_hi - q0 - 8 * hh;
      // a wavefront none of whose keys this tile's queries see (keys past
      // the tile's queries, or of other samples) skips the tile's products,
      // leaving the matrix core to the other wavefront of its SIMD
      seen = __builtin_amdgcn_ballot_w64((lane_lo < lane_hi) & (lane_lo < q0 + BN) & (lane_hi > q0)) != 0;
    }
#pragma unroll
    for (int blk = 0; blk < 2 * seen; ++blk) {
      // S = Q K^T, then P (kept in fp32 for dS, rounded for dV), dV^T +=
      // dO^T P, then dP = dO V^T, dS and dK^T += Q^T dS: P's rounding and
      // the dV products are done before dP takes its registers
      f32x16 S = f32x16{};
      __builtin_amdgcn_s_setprio(1);
      {
        bf16x8 qa[2];
        qa[0] = *reinterpret_cast<const bf16x8 *>(sQ + off.row[0] + blk * 32 * Lds<D>::ROW);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          if (ks + 1 < D / 16)
            qa[(ks + 1) & 1] = *reinterpret_cast<const bf16x8 *>(sQ + off.row[ks + 1] + blk * 32 * Lds<D>::ROW);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks & 1], kf[ks], S, 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      const float4 *d4 = reinterpret_cast<const float4 *>(sst + 32 * blk + 8 * hh);
      const float4 *l4 = reinterpret_cast<const float4 *>(sst + 64 + 32 * blk + 8 * hh);
      if (!full) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int qc = 32 * blk + 16 * (rr / 8) + (rr % 8);
          S[rr] = ((qc >= vlo) & (qc < vhi)) ? S[rr] : -INFINITY;
        }
      }
      bf16x8 pf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 lq4 = l4[(q4 / 2) * 4 + (q4 % 2)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * q4 + e;
          const float ls = e == 0 ? lq4.x : e == 1 ? lq4.y : e == 2 ? lq4.z : lq4.w;
          S[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rr], sl2, -ls));
          pf[rr / 8][rr % 8] = (__bf16)S[rr];
        }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const bf16x8 dt = read_tr<D>(sD, off, mb, 2 * blk + sl);
          accv[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dt, pf[sl], accv[mb], 0, 0, 0);
        }
      }
      f32x16 P = f32x16{};
      {
        bf16x8 da[2], va[2];
        da[0] = *reinterpret_cast<const bf16x8 *>(sD + off.row[0] + blk * 32 * Lds<D>::ROW);
        va[0] = *reinterpret_cast<const bf16x8 *>(myv + off.row[0]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          if (ks + 1 < D / 16) {
            da[(ks + 1) & 1] = *reinterpret_cast<const bf16x8 *>(sD + off.row[ks + 1] + blk * 32 * Lds<D>::ROW);
            va[(ks + 1) & 1] = *reinterpret_cast<const bf16x8 *>(myv + off.row[ks + 1]);
          }
          P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks & 1], va[ks & 1], P, 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      bf16x8 dsf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 dq4 = d4[(q4 / 2) * 4 + (q4 % 2)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * q4 + e;
          const float dlt = e == 0 ? dq4.x : e == 1 ? dq4.y : e == 2 ? dq4.z : dq4.w;
          dsf[rr / 8][rr % 8] = (__bf16)(S[rr] * (P[rr] - dlt));
        }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const bf16x8 qt = read_tr<D>(sQ, off, mb, 2 * blk + sl);
          acck[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, dsf[sl], acck[mb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    --pending;
    advance(cur);
  };

  while (true) {
    body(StageTag<0>{});
    if (pending == 0) break;
    body(StageTag<1>{});
    if (pending == 0) break;
  }

  if (!kvalid) return;
  float *dv = a.dv + kvo + b * a.v_sb + g * a.v_sh + (int64_t)krow * a.v_ss;
  float *dk = a.dk + kvo + b * a.k_sb + g * a.k_sh + (int64_t)krow * a.k_ss;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 *pv = reinterpret_cast<float4 *>(dv + 32 * mb + 8 * r4 + 4 * hh);
      float4 v = *pv;
      v.x += accv[mb][4 * r4 + 0];
      v.y += accv[mb][4 * r4 + 1];
      v.z += accv[mb][4 * r4 + 2];
      v.w += accv[mb][4 * r4 + 3];
      *pv = v;
      float4 *pk = reinterpret_cast<float4 *>(dk + 32 * mb + 8 * r4 + 4 * hh);
      float4 k = *pk;
      k.x += acck[mb][4 * r4 + 0] * a.scale;
      k.y += acck[mb][4 * r4 + 1] * a.scale;
      k.z += acck[mb][4 * r4 + 2] * a.scale;
      k.w += acck[mb][4 * r4 + 3] * a.scale;
      *pk = k;
    }
  }
}

// Key tiles (of BN keys) that query tile lt (BM rows) of `rank` visits over
// the launch's ring steps: the dQ pass's per-step tile range, computed on the
// host.
int query_tile_work(const BwdArgs &a, int rank, int lt) {
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  int q0, qend;
  if (a.sm.per_sample) {
    piece_tile(a.sm, a.ps_tiles, a.cp, BM, lt, q0, qend);
  } else {
    q0 = lt * BM;
    qend = std::min(q0 + BM, a.L);
  }
  const int pmax = sm.pos(rank, qend - 1), smin = sm.packed() ? sm.seg_start(sm.pos(rank, q0)) : 0;
  int work = 0;
  for (int t = a.t_lo; t < a.t_hi; ++t) {
    const int j = ((rank - t) % a.cp + a.cp) % a.cp;
    const int hi = a.causal ? sm.count_le(j, pmax) : a.L, lo = sm.packed() ? sm.count_le(j, smin - 1) : 0;
    if (hi > lo) work += (hi - lo + BN - 1) / BN;
  }
  return work;
}

// Sets a.order to items 0 .. m - 1 by decreasing work (stable).
void order_by_work(BwdArgs &a, const int *work, int m) {
  int idx[kMaxBwdOrder];
  for (int i = 0; i < m; ++i) idx[i] = i;
  std::stable_sort(idx, idx + m, [&](int x, int y) { return work[x] > work[y]; });
  for (int i = 0; i < m; ++i) a.order[i] = (uint16_t)idx[i];
  a.n_order = m;
}

// The dQ pass's query tiles heaviest first.  The tile index orders work only
// within one zigzag chunk of one rank; across the ranks of an all-ranks launch
// and across the pieces of per-sample shares it does not.
void order_query_tiles(BwdArgs &a) {
  a.n_order = 0;
  a.order_sub = 1;
  const int m = a.n_ranks * a.n_tiles;
  if (m > kMaxBwdOrder) return;
  int work[kMaxBwdOrder];
  for (int i = 0; i < m; ++i)
    work[i] = query_tile_work(a, a.ring_rank >= 0 ? a.ring_rank : i / a.n_tiles, i % a.n_tiles);
  order_by_work(a, work, m);
}

// Query tiles (of BN rows) that see key tile kt (BK keys) of block j, summed
// over the ranks the launch covers: the dK/dV pass's per-tile range, computed
// on the host.
int key_tile_work(const BwdArgs &a, int BK, int j, int kt) {
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  const int k0 = kt * BK, klast = std::min(k0 + BK, a.L) - 1;
  const int kpos_min = sm.pos(j, k0), kpos_max = sm.pos(j, klast);
  const int kend_max = sm.packed() ? sm.seg_end(kpos_max) : 0x7fffffff;
  const int r_first = a.ring_rank >= 0 ? a.ring_rank : 0, r_last = a.ring_rank >= 0 ? a.ring_rank : a.cp - 1;
  int work = 0;
  for (int r = r_first; r <= r_last; ++r) {
    const int lo = a.causal ? sm.count_le(r, kpos_min - 1) : 0;
    const int hi = sm.packed() ? sm.count_le(r, kend_max - 1) : a.L;
    if (hi > lo) work += (hi - lo + BN - 1) / BN;
  }
  return work;
}

// The dK/dV pass's workgroups heaviest first.  A key tile's work spans a
// wide range (under causal zigzag shares the first key tiles of the rank's
// own block see up to twice a full block's query tiles, the last ones a
// handful), one workgroup fills a CU, and in grid order the heavy tiles were
// spread over the launch, leaving some CUs a full tile behind at the end.
// Above kMaxBwdOrder (key tile, block) items the entries are groups of
// order_sub consecutive key tiles of one block, whose work is alike; the
// grid then has order_sub workgroups per entry.  Returns the entries' count.
int order_key_tiles(BwdArgs &a, int BK, int n_slots) {
  a.n_order = 0;
  a.order_sub = 1;
  if (n_slots <= 0 || a.n_tiles <= 0) return 0;
  if (n_slots > kMaxBwdOrder) return a.n_tiles * n_slots;
  const int per_slot = kMaxBwdOrder / n_slots;
  a.order_sub = (a.n_tiles + per_slot - 1) / per_slot;
  const int groups = (a.n_tiles + a.order_sub - 1) / a.order_sub, m = groups * n_slots;
  int work[kMaxBwdOrder];
  for (int i = 0; i < m; ++i) {
    const int slot = i % n_slots, grp = i / n_slots;
    const int j = a.ring_rank >= 0 ? ((a.ring_rank - (a.t_lo + slot)) % a.cp + a.cp) % a.cp : slot;
    work[i] = 0;
    for (int kt = grp * a.order_sub; kt < std::min((grp + 1) * a.order_sub, a.n_tiles); ++kt)
      work[i] += key_tile_work(a, BK, j, kt);
  }
  order_by_work(a, work, m);
  return m;
}

template <int D>
hipError_t launch_d(BwdArgs a, hipStream_t stream) {
  // dQ pass
  a.n_tiles = (a.L + BM - 1) / BM;
  if (a.sm.per_sample) a.n_tiles = fill_piece_tiles(a.sm, a.cp, BM, a.ps_tiles);
  const int64_t groups = (int64_t)a.n_ranks * a.n_tiles * a.B * a.Hkv;
  a.xcd_remap = groups % 8 == 0;
  order_query_tiles(a);
  const int64_t q_blocks = groups * a.G;
  if (q_blocks > 0) {
    const dim3 grid((uint32_t)q_blocks), block(64 * NW);
    if (a.sm.per_sample) {
      if (a.dq_acc)
        hipLaunchKernelGGL((dq_bf16_kernel<D, true, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((dq_bf16_kernel<D, false, true>), grid, block, 0, stream, a);
    } else {
      if (a.dq_acc)
        hipLaunchKernelGGL((dq_bf16_kernel<D, true, false>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((dq_bf16_kernel<D, false, false>), grid, block, 0, stream, a);
    }
  }
  // dK/dV pass
  a.n_tiles = (a.L + 32 * KW - 1) / (32 * KW);
  a.xcd_remap = 0;
  const int n_slots = a.ring_rank >= 0 ? a.t_hi - a.t_lo : a.cp;
  const int64_t entries = order_key_tiles(a, 32 * KW, n_slots);
  const int64_t k_blocks = entries * a.order_sub * a.B * a.Hkv;
  if (k_blocks > 0) {
    const dim3 grid((uint32_t)k_blocks), block(64 * KW);
    if (a.sm.per_sample)
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdArgs &a, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace usp
