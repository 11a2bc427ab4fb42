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
//   * O^T += V^T P^T with P (the probabilities rounded to bf16) straight
//     from the S^T registers as the N operand: the K-row order of the first
//     product is permuted so that each lane's eight bf16 probabilities are
//     eight consecutive keys.  V stays row-major in LDS and is read
//     transposed into the M operand with ds_read_b64_tr_b16 (each 16-lane
//     group turns four 4-lane row reads into one column per lane);
//   * K and V tiles of 64 keys go global -> LDS directly with buffer loads
//     (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at the wave's
//     LDS base + 16 * lane, no registers involved).  A buffer descriptor per
//     KV block carries the block's exact byte extent, so no load can leave
//     the block; per-lane offsets are loop invariant and the tile offset is a
//     scalar.  Two LDS stages: the next tile is in flight while the current
//     one is computed, each tile costs one barrier, and the loop is unrolled
//     over the two stages so every LDS operand read uses an immediate offset
//     on a per-lane base computed once.  The 16-byte chunks of every key row
//     are XOR-swizzled by the row index, chosen so that the K operand reads
//     (16 rows, one chunk) and the transposed V reads (4 rows, two chunks)
//     hit distinct banks;
//   * the running max is a reference point, not the exact max: a tile's
//     probabilities are computed against it as long as they stay in range
//     (every lane's sum of its 32 below 2^64), so the tile max is only taken
//     on the first tiles of a row or when that check fails, and the reference
//     then moves (and O is rescaled) only if the tile max exceeds it by more
//     than 2^8.  This changes nothing but the reference point of the final
//     division: lse = m + log l stays exact (l sums the fp32 probabilities).
//     Wavefronts holding a row that sees at most kRoundedSumKeys keys divide
//     O by the sum of the bf16-rounded probabilities, the weights the PV
//     product applied, so that o's weights add up to one and a dominant key's
//     rounding (its P is not 1 under a stale reference) cancels; on longer
//     rows O is divided by l, the rounding of each P averaging out.
//
// Grid order: heaviest query tiles first (the last rows of a share see the
// most keys), and the Hq / Hkv query heads that read one KV head run back to
// back on one XCD (workgroups are dealt to the 8 XCDs round-robin) so that
// their K/V tiles are shared through that XCD's L2.
#include <algorithm>
#include <atomic>

#include "attn_tiles.h"
#include "lse_rule.h"
#include "usp_internal.h"

namespace usp {
namespace {

using namespace tiles;

// NW wavefronts per workgroup, 32 query rows each: BM = 32 NW query rows and
// 64 NW threads per workgroup.

constexpr float TAU = 8.0f;  // log2 headroom before the running max must move

// Rows that see at most this many keys in all divide O by the sum of the
// bf16-rounded probabilities (see the softmax below); longer rows by the fp32
// sum, where the rounding of each P averages out over the keys.
constexpr int kRoundedSumKeys = 2048;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// K and V tiles of TB keys in LDS (TB = 32 or 64).
template <int D, int TB>
struct KvLds {
  static constexpr int ROW = D * 2;                 // bytes per key row
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = TB * ROW;             // one K or V tile
  static constexpr int STAGE = 2 * TILE;            // K then V
  static constexpr int KEYS_PER_KIB = 1024 / ROW;   // rows one wave-wide direct load fills
  static constexpr int KIB_PER_TILE = TILE / 1024;
};

// Issue one TB-key tile of a KV block (K or V) into LDS with buffer loads
// straight to LDS.  Wave w fills KiB blocks w, w + NW, ...; the rows of
// block i are those of block 0 plus a multiple of 16, which the XOR swizzle
// (row bits 0..3) does not see, so one per-lane offset `voff0` (the logical
// chunk that the swizzle places at the lane's 16 bytes) serves every block
// and the rest of the address is a scalar.  The descriptor is bounded to the
// block's extent.  When the share ends inside the tile, rows past it repeat
// the last row (their logits are masked, probabilities zero).
template <int D, int TB, int NW>
__device__ inline void issue_kv_tile(char *tile, const char *blk, uint32_t extent, int64_t rowbytes, int k0, int L,
                                     int wave, int lane, uint32_t voff0) {
  using G = KvLds<D, TB>;
  constexpr int NBLK = G::KIB_PER_TILE / NW;
  constexpr int RSTEP = NW * G::KEYS_PER_KIB;
  static_assert(G::KIB_PER_TILE % NW == 0 && RSTEP % 16 == 0, "every wave fills whole 16-row swizzle periods");
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(blk), 0, extent, RSRC_WORD3);
  if (k0 + TB <= L) {
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(tile + (wave + NW * i) * 1024), 16, voff0,
                                               (uint32_t)((k0 + RSTEP * i) * rowbytes), 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
      const int row = (wave + NW * i) * G::KEYS_PER_KIB + lane / G::CH;
      const int lch = swz<D>(row, lane % G::CH);
      const int key = min(k0 + row, L - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(tile + (wave + NW * i) * 1024), 16,
                                               (uint32_t)(key * rowbytes + lch * 16), 0, 0, 0);
    }
  }
}

// PS: built for the per-sample split (the other build serves the split of the
// whole stream and holds no per-sample state).  TB: keys per tile, 64 (two
// workgroups per CU: 64 KiB of LDS and up to 256 registers each) or 32
// (three: 32 KiB and at most 168 registers, one logit accumulator and half
// the probabilities live), so that three waves share each SIMD.
template <int D, bool PARTIAL, int NW, bool PS, int TB>
__global__ __launch_bounds__(64 * NW, TB == 32 ? 3 : 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int BM = 32 * NW;
  constexpr int NBK = TB / 32;   // 32-key logit blocks per tile
  using KL = KvLds<D, TB>;
  // one array per stage: reads of one stage and the direct loads filling the
  // other are then provably disjoint, and the compiler does not make the
  // reads wait for those loads
  __shared__ __attribute__((aligned(1024))) char smem0[KL::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[KL::STAGE];

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
  // ring steps [t_begin, t_end) of this workgroup and its partial's slot
  int t_begin = a.t_lo, t_end = a.t_hi, slot = 0;
  if (a.n_order > 0) {  // the launch's heaviest-first order
    const int e = a.tile_order[order];
    const int idx = e & kOrderTile;
    rank = a.ring_rank >= 0 ? a.ring_rank : idx / a.n_qtiles;
    lt = idx % a.n_qtiles;
    if (PARTIAL && a.split) {  // a split tile: its first or second run of steps
      const int part = (e >> kOrderPartShift) & 3, t_mid = e >> kOrderMidShift;
      if (part == 1) t_end = t_mid;
      if (part == 2) {
        t_begin = t_mid;
        slot = 1;
      }
    }
  } else if (a.ring_rank >= 0) {
    rank = a.ring_rank;
    lt = a.n_qtiles - 1 - order;
  } else {
    rank = order % a.cp;
    lt = a.n_qtiles - 1 - order / a.cp;
  }
  const int hq = kvh * a.G + g;
  const int cp = a.cp, L = a.L;
  const ShareMap sm(a.c, a.cp, a.L, a.sm, PS);
  const bool causal = a.causal != 0, packed = sm.packed();

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  // Rows [q0, qend) of the share.  Under the per-sample split the share is a
  // run of pieces, two per sample (its chunks r and 2 cp - 1 - r, m rows
  // each), and tiles are cut at piece starts, so a tile's rows lie in one
  // sample and one chunk and its key range holds no other sample's keys.
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
  int sst_min = 0, sst_max = 0, my_sst = 0;
  if (packed) {
    sst_min = sm.seg_start(qpos_min);
    sst_max = sm.seg_start(qpos_max);
    my_sst = qvalid ? sm.seg_start(my_qpos) : 0x7fffffff;
  }
  // keys this lane's query sees over the whole walk: its position's distance
  // from the start of its sample, or every key without the causal mask
  const int my_keys = causal ? my_qpos - (packed ? my_sst : 0) + 1 : cp * L;
  const bool rounded_sum = __builtin_amdgcn_ballot_w64(qvalid && my_keys <= kRoundedSumKeys) != 0;

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
    const int hi = a.causal ? sm.count_le(r.j, qpos_max) : L;
    const int lo = packed ? sm.count_le(r.j, sst_min - 1) : 0;
    // the step's tiles start at lo (key row kt * TB + shift): in a packed
    // stream the first tile then holds no key of an earlier sample
    r.shift = lo % TB;
    if (hi <= lo) {
      r.kt = r.ke = 0;
    } else {
      r.kt = lo / TB;
      r.ke = r.kt + (hi - lo + TB - 1) / TB;
    }
    // a key row i of block j is at or before position p iff i < count_le(j, p),
    // so "every key <= the first query" and "every key in the last query's
    // sample" are bounds on the tile's rows
    r.fhi = a.causal ? sm.count_le(r.j, qpos_min) : L;
    r.flo = packed ? sm.count_le(r.j, sst_max - 1) : 0;
    r.lhi = qvalid ? (causal ? sm.count_le(r.j, my_qpos) : L) : 0;
    r.llo = packed ? sm.count_le(r.j, my_sst - 1) : 0;
    return r;
  };
  int t = t_begin;
  StepRange cur = step_range(t);
  while (cur.kt >= cur.ke && ++t < t_end) cur = step_range(t);

  // ------------------------------------------------ global -> LDS tiles --
  // per-lane byte offsets (within a tile) of the direct loads; see issue_kv_tile
  const int64_t kbytes = a.k_ss * 2, vbytes = a.v_ss * 2;
  uint32_t kvoff0, vvoff0;
  {
    const int row = wave * KL::KEYS_PER_KIB + lane / KL::CH;
    const int lch = swz<D>(row, lane % KL::CH);
    kvoff0 = (uint32_t)(row * kbytes + lch * 16);
    vvoff0 = (uint32_t)(row * vbytes + lch * 16);
  }
  const char *const kbase = static_cast<const char *>(a.k) + 2 * (b * a.k_sb + kvh * a.k_sh);
  const char *const vbase = static_cast<const char *>(a.v) + 2 * (b * a.v_sb + kvh * a.v_sh);
  const uint32_t k_extent = (uint32_t)((L - 1) * kbytes + 2 * D);
  const uint32_t v_extent = (uint32_t)((L - 1) * vbytes + 2 * D);
  auto issue_tile = [&](int j, int k0, int stg) {
    char *const st = stg == 0 ? smem0 : smem1;
    issue_kv_tile<D, TB, NW>(st, kbase + 2 * j * a.kv_blk, k_extent, kbytes, k0, L, wave, lane, kvoff0);
    issue_kv_tile<D, TB, NW>(st + KL::TILE, vbase + 2 * j * a.kv_blk, v_extent, vbytes, k0, L, wave, lane, vvoff0);
  };
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // Per-lane LDS byte offsets of the MFMA operand reads, relative to a tile.
  // K operand: row 32*kb + sig, logical chunk 2*ks + hh (rows sig and 32 + sig
  // share the swizzle mask).  V operand (transposed reads): lane 16*g + 4*r + q
  // reads row 16*p + 8*(g/2) + 4*e + r at dims 32*mb + 16*(g%2) + 4q .. +3;
  // the mask depends on the row mod 16 only, so p moves by whole 16-row blocks.
  const int sig = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = sig * KL::ROW + swz<D>(sig, 2 * ks + hh) * 16;
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  int voff[D / 32][2];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 8 * (tg >> 1) + 4 * e + tr;
      voff[mb][e] = row * KL::ROW + swz<D>(row, 4 * mb + 2 * (tg & 1) + (tq >> 1)) * 16 + (tq & 1) * 8;
    }
  }

  // --------------------------------------------------------- main loop --
  f32x16 O[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) O[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f, lr_run = 0.0f;
  const float sl2 = a.scale_log2;

  // next tile of the walk after `x` (workgroup-uniform); `tx` is its step
  auto advance = [&](int &tx, StepRange &x) {
    ++x.kt;
    while (x.kt >= x.ke && ++tx < t_end) x = step_range(tx);
  };

  // The pieces of one tile.  Every LDS operand read below is a per-lane base
  // plus an immediate offset when the tile's stage is a compile-time
  // constant at the call.
  f32x16 S[NBK];
  bf16x8 pf[2 * NBK];

  // S^T = K Q^T for the tile's NBK 32-key blocks.  The K rows of k-step
  // ks + AH are read while k-step ks's products run, and the products
  // alternate between the blocks' accumulators, so no chain waits on
  // another.
  auto qk = [&](const char *sK) {
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) S[kb] = f32x16{};
    constexpr int NKS = D / 16, AH = 3;
    bf16x8 kr[AH + 1][NBK];
#pragma unroll
    for (int i = 0; i < AH; ++i) {
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
        kr[i][kb] = *reinterpret_cast<const bf16x8 *>(sK + koff[i] + 32 * kb * KL::ROW);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + AH < NKS) {
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
          kr[(ks + AH) % (AH + 1)][kb] = *reinterpret_cast<const bf16x8 *>(sK + koff[ks + AH] + 32 * kb * KL::ROW);
      }
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[ks % (AH + 1)][kb], qf[ks], S[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NBK * AH, 0);
#pragma unroll
    for (int i = 0; i < NKS - AH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NBK, 0);
      if (NBK == 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NBK * AH, 0);
  };

  // A tile that straddles the diagonal, a sample boundary or the ragged end
  // (not every pair of the workgroup visible) takes the elementwise mask.
  // Positions grow with the local row, so the keys of block j this lane's
  // query sees are one local range; as offsets from the lane's first key row
  // in the tile, [vlo, vhi).
  auto mask = [&](const StepRange &x) {
    const int k0 = x.kt * TB + x.shift;
    const bool full = __builtin_amdgcn_readfirstlane((k0 >= x.flo) & (k0 + TB <= x.fhi));
    if (!full) {
      const int vlo = x.llo - k0 - 8 * hh, vhi = x.lhi - k0 - 8 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kc = 16 * (r / 8) + (r % 8);
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
          S[kb][r] = ((kc + 32 * kb >= vlo) & (kc + 32 * kb < vhi)) ? S[kb][r] : -INFINITY;
      }
    }
  };

  // online softmax (base 2, scale folded in) against the running reference
  // m_run.  The tile's row max is only taken when some row has no reference
  // yet or when a probability left the safe range (a lane's sum of its
  // probabilities is not below 2^64, which also catches inf); otherwise the
  // probabilities of the stale reference are used as they are, which
  // changes nothing but the reference point of the final division.  When
  // the max is taken, the reference only moves if the tile max exceeds it
  // by more than 2^TAU.
  auto softmax = [&]() {
    float ps, pr;
    auto probs = [&](float m_use) {
      // Two row sums.  lse takes the unrounded probabilities, so it is exact
      // to fp32 rounding.  On waves holding a row with few keys O is divided
      // by the sum of their bf16 roundings, the weights the PV product
      // actually applied: the weights of the final o then add up to one, and
      // a key that dominates its row (P far above the others, not 1 under
      // the lazy reference) contributes its value with no error from the
      // rounding of its P.  Two partial sums keep two add chains.
      float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], sl2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r + 1], sl2, -m_use));
          ps0 = kb == 0 && r == 0 ? p0 : ps0 + p0;
          ps1 = kb == 0 && r == 0 ? p1 : ps1 + p1;
          pf[2 * kb + r / 8][r % 8] = (__bf16)p0;
          pf[2 * kb + r / 8][r % 8 + 1] = (__bf16)p1;
        }
      }
      ps = ps0 + ps1;
      if (rounded_sum) {  // wave-uniform
        float pr0 = 0.0f, pr1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 2 * NBK; ++i) {
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            pr0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[i][e], pf[i][e + 1]}, kOnes2, pr0, false);
            pr1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[i][e + 2], pf[i][e + 3]}, kOnes2, pr1, false);
          }
        }
        pr = pr0 + pr1;
      } else {
        pr = ps;
      }
    };
    bool need_max = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    if (!need_max) {
      probs(m_run);
      need_max = __builtin_amdgcn_ballot_w64(!(ps < 0x1p64f)) != 0;
    }
    if (need_max) {  // wave-uniform
      float mx = S[0][0];
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
      }
      mx = partner_max(mx) * sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {  // some row's reference moves: rescale
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        lr_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) O[mb] *= alpha;
        m_run = m_new;
      }
      probs(m_run == -INFINITY ? 0.0f : m_run);
    }
    l_run += ps;
    lr_run += pr;
  };

  // O^T += V^T P^T, 16 keys per MFMA; V^T read transposed from row-major V.
  // One 16-key group of P at a time across all D / 32 accumulators (the
  // chains interleave); the next group's V operands are read meanwhile.
  auto pv = [&](const char *sV) {
    auto read_v = [&](int mb, int p) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(const_cast<char *>(sV) + voff[mb][0] + p * 16 * KL::ROW));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(const_cast<char *>(sV) + voff[mb][1] + p * 16 * KL::ROW));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vt[2][D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) vt[0][mb] = read_v(mb, 0);
#pragma unroll
    for (int p = 0; p < 2 * NBK; ++p) {
      if (p + 1 < 2 * NBK) {
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) vt[(p + 1) & 1][mb] = read_v(mb, p + 1);
      }
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt[p & 1][mb], pf[p], O[mb], 0, 0, 0);
    }
    schedule_tr_products<2 * NBK * (D / 32), D / 32>();
  };

  // One tile on LDS stage STG: the next tile goes into the other stage
  // while this one is computed.
  auto body = [&](auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    int t_nxt = t;
    StepRange nxt = cur;
    advance(t_nxt, nxt);
    if (t_nxt < t_end) issue_tile(nxt.j, nxt.kt * TB + nxt.shift, STG ^ 1);
    const char *const sK = STG == 0 ? smem0 : smem1;
    __builtin_amdgcn_s_setprio(1);  // keep the matrix core fed while the SIMD's other waves run softmax
    qk(sK);
    __builtin_amdgcn_s_setprio(0);
    mask(cur);
    softmax();
    __builtin_amdgcn_s_setprio(1);
    pv(sK + KL::TILE);
    __builtin_amdgcn_s_setprio(0);
    wait_tiles();
    __syncthreads();
    t = t_nxt;
    cur = nxt;
  };

  // prologue: tile 0 into stage 0
  if (t < t_end) issue_tile(cur.j, cur.kt * TB + cur.shift, 0);
  wait_tiles();
  __syncthreads();
  while (t < t_end) {
    body(StageTag<0>{});
    if (t >= t_end) break;
    body(StageTag<1>{});
  }

  // ---------------------------------------------------------- epilogue --
  const float l = partner_sum(l_run), lr = partner_sum(lr_run);
  const bool empty = !(l > 0.0f);
  const float inv = empty || !(lr > 0.0f) ? 0.0f : 1.0f / lr;
  const float lse = empty ? -INFINITY : (m_run + __log2f(l)) * 0.69314718055994530942f;
  if (!qvalid) return;
  if (PARTIAL && a.merge) {
    // the step's partial folded into the accumulator by the LSE rule: a row
    // whose accumulator is empty (lse -inf) takes the partial as it is, a row
    // with no key in this step leaves it alone.  Both lanes of a row read the
    // accumulator's lse before the row's writer lane (hh = 0) stores the new
    // one: one instruction each, in program order within the wavefront.
    const int64_t prow = (((a.ring_rank < 0 ? (int64_t)rank * a.Hq : 0) + hq) * a.B + b) * L + qrow;
    float *o = static_cast<float *>(a.o) + prow * D;
    const float la = a.lse[prow];
    double w1, w2, lm;
    merge_weights((double)la, (double)lse, w1, w2, lm);
    const bool take = la == -INFINITY, keep = !take && empty;
    if (!keep) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4 y;
          y.x = O[mb][4 * r4 + 0] * inv;
          y.y = O[mb][4 * r4 + 1] * inv;
          y.z = O[mb][4 * r4 + 2] * inv;
          y.w = O[mb][4 * r4 + 3] * inv;
          float4 *po = reinterpret_cast<float4 *>(o + 32 * mb + 8 * r4 + 4 * hh);
          *po = take ? y : blend(w1, *po, w2, y);
        }
      }
    }
    if (hh == 0 && !keep) a.lse[prow] = take ? lse : (float)lm;
    return;
  }
  if (PARTIAL) {
    const int64_t prow = (((a.ring_rank < 0 ? (int64_t)rank * a.Hq : 0) + hq) * a.B + b) * L + qrow;
    float *o = static_cast<float *>(a.o) + slot * a.slot_o + prow * D;
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
    a.lse[li + slot * a.slot_lse] = lse;
  }
}

}  // namespace

template <int D, int NW, bool PS, int TB>
void launch_one(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.partial)
    hipLaunchKernelGGL((attn_bf16_kernel<D, true, NW, PS, TB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, false, NW, PS, TB>), grid, block, 0, stream, a);
}

// Keys per tile: 64.  The kernel also builds with 32-key tiles (TB = 32:
// 168 registers and 32 KiB of LDS, three workgroups per CU instead of two).
// Measured, those ran the whole 16-head block of the 128K-token hybrid share
// 0.5-1.3% faster but a 4096-token share 2.5-5% slower and the share in head
// chunks 3-15% slower (a workgroup lives about 1.5 times as long, so each
// launch's last, partly filled round idles more of the chip), and they are
// not used.
constexpr int kWalkTile = 64;

// Key tiles a query tile of `rank` visits over ring steps [t0, t1): the
// kernel's per-step tile range, computed on the host.
int tile_work(const AttnArgs &a, int BM, int rank, int lt, int t0, int t1) {
  const ShareMap sm(a.c, a.cp, a.L, a.sm);
  int q0, qend;
  if (a.sm.per_sample) {
    piece_tile(a.sm, a.ps_tiles, a.cp, BM, lt, q0, qend);
  } else {
    q0 = lt * BM;
    qend = q0 + BM < a.L ? q0 + BM : a.L;
  }
  const int pmin = sm.pos(rank, q0), pmax = sm.pos(rank, qend - 1), smin = sm.seg_start(pmin);
  int work = 0;
  for (int t = t0; t < t1; ++t) {
    const int j = ((rank - t) % a.cp + a.cp) % a.cp;
    const int hi = a.causal ? sm.count_le(j, pmax) : a.L, lo = sm.count_le(j, smin - 1);
    if (hi > lo) work += (hi - lo + kWalkTile - 1) / kWalkTile;
  }
  return work;
}

// Compute units of the current device (queried once per device; calls from
// several host threads may query it concurrently and store the same value).
int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// The workgroups of a launch in decreasing order of work, so that long ones
// start first and short ones fill the last round.  The tile index alone
// orders work only within one zigzag chunk of one rank: across the ranks of
// an all-ranks launch the first chunk's tiles grow with the rank and the
// second chunk's shrink, and packed samples restart at every sample.
// A launch whose workgroups are all resident at once (one round at two
// workgroups per CU) takes the second half in increasing order, so that the
// CU given the heaviest tile of the first half gets the lightest of the
// second (the 128K-token share in chunks of two query heads: 19.88 -> 19.41
// ms per step).
void order_items(AttnArgs &a, const uint16_t *item, const int *work, int m, int per_cu) {
  int idx[kMaxTileOrder];
  for (int i = 0; i < m; ++i) idx[i] = i;
  std::stable_sort(idx, idx + m, [&](int x, int y) { return work[x] > work[y]; });
  const int64_t wgs = (int64_t)m * a.B * a.Hkv * a.G;
  if (per_cu == 2 && wgs <= 2 * (int64_t)device_cus()) std::reverse(idx + m / 2, idx + m);
  for (int i = 0; i < m; ++i) a.tile_order[i] = item[idx[i]];
  a.n_order = m;
}

void order_tiles(AttnArgs &a, int BM, int per_cu) {
  a.n_order = 0;
  const int n = a.n_ranks * a.n_qtiles;
  if (n > kMaxTileOrder) return;
  uint16_t item[kMaxTileOrder];
  int work[kMaxTileOrder];
  for (int i = 0; i < n; ++i) {
    item[i] = (uint16_t)i;
    work[i] = tile_work(a, BM, a.ring_rank >= 0 ? a.ring_rank : i / a.n_qtiles, i % a.n_qtiles, a.t_lo, a.t_hi);
  }
  order_items(a, item, work, n, per_cu);
}

// Split walk: every tile whose work is above the launch's mean is walked by
// two workgroups, one over the ring steps before t_mid and one from t_mid,
// with t_mid the step boundary that halves its work best; each writes an
// fp32 partial (o, lse) into its own slot, and the finalize kernel merges
// the two by the LSE rule.  For launches of at most one round of workgroups,
// where a heavy tile would otherwise run alone at the tail.  False when no
// tile is split (the caller then runs the plain walk).  per_cu: workgroups
// per CU, for the order of the items.
bool split_tiles(AttnArgs &a, int BM, uint32_t *mask, int per_cu) {
  const int n = a.n_ranks * a.n_qtiles;
  if (a.cp < 2 || a.cp > kMaxSplitCp || a.sm.nseq > 0 || n > kMaxTileOrder) return false;
  int work[kMaxTileOrder];
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    work[i] = tile_work(a, BM, a.ring_rank >= 0 ? a.ring_rank : i / a.n_qtiles, i % a.n_qtiles, a.t_lo, a.t_hi);
    total += work[i];
  }
  for (int w = 0; w < kMaxTileOrder / 32; ++w) mask[w] = 0;
  uint16_t item[kMaxTileOrder];
  int iw[kMaxTileOrder];
  int m = 0;
  bool any = false;
  for (int i = 0; i < n; ++i) {
    const int rank = a.ring_rank >= 0 ? a.ring_rank : i / a.n_qtiles, lt = i % a.n_qtiles;
    int best = -1, best_w = 0, best_d = 0;
    if ((int64_t)work[i] * n > total) {
      int acc = 0;
      for (int t = a.t_lo + 1; t < a.t_hi; ++t) {
        acc += tile_work(a, BM, rank, lt, t - 1, t);
        const int d = std::abs(2 * acc - work[i]);
        if (best < 0 || d < best_d) {
          best = t;
          best_w = acc;
          best_d = d;
        }
      }
    }
    // both parts need work, and the items must fit the table
    if (best > 0 && best_w > 0 && best_w < work[i] && m + 2 + (n - 1 - i) <= kMaxTileOrder) {
      item[m] = (uint16_t)(i | 1 << kOrderPartShift | best << kOrderMidShift);
      iw[m++] = best_w;
      item[m] = (uint16_t)(i | 2 << kOrderPartShift | best << kOrderMidShift);
      iw[m++] = work[i] - best_w;
      mask[i >> 5] |= 1u << (i & 31);
      any = true;
    } else {
      item[m] = (uint16_t)i;
      iw[m++] = work[i];
    }
  }
  if (!any) return false;
  order_items(a, item, iw, m, per_cu);
  a.split = 1;
  return true;
}

template <int NW>
hipError_t launch_nw(AttnArgs a, int head_dim, hipStream_t stream, bool ordered = false) {
  constexpr int BM = 32 * NW;
  if (!ordered) {
    a.n_qtiles = (a.L + BM - 1) / BM;
    if (a.sm.per_sample) a.n_qtiles = fill_piece_tiles(a.sm, a.cp, BM, a.ps_tiles);
    order_tiles(a, BM, NW == 4 ? 2 : 1);
  }
  // the grid: one workgroup per (order item, batch, KV head, query head of the group)
  const int64_t items = a.n_order > 0 ? a.n_order : (int64_t)a.n_ranks * a.n_qtiles;
  const int64_t groups = items * a.B * a.Hkv;
  a.xcd_remap = groups % 8 == 0;
  const int64_t blocks = groups * a.G;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((uint32_t)blocks), block(64 * NW);
  if constexpr (NW == 8) {  // unpacked launches only: no per-sample split
    if (head_dim == 128)
      launch_one<128, NW, false, kWalkTile>(a, grid, block, stream);
    else
      launch_one<64, NW, false, kWalkTile>(a, grid, block, stream);
  } else {
    const bool ps = a.sm.per_sample != 0;
    if (head_dim == 128)
      ps ? launch_one<128, NW, true, kWalkTile>(a, grid, block, stream)
         : launch_one<128, NW, false, kWalkTile>(a, grid, block, stream);
    else
      ps ? launch_one<64, NW, true, kWalkTile>(a, grid, block, stream)
         : launch_one<64, NW, false, kWalkTile>(a, grid, block, stream);
  }
  return hipGetLastError();
}

// Eight wavefronts (256 query rows) per workgroup share each K/V tile, which
// halves the tile loads per query row: alternating on one box, 2.8% faster on
// the 128K-token share and 4.2% on a 4096-token GQA share than four.  Packed
// samples keep four wavefronts (128 rows): their query tiles are cut at
// samples or pieces, and 256-row tiles ran the packed 32K ranks 16% slower.
// So do launches that would give fewer than two eight-wave workgroups per CU
// (one round of tiles of unequal work, e.g. two query heads of the 128K
// share): four-wave workgroups run two per CU and halve each tile's work.
bool four_waves(const AttnArgs &a) {
  const int64_t blocks8 = (int64_t)a.n_ranks * ((a.L + 255) / 256) * a.B * a.Hkv * a.G;
  return a.sm.nseq > 0 || blocks8 < 2 * (int64_t)device_cus();
}

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t stream) {
  return four_waves(a) ? launch_nw<4>(a, head_dim, stream) : launch_nw<8>(a, head_dim, stream);
}

// The split walk runs eight-wave workgroups (256 query rows), one per CU:
// with the heavy tiles split, the launch is about one and a half rounds
// either way, and eight waves share each K/V tile.  Measured on the 128K
// share in chunks of two query heads (one stream): 16.86 ms per step with
// four-wave workgroups (128 rows, two per CU), 15.52 ms with eight, against
// 14.60 ms for the whole block.
hipError_t launch_attn_bf16_split(const AttnArgs &a0, int head_dim, SplitPlan &plan, hipStream_t stream) {
  plan.split = 0;
  if (!four_waves(a0) || a0.sm.nseq > 0) return launch_attn_bf16(a0, head_dim, stream);
  constexpr int BM = 256;
  AttnArgs a = a0;
  a.n_qtiles = (a.L + BM - 1) / BM;
  const int64_t wgs = (int64_t)a.n_ranks * a.n_qtiles * a.B * a.Hkv * a.G;
  if (wgs > (int64_t)device_cus() || !split_tiles(a, BM, plan.mask, 1)) return launch_attn_bf16(a0, head_dim, stream);
  a.o = plan.po;
  a.lse = plan.pl;
  a.slot_o = plan.slot_o;
  a.slot_lse = plan.slot_lse;
  a.partial = 1;
  plan.split = 1;
  plan.bm = BM;
  plan.n_qtiles = a.n_qtiles;
  return launch_nw<8>(a, head_dim, stream, true);
}

}  // namespace usp
