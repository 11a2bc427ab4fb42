// Device helpers shared by the bf16 attention kernels (forward and
// backward): 64-row bf16 tiles staged global -> LDS with direct buffer loads
// and the XOR swizzle of their 16-byte chunks.  Positions of share rows come
// from positions.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace usp {
namespace tiles {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 64;   // rows per LDS tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int RSRC_WORD3 = 0x00020000;  // raw (untyped) buffer descriptor, gfx9 family

template <int S>
struct StageTag {
  static constexpr int value = S;
};

template <int D>
struct Lds {
  static constexpr int ROW = D * 2;               // bytes per key row (K and V alike)
  static constexpr int CH = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BN * ROW;           // one K or V tile
  static constexpr int STAGE = 2 * TILE;          // K then V
  static constexpr int BYTES = 2 * STAGE;         // double buffered
  static constexpr int KEYS_PER_KIB = 1024 / ROW; // rows one wave-wide direct load fills
  static constexpr int KIB_PER_TILE = TILE / 1024;
};

// Physical 16-byte chunk of logical chunk `ch` in key row `key`.  The XOR
// mask is a permutation of the low row bits onto chunk bits.  D = 128
// (256-byte rows, one bank sweep each): the 16 rows one K read touches get 16
// distinct masks, and the 4 rows of a transposed V read (row bits 0 and 1)
// move whole 4-chunk groups (chunk bits 2 and 3), so 32 lanes reading 4 rows
// x 4 chunks cover 16 distinct chunk slots.  D = 64 (two rows per sweep):
// the row parity picks the half sweep and row bits 1..3 are permuted, bit 1
// onto chunk bit 2.
template <int D>
__device__ inline int swz(int key, int ch) {
  if (D == 128) {
    const int f = ((key & 1) << 2) | ((key & 2) << 2) | ((key >> 2) & 1) | (((key >> 3) & 1) << 1);
    return ch ^ f;
  } else {
    const int f = (((key >> 1) & 1) << 2) | ((key >> 2) & 1) | (((key >> 3) & 1) << 1);
    return ch ^ f;
  }
}

// Lane l and lane l ^ 32 exchange a value (one VALU op, no LDS round trip).
__device__ inline float partner_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float partner_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Issue one 64-key tile of a KV block (K or V) into an LDS tile with buffer
// loads straight to LDS.  Wave w fills KiB blocks w, w + 4, ...; lane l of a
// block writes 16 bytes at block base + 16 l, so its per-lane offset `voff`
// names the logical chunk that the swizzle places there.  The descriptor is
// bounded to the block's extent.  When the share ends inside the tile, rows
// past it repeat the last row (their logits are masked, probabilities zero).
template <int D, int NW>
__device__ inline void issue_tile_lds(char *tile, const char *blk, uint32_t extent, int64_t rowbytes, int k0,
                                      int L, int wave, int lane, const uint32_t *voff) {
  constexpr int CH = Lds<D>::CH;
  constexpr int NBLK = Lds<D>::KIB_PER_TILE / NW;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(blk), 0, extent, RSRC_WORD3);
  if (k0 + BN <= L) {
    const uint32_t so = (uint32_t)(k0 * rowbytes);
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(tile + (wave + NW * i) * 1024), 16, voff[i], so, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
      const int row = (wave + NW * i) * Lds<D>::KEYS_PER_KIB + lane / CH;
      const int lch = swz<D>(row, lane % CH);
      const int key = min(k0 + row, L - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(tile + (wave + NW * i) * 1024), 16,
                                               (uint32_t)(key * rowbytes + lch * 16), 0, 0, 0);
    }
  }
}

// The key range of block j one query tile can see, in 64-key tiles.
// Schedule of N products whose M operand is read transposed from LDS (two
// reads per product): the reads of AHEAD products first, then two reads per
// product, so reads run that many products ahead of their use.  Without it
// the compiler reads each operand right before its product and waits there.
template <int N, int AHEAD>
__device__ inline void schedule_tr_products() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// One ring step of a tile walk: block j, its tiles [kt, ke) that hold some
// visible pair, the tiles with every pair visible (first row >= flo and one
// past the last row <= fhi), and the lane's own visible rows [llo, lhi).  All
// are local rows of the walked share, found once per step.
struct StepRange {
  int j, kt, ke;
  int shift;  // tiles of this step start at key row kt * tile + shift (forward walk)
  int flo, fhi;
  int llo, lhi;
};

}  // namespace tiles
}  // namespace usp
