// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Host code validates every argument before calling a launcher; launchers
// only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/usp.h"
#include "positions.h"

namespace usp {

// ---------------------------------------------------------------- copies --

// A batch of 2D row copies.  Item i copies `rows_per_item` rows of
// `row_bytes` bytes; rows of an item start at base offsets that depend on
// the copy kind and advance by fixed strides, with at most one jump (the
// zigzag share is two runs of positions).
enum CopyKind : int32_t {
  kZigzagFwd = 0,  // global (B,S,H,D) -> shards
  kZigzagInv = 1,  // shards -> global
  // Ulysses kinds move heads [h0, h0 + nh) of every head block (all hc/N by default)
  kUlyssesFwd = 2, // (N, bs, L/N, hc, hd) -> (G, nh, bs, L, hd)
  kUlyssesInv = 3, // (N, nh, bs, L, hd) -> (G, bs, L/N, hc, hd), the chunk's heads
  kUlyssesInvRows = 4, // the same, a row being one token's heads of the chunk in the output
  kUlyssesFwdRows = 5, // kUlyssesFwd, a row being one token's heads of the chunk in the source
};

struct CopyPlan {
  const char *src;
  char *dst;
  int32_t kind;
  uint32_t n_items;
  uint32_t rows_per_item;
  uint32_t row_vecs;        // 16-byte vectors per row
  uint32_t row_vecs_shift;  // log2(row_vecs) when a power of two, else 31
  uint32_t rows_per_piece;  // rows a workgroup copies per piece
  uint32_t pieces_per_item;
  uint64_t row_bytes;      // destination row
  uint64_t dst_unit_bytes; // unit of destination row offsets (row_bytes, or one head's hd elements)
  uint64_t src_row_bytes;  // source row (row_bytes, or one head's hd elements for kUlyssesInvRows)
  uint32_t grp_shift;      // log2(16-byte vectors per head row) when a row gathers (kUlyssesInvRows) or
                           // scatters (kUlyssesFwdRows) head rows, else 31
  // zigzag: B, S (rows), chunk c, rd, ud, shard rows T, fixed ranks (or -1)
  // ulysses: bs, L, hc, N, hb = hc/N, Ls = L/N, fixed rank (or -1), h0, nh,
  //          peers per item (kUlyssesInvRows, kUlyssesFwdRows)
  int64_t p[10];
};

hipError_t launch_copy(const CopyPlan &plan, hipStream_t stream);

// Up to kMaxCopyBatch plans in one launch (Q, K and V of one layout step).
constexpr int kMaxCopyBatch = 4;
struct CopyBatch {
  CopyPlan plan[kMaxCopyBatch];
  uint32_t first[kMaxCopyBatch + 1];  // first global piece of each plan; first[n] = total
  int32_t n;
};

hipError_t launch_copy_n(const CopyPlan *plans, int n, hipStream_t stream);

// Per-sample zigzag extract (or its inverse): a row gather whose source row
// comes from the share map of Samples.
struct ZigzagVarlenArgs {
  const char *src;
  char *dst;
  int64_t row_bytes;  // H * D * element size (a multiple of 16)
  int32_t B, S, rd, ud, T;  // T = S / (rd ud) rows per shard
  int32_t ring_rank, ulysses_rank;  // fixed ranks, or -1 for all
  int32_t inverse;
  Samples sm;
};

hipError_t launch_zigzag_varlen(const ZigzagVarlenArgs &a, hipStream_t stream);

// ----------------------------------------------------------------- merge --

hipError_t launch_lse_merge(float *o_acc, float *lse_acc, const float *o_step,
                            const float *lse_step, int64_t rows, int64_t head_dim,
                            hipStream_t stream);

// ------------------------------------------------------------- attention --

constexpr int kMaxTileOrder = 640;
constexpr int kMaxBwdOrder = 768;  // entries of a backward pass's work order
// A tile_order entry: the tile index in bits 0-9; under a split walk the
// part in bits 10-11 (0: every step, 1: steps before t_mid, 2: from t_mid)
// and t_mid in bits 12-15.
constexpr int kOrderTile = 1023, kOrderPartShift = 10, kOrderMidShift = 12;
constexpr int kMaxSplitCp = 15;

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  void *o;       // fp32 partial (Hq,B,L,D) [(cp,Hq,B,L,D) for every rank] or final in dtype with strides
  float *lse;    // (Hq,B,L), or (cp,Hq,B,L) for every rank
  int32_t B, Hq, Hkv, G;
  int32_t L;     // share length 2c
  int32_t c;     // chunk length
  int32_t cp;
  int32_t causal;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t kv_blk;
  int64_t q_rank, o_rank;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int32_t ring_rank; // >= 0, or -1 for every rank
  int32_t t_lo, t_hi; // ring steps to walk
  int32_t partial;    // 1: write fp32 partial (o_step, lse_step)
  int32_t merge;      // with partial: merge it into (o, lse) by the LSE rule instead of writing it
  int32_t n_qtiles;   // query tiles per share
  int32_t n_ranks;    // ranks in this launch (1 or cp)
  int32_t xcd_remap;  // 1: group blocks sharing a KV head on one XCD
  Samples sm;         // packed samples and the split of the shares
  int32_t ps_tiles[kMaxSeqs + 1];  // per-sample split, bf16: fill_piece_tiles at launch
  // bf16 walk: the (rank, query tile) pairs, rank * n_qtiles + tile,
  // heaviest first (set at launch when there are at most kMaxTileOrder;
  // n_order = 0: the tile index gives the order)
  int32_t n_order;
  uint16_t tile_order[kMaxTileOrder];
  // split walk (partial output only): the entries carry parts; part 2 writes
  // its partial slot_o / slot_lse elements after part 1's
  int32_t split;
  int64_t slot_o, slot_lse;
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments above 4 KiB");

hipError_t launch_attn_bf16(const AttnArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_attn_fp32(const AttnArgs &a, int head_dim, hipStream_t stream);

// Split walk of a bf16 launch of at most one round of workgroups: heavy
// tiles' ring steps over two workgroups, fp32 partials in the caller's
// workspace, then a finalize that merges them.
struct SplitPlan {
  float *po, *pl;            // partial o (two slots of rows x D) and lse (two slots of rows)
  int64_t slot_o, slot_lse;  // elements from slot 0 to slot 1
  int32_t split;             // set by the launch: 1 if tiles were split (finalize needed)
  int32_t bm, n_qtiles;      // query rows per tile and tiles per share of the split launch
  uint32_t mask[kMaxTileOrder / 32];  // the tiles (rank * n_qtiles + tile) that were split
};
hipError_t launch_attn_bf16_split(const AttnArgs &a, int head_dim, SplitPlan &plan, hipStream_t stream);

struct FinalizeArgs {
  const float *po, *pl;
  int64_t slot_o, slot_lse;
  void *o;                   // bf16, the caller's strides
  float *lse;                // (Hq,B,L), or (cp,Hq,B,L) for every rank
  int64_t o_sb, o_ss, o_sh, o_rank;
  int64_t rows;              // ranks x Hq x B x L
  int32_t B, Hq, L, d4;      // d4 = head_dim / 4
  int32_t ring_rank, bm, n_qtiles;
  uint32_t mask[kMaxTileOrder / 32];
};
hipError_t launch_split_finalize(const FinalizeArgs &f, hipStream_t stream);

// -------------------------------------------------------------- backward --

struct BwdArgs {
  const void *q;
  const void *k;
  const void *v;
  const void *dout;   // dO, dtype, O's strides
  const float *stats; // [delta (rows) | lse * log2(e) (rows)]
  int64_t rows;       // statistics rows: n_ranks * Hq * B * L
  void *dq;           // dtype with Q's strides, or fp32 (Hq,B,L,D) when dq_acc
  float *dk;          // fp32, K's strides
  float *dv;          // fp32, V's strides
  int32_t B, Hq, Hkv, G;
  int32_t L, c, cp, causal;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t kv_blk;
  int64_t q_rank, do_rank;
  float scale;
  float scale_log2;
  int32_t ring_rank;  // >= 0, or -1 for every rank (full walk only)
  int32_t t_lo, t_hi; // ring steps; the dK/dV pass covers the blocks they reach
  int32_t dq_acc;     // 1: add into the fp32 dq accumulator (one step)
  int32_t n_ranks;
  int32_t n_tiles;    // set by the launchers
  int32_t xcd_remap;  // set by the launchers
  Samples sm;         // packed samples and the split of the shares
  int32_t ps_tiles[kMaxSeqs + 1];  // per-sample split, dQ pass: fill_piece_tiles at launch
  // each pass's work items heaviest first, set at its launch (n_order = 0:
  // grid order).  dQ pass: rank * n_tiles + query tile, when there are at
  // most kMaxBwdOrder; dK/dV pass: key tile group * blocks + block slot, a
  // group being order_sub consecutive key tiles (one workgroup each)
  int32_t n_order;
  int32_t order_sub;
  uint16_t order[kMaxBwdOrder];
};
static_assert(sizeof(BwdArgs) <= 4096, "kernel arguments above 4 KiB");

struct PrepArgs {
  const void *o;
  const void *dout;
  const float *lse;
  float *stats;
  int64_t rows;  // n_ranks * Hq * B * L
  int32_t B, Hq, L;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t o_rank, do_rank;
};

hipError_t launch_bwd_prep(const PrepArgs &p, int head_dim, bool bf16, hipStream_t stream);

// ------------------------------------------ entry-point pieces (api.cpp) --

// Sets the calling thread's error detail to `msg` (cleared for USP_OK) and
// returns `s`.
usp_status report(usp_status s, const char *msg);

// Statistics rows of the backward for ring_rank (every rank for -1); the
// descriptor's sizes must be >= 1.
int64_t bwd_stats_rows(const usp_attn_desc *d, int32_t ring_rank);

// usp_attn_bwd with the statistics rows at `stats` (validation, prep, passes).
usp_status attn_bwd_with_stats(const void *q, const void *k_all, const void *v_all, const void *o, const void *d_o,
                               const float *lse, void *dq, float *dk_all, float *dv_all, float *stats,
                               const usp_attn_desc *desc, int32_t ring_rank, void *stream, const char *who);
hipError_t launch_attn_bwd_bf16(const BwdArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_attn_bwd_fp32(const BwdArgs &a, int head_dim, hipStream_t stream);

}  // namespace usp
