// Host-side planning helpers of libsvq: LDS and workspace sizes and the
// block shapes of the small-batch and dequant-GEMM launches.  Plain C++ (no
// device code), shared by the library and the host-only launch checks.
#include "svq_internal.h"

namespace svq {

// LDS of the m = 2..4 main launch: radius table, direction copies of the
// largest bd, partial sums of R tiles.
size_t gemv_smem_bytes(int m, int bd_max, int r_max) {
  return (size_t)GV_OFF_D + ((size_t)gv_copies(bd_max) << bd_max) * 16 +
         (size_t)r_max * GV_WAVES * 64 * m * 4;
}

// LDS of one fused block at m = 1 for a matrix of k channels, `units` units,
// r row tiles per block.
size_t gemv_fused_smem_bytes(int k, int units, int bd, int r) {
  return (size_t)gf_lds(bd, k, units, 1, r).total;
}

// Items per block: all blocks of a call resident at once (two 4-wave
// blocks per compute unit) when that takes at most SB_NMAX items per wave,
// and at least SB_ITEMS_MIN.
int sb_block_items(int64_t total_items, int cus) {
  const int64_t slots = 2 * (int64_t)cus;
  int64_t it = (total_items + slots - 1) / slots;
  if (it < SB_ITEMS_MIN) it = SB_ITEMS_MIN;
  if (it > SB_WAVES * SB_NMAX) it = SB_WAVES * SB_NMAX;
  return (int)it;
}

// Matrices of up to SB_MAX_RANGE units keep all of K in one block, longer
// ones are cut into ranges of about 5 units; then as many row tiles per
// block (up to SB_TMAX) as give about `items` items, at most SB_NMAX per
// wave.
SbPlan sb_plan(int n_tiles, int units, int items) {
  SbPlan p;
  p.splits = units <= SB_MAX_RANGE ? 1 : (units + 4) / 5;
  p.upr = (units + p.splits - 1) / p.splits;
  p.splits = (units + p.upr - 1) / p.upr;
  p.tiles = (items + p.upr / 2) / p.upr;
  p.tiles = p.tiles < 1 ? 1 : (p.tiles > SB_TMAX ? SB_TMAX : p.tiles);
  while (p.tiles > 1 && p.tiles * p.upr > SB_WAVES * SB_NMAX) --p.tiles;
  p.groups = (n_tiles + p.tiles - 1) / p.tiles;
  return p;
}

size_t sb_ws_bytes(int n_tiles, int units, int items) {
  const SbPlan p = sb_plan(n_tiles, units, items);
  size_t bytes = align256((size_t)units * SB_XA_UNIT_BYTES) + align256((size_t)units * 16 * 4);
  if (p.splits > 1)
    bytes += align256((size_t)p.groups * p.tiles * p.splits * 1024) + align256((size_t)p.groups * 4);
  return bytes;
}

// LDS of a dequant-GEMM prep block: rpb staged rows of k + 8 values.
size_t prefill_prep_lds(int rpb, int k) { return (size_t)rpb * (k + 8) * 2; }

// Up to 8 rows, fewer for long rows: a block's staging stays near 40 KB, so
// that several prep blocks share a compute unit (with whole 156 KB of rows
// per block, one block per unit waits out each row load alone).
constexpr size_t PREP_LDS_TARGET = 40 * 1024;
int prefill_prep_rows(int k) {
  int rpb = 8;
  while (rpb > 1 && prefill_prep_lds(rpb, k) > PREP_LDS_TARGET) rpb /= 2;
  return rpb;
}

int prefill_bm(int m) { return m >= PREFILL_MIN_M ? 256 : 64; }

int prefill_m_pad(int m) {
  const int bm = prefill_bm(m);
  return ((m + bm - 1) / bm) * bm;
}

}  // namespace svq
