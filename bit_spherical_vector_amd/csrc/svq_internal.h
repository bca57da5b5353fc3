// Internal layout and launch interfaces of libsvq (not part of the public ABI).
//
// Packed matrix buffer (all offsets 256-byte aligned, see svq_handle):
//
//   dtab   256 x 8 fp16   row b = D[b & ((1<<bd)-1)]: the direction row picked
//                         by the low byte of a code's 10-bit index
//   rtab   1024 fp16      entry idx = R[idx >> bd]: the radius picked by the
//                         10-bit index (direction | radius << bd)
//   btab   1024 x 8 bf16  row idx = RNE_bf16(R[idx >> bd] * D[idx & mask][l])
//   perm   units*512 uint16  slot p takes input channel perm[p]; slots
//                         p >= k hold 0 (padding, multiplied by zero)
//   codes  n_tiles x units coded units of UNIT_BYTES each
//
// A coded unit covers 16 output rows x 64 consecutive codes (512 permuted
// input slots) and is laid out for one wavefront of 64 lanes.  Lane
// L = 4b + j (b = L >> 2, j = L & 3) owns 16 codes; its code i = 4*ri + ci
// (ri, ci in 0..3) sits in row 4*ri + j of the tile and code column
// 16*ci + b of the unit.  The four lanes 4b..4b+3 thus hold four rows of one
// code column, the shape of one block of v_mfma_f32_4x4x4_16b_f16 (the
// activations of that column are shared by the block), and a lane holds only
// four distinct code columns.  The 18 bits of the lane's 16 codes are split
// into three planes so that every lane reads them with three coalesced loads:
//
//   bytes    0..1023  sign plane: lane L's 16 bytes are dwords S0..S3;
//                     bit (15-i) of S_j = sign bit 2j of code i,
//                     bit (31-i) of S_j = sign bit 2j+1 of code i,
//                     so (S_j << i) carries the two signs of pair j of code
//                     i at the fp16/bf16 sign positions 15 and 31
//   bytes 1024..2047  index-low plane: byte i of lane L's 16 bytes = low 8
//                     bits of code i's 10-bit index (direction | radius<<bd)
//   bytes 2048..2303  index-high plane: bits 2i..2i+1 of lane L's dword =
//                     index bits 8..9 of code i
//
// 64 codes x 18 bits = 2304 bytes: the layout keeps 18 bits per 8 weights.
// Padding codes (rows >= n, slots >= k) are zero.
#pragma once
#include <stdint.h>
#include <stddef.h>
#include <hip/hip_runtime.h>

namespace svq {

constexpr int UNIT_ROWS = 16;
constexpr int UNIT_CODES = 64;
constexpr int UNIT_SLOTS = UNIT_CODES * 8;  // 512 permuted input slots
constexpr int UNIT_BYTES = 2304;
constexpr int PLANE_SIGN = 0;
constexpr int PLANE_LOW = 1024;
constexpr int PLANE_HIGH = 2048;
constexpr int DTAB_BYTES = 256 * 16;
constexpr int RTAB_BYTES = 1024 * 2;  // radius by 10-bit index, fp16
constexpr int BTAB_BYTES = 1024 * 16;
constexpr int XTAB_BYTES = 1024 * 32;
constexpr int EXACT_MAX_M = 4;    // m <= 4: exact fp32 decode path
constexpr int MAX_EXPERTS = 256;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---- per-wave load schedules, shared by the kernels and the host-side
// launch checks (every code address a wave loads is derived from these) ----
// Exact path, m = 2..4 (4-wave blocks): the wave's items are the flat units
// f = wv + k*4 < F of its block; a load for f past the block's last item
// reads the last item instead (never used), so loads stay inside the block.
__host__ __device__ inline int gv_wave_items(int F, int wv) { return F > wv ? (F - wv + 3) / 4 : 0; }
__host__ __device__ inline int gv_load_flat(int f, int F) { return f < F ? f : F - 1; }
// Exact path, m = 1 (fused, `waves` waves per block): the wave's items are
// [begin, end) of the block's n_items; a load past `end` reads the packed
// buffer's first bytes instead (unit -1 here: never used).
__host__ __device__ inline int gf_wave_begin(int n_items, int waves, int wv) { return wv * n_items / waves; }
__host__ __device__ inline int gf_load_unit(int u, int end) { return u < end ? u : -1; }

// Scratch of svq_linear_noalloc: a file-scope device array of this size
// (svq_scratch.hip); scratch_ptr returns the current device's address of it.
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
hipError_t scratch_ptr(void **ptr);

// Matrix view passed to kernels by value.
struct MatView {
  const uint8_t *base;  // packed buffer
  uint32_t off_dtab, off_rtab, off_btab, off_xtab, off_perm;
  uint64_t off_codes;
  int32_t n, k, bd;
  int32_t n_tiles, units;
};

// ---- dense path ---------------------------------------------------------
// Exact path, m = 2..4: a gather launch writes every matrix's permuted,
// per-unit scaled fp16 activations to the workspace (xg: row a of unit u at
// xg + (a*units + u) * GV_XG_UNIT_BYTES, 64 code columns x 8 slots; xs: the
// unit's 2^-e per row at xs[4*u + a]); one main launch then covers up to
// GV_MAX_JOBS matrices ("jobs"), a block owning R consecutive row tiles of
// one job.
constexpr int GV_MAX_JOBS = 8;
constexpr int GV_XG_UNIT_BYTES = UNIT_SLOTS * 2;  // one unit of one row, fp16
constexpr int GV_MAX_R = 4;                       // row tiles per main block
// First block of each job of one launch (job t owns blocks
// [first[t], first[t + 1])).  The starts sit in one 32-byte array at the
// head of the launch arguments, so a block finds its job with a single
// scalar load rather than a chain of dependent loads through the job records.
struct JobStarts {
  int32_t first[GV_MAX_JOBS];
};
struct GemvJob {
  MatView w;
  const uint16_t *x;
  int64_t ldx;
  uint8_t *xg;          // gathered activations (workspace)
  float *xs;            // their scales, [units][4]
  void *y;
  int64_t ldy;
  int32_t R;            // row tiles per main block
  int32_t block_begin;  // first main block of this job
};
struct GemvBatch {
  JobStarts starts;         // main launch
  JobStarts gather_starts;  // gather launch (4 waves per block, one per (row, unit))
  GemvJob job[GV_MAX_JOBS];
  int32_t count, m, ydt;
  int32_t red_off;          // LDS offset of the partial sums (after the tables)
  int32_t touch_begin;      // gather launch: first of the 8*count table-touch blocks
  int32_t xvec;             // every activation row starts 16-byte aligned
};
constexpr size_t GV_LDS_LIMIT = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int GV_WAVES = 4;
// lane-interleaved copies of a direction table of 2^bd rows (at most 32 KB)
__host__ __device__ constexpr int gv_copies(int bd) { return bd >= 8 ? 8 : 16; }
// LDS of the m = 2..4 main launch (absolute addresses): radius by 10-bit
// index, then the direction copies (2^bd rows of 256 bytes), then the
// cross-wave partial sums [R][GV_WAVES][4][4][4][M] fp32 at GemvBatch::red_off.
constexpr int GV_OFF_RTAB = 0;
constexpr int GV_OFF_D = RTAB_BYTES;
// Workspace of the exact path for one matrix of `units` units.
inline size_t gemv_ws_bytes(int m, int units) {
  return align256((size_t)m * units * GV_XG_UNIT_BYTES) + align256((size_t)units * 16);
}
// LDS of the main launch for the largest bd of its jobs and R <= r_max.
size_t gemv_smem_bytes(int m, int bd_max, int r_max);
hipError_t launch_gemv_batched(GemvBatch &b, int gather_blocks, int k_max, int blocks, size_t smem,
                               hipStream_t s);
constexpr int GV_UNITS_PER_WAVE = 4;  // units per wave the planner aims for
// m = 1: one fused launch (gather in the block); R <= GF_MAX_R row tiles
// per block, whose R x units items the 4 waves split into equal runs.
constexpr int GF_MAX_R = 8;
// LDS of the fused m = 1 block: the radius table (64 lane copies of the
// 2^(10-bd) fp32 radii) [0, gf_off_d(bd)); then the direction copies (bd <= 7: 16 copies
// of 2^bd rows at a 256-byte stride; bd = 8: 8 copies of 256 rows at a
// 128-byte stride, sharing their region with the activation staging row,
// which is dead once the gather is done; bd <= 7: the staging row follows the
// copies), so the staging row starts at a fixed offset for each bd and the
// gather's reads carry it as an instruction offset; then unit scales,
// cross-wave partial sums and the permuted activations.
constexpr int GF_OFF_R = 0;
__host__ __device__ constexpr int gf_off_d(int bd) { return 256 << (10 - bd); }  // after 2^(10-bd) radii x 64 lanes
__host__ __device__ constexpr int gf_dir_bytes(int bd) { return bd >= 8 ? 256 * 8 * 16 : (16 << bd) * 16; }
__host__ __device__ constexpr int gf_off_stage(int bd) { return bd >= 8 ? gf_off_d(bd) : gf_off_d(bd) + gf_dir_bytes(bd); }
struct GfLds {
  int scale, red, xp, stage, total;
};
// r: row tiles per block (the cross-wave partial sums hold r tiles)
__host__ __device__ inline GfLds gf_lds(int bd, int k, int units, int m, int r) {
  GfLds L;
  const int stage = (k * 2 + 15) & ~15, dir = gf_dir_bytes(bd);
  L.stage = gf_off_stage(bd);
  int off = bd >= 8 ? gf_off_d(bd) + (dir > stage ? dir : stage) : L.stage + stage;
  L.scale = off;
  off += (units * m * 4 + 15) & ~15;
  L.red = off;
  off += r * GV_WAVES * 4 * 4 * 4 * m;
  L.xp = off;
  off += units * UNIT_SLOTS * 2 * m;
  L.total = off;
  return L;
}
size_t gemv_fused_smem_bytes(int k, int units, int bd, int r);  // one matrix, r row tiles per block
hipError_t launch_gemv_fused(GemvBatch &b, int blocks, size_t smem, hipStream_t s);

// Small-batch path (EXACT_MAX_M < m <= SB_MAX_M): a prep launch writes
// every matrix's permuted activations as 16-row fp16 MFMA fragments with a
// power-of-two scale per (activation row, unit) (xa: unit u at
// xa + u * SB_XA_UNIT_BYTES; xs: the unit's 16 inverse scales at
// xs + 16 u), then one launch decodes each code straight into two 16x16x32
// fp16 MFMA operands, the halves of the exact split of R*D (xtab).  Work item = one coded unit of
// one row tile.  A block of SB_WAVES waves owns `tiles` consecutive row
// tiles and one K range of `upr` units (block lb of a job: group
// lb / splits, range lb % splits); its tiles x units items, unit-major, are
// cut into SB_WAVES contiguous runs, one per wave.  Matrices of more than
// SB_MAX_RANGE units are cut into `splits` K ranges whose fp32 partial
// tiles (part: [groups * tiles][splits][256]) are summed by the last block
// of the group to arrive (cnt: one arrival counter per group, cleared by the
// prep launch).
constexpr int SB_MAX_M = 16;
constexpr int SB_WAVES = 4;
constexpr int SB_TMAX = 6;       // row tiles per block, at most
constexpr int SB_NMAX = 8;       // items per wave, at most
constexpr int SB_ITEMS_MIN = 16; // items per block, at least (when the matrix allows)
constexpr int SB_MAX_RANGE = 8;  // units a block covers without a K split
constexpr int SB_XA_UNIT_BYTES = 16 * UNIT_SLOTS * 2;
struct SbJob {
  MatView w;
  const uint16_t *x;    // activations, bf16 [m][ldx]
  int64_t ldx;
  uint8_t *xa;          // fragment-ordered fp16 activations (workspace)
  float *xs;            // their inverse scales, [units][16] (workspace)
  float xinv;           // 2^-xscale_log2 of the matrix's exact split
  float *part;          // splits > 1: partial tiles (workspace)
  int32_t *cnt;         // splits > 1: arrival counters (workspace)
  void *y;
  int64_t ldy;
  int32_t tiles, upr;   // row tiles per block, units per K range
  int32_t groups, splits;
  int32_t block_begin;  // first main block of this job
  int32_t prep_begin;   // first prep block (4 per unit)
};
struct SbBatch {
  JobStarts starts, prep_starts;
  SbJob job[GV_MAX_JOBS];
  int32_t count, m, ydt;
};
// Block shape of one matrix: tiles per block, units per range, ranges,
// tile groups.  `items` = work items per block the call aims for
// (sb_block_items over all matrices of the call).
struct SbPlan {
  int tiles, upr, splits, groups;
};
int sb_block_items(int64_t total_items, int cus);
SbPlan sb_plan(int n_tiles, int units, int items);
// Workspace of one matrix on the small-batch path.
size_t sb_ws_bytes(int n_tiles, int units, int items);
hipError_t launch_sb(SbBatch &b, int prep_blocks, int blocks, hipStream_t s);

// Dequant-GEMM path (m > EXACT_MAX_M; "prefill" for m >= PREFILL_MIN_M, with
// 64-row block tiles below that): a prep launch writes the permuted
// activations of every matrix of the call ("jobs") in MFMA fragment order
// (xb, padded to prefill_m_pad(m) rows), then one LDS-tiled dequant-GEMM
// launch covers all jobs; a GEMM block owns one output tile of one job.
constexpr int PREFILL_MIN_M = 256;
constexpr int PREFILL_BN = 256;  // weight rows per GEMM block tile
struct PrefillJob {
  MatView w;
  const uint16_t *x;    // activations, bf16 [m][ldx]
  int64_t ldx;
  uint16_t *xb;         // permuted activations in fragment order (workspace)
  int32_t m;
  void *y;
  int64_t ldy;
  int32_t tiles_n;      // output tiles along n
  int32_t tiles_m;      // output tiles along m
  int32_t block_begin;  // first GEMM block of this job
  int32_t prep_begin;   // first prep block of this job
  int32_t prep_csplit;  // prep blocks per row group (chunk ranges)
  int32_t prep_rpb;     // activation rows per prep block (prefill_prep_rows(k))
  // K split (small m): GEMM block (mt, nt, sp) covers units
  // [sp * units_per_split, ...); with splits > 1 each writes an fp32 partial
  // tile to part[sp][m_pad][n_pad] and the reduce launch sums them into y
  int32_t splits, units_per_split;
  float *part;
  int32_t m_pad, n_pad;
  int32_t red_begin;    // first reduce block of this job
};
struct PrefillBatch {
  JobStarts gemm_starts, prep_starts, red_starts;  // copies of block/prep/red_begin
  PrefillJob job[GV_MAX_JOBS];
  int32_t count, ydt;
  int32_t yvec;  // every output row of every job starts 16-byte aligned
};
int prefill_bm(int m);      // activation rows per block tile: 256 (m >= PREFILL_MIN_M) or 64
int prefill_m_pad(int m);   // m rounded up to prefill_bm(m)
__host__ __device__ inline int prefill_tiles_n(int n_tiles) {
  return (n_tiles + PREFILL_BN / UNIT_ROWS - 1) / (PREFILL_BN / UNIT_ROWS);
}
int prefill_prep_rows(int k);  // activation rows per prep block for rows of k values
size_t prefill_prep_lds(int rpb, int k);  // LDS of such a block
// xvec: every activation row of every job starts 16-byte aligned.
hipError_t launch_prefill_prep(PrefillBatch &b, int blocks, size_t lds, bool xvec,
                               hipStream_t s);
hipError_t launch_prefill_batched(PrefillBatch &b, int bm, int blocks, hipStream_t s);
hipError_t launch_prefill_reduce(PrefillBatch &b, int blocks, hipStream_t s);

// ---- encoder ------------------------------------------------------------
// Tables of svq_encode as staged in the workspace: the codebook in float64
// (rows x 8), the squared midpoints of consecutive radii (float64) and the
// permutation.
struct EncArgs {
  const float *w;
  int64_t ldw;
  int32_t n, k, bd, n_mid;
  const double *cb;
  const double *msq;
  const int32_t *perm;
  uint8_t *codes;  // canonical stream
  int64_t count;   // n * k / 8 codes
  // optional activation-weighted reconstruction error of every code (err
  // non-null): the radius values (float64, n_mid + 1) and the per-channel
  // weights h [k]; err[g] for code g
  const double *rad;
  const double *h;
  double *err;
  // activation-weighted fit (non-null): the per-channel weights h [k] that
  // choose direction and radius jointly (rad must then be staged too)
  const double *fit_h;
};
hipError_t launch_encode(const EncArgs &a, hipStream_t s);

// ---- calibration: ESG energies and permutation, ABS error sums -----------
struct EsgArgs {
  const uint16_t *x;  // bf16 [t][ldx], 16-byte aligned rows
  int64_t t, ldx;
  int32_t k;
  double *energy;     // [k] out
  int32_t *rank;      // [k] scratch
  int32_t *perm;      // [k] out
};
hipError_t launch_esg(const EsgArgs &a, hipStream_t s);
// rows[c * n + i] = sequential sum over the C codes of row i of err (per
// candidate c, launched per candidate); totals[c] = sequential sum over rows
hipError_t launch_abs_rows(const double *err, int32_t n, int32_t C, double *rows, hipStream_t s);
hipError_t launch_abs_totals(const double *rows, int32_t n, int32_t n_cand, double *totals,
                             hipStream_t s);

// ---- MoE ----------------------------------------------------------------
struct ExpertTable {
  const uint8_t *base[MAX_EXPERTS];
  uint8_t bd[MAX_EXPERTS];
};

struct MoeShape {
  uint32_t off_dtab, off_rtab, off_btab, off_xtab, off_perm;
  uint64_t off_codes;
  int32_t n, k, n_tiles, units;
  int32_t num_experts;
};

// Projections of one svq_moe_linear_batched call that share the routing
// (the per-slot launch serves all of them; their experts fill one
// ExpertTable, projection c at entries c*E .. c*E + E - 1).
constexpr int MOE_BATCH_MAX = 4;
struct MoeGemvBatch {
  MoeShape sh[MOE_BATCH_MAX];
  const uint16_t *x[MOE_BATCH_MAX];
  int64_t ldx[MOE_BATCH_MAX];
  void *y[MOE_BATCH_MAX];
  int64_t ldy[MOE_BATCH_MAX];
  int32_t R[MOE_BATCH_MAX];  // row tiles per block
};

// Grouped MoE product (svq_moe.hip) for routed slots: activation rows per
// work item, workspace bytes of the fragment-ordered activations, and the
// prep + product launches over the routing's work list (expert, sorted rows
// r0..r1).  Up to MOE_FUSED_MAX_SLOTS slots the prep launch also does the
// routing (route.ids set): every prep block sorts the slots itself;
// projection 0's blocks write the work list and the sorted slots, and every
// projection's blocks zero their output rows of slots with invalid ids.
// Beyond that moe_route_kernel has written them (route.ids null, one
// projection per call).  The launches serve every projection of the batch
// (grid y), each with its own staged activations.
constexpr int MOE_SB_ROWS = 48;
constexpr int MOE_FUSED_MAX_SLOTS = 8192;
struct MoeRoute {
  const int32_t *ids;  // expert id per slot, or null when the work list is given
  int32_t slots;       // S = m * topk
  int32_t ydt;
};
struct MoeSbProj {  // one projection: its experts' layout, input, staging and output
  MoeShape sh;
  const uint16_t *x;
  int64_t ldx;
  uint8_t *xa;  // fragment-ordered activations (moe_sb_xa_bytes)
  void *y;
  int64_t ldy;
  int32_t rb;   // rows staged per pass of the prep launch
};
struct MoeSbBatch {
  MoeSbProj p[MOE_BATCH_MAX];
  int32_t count;
  int32_t vec;   // every x and ldx allow 16-byte loads
  int32_t yvec;  // every y and ldy allow 16-byte stores
};
size_t moe_sb_xa_bytes(int max_work, int units);
int moe_sb_prep_rb(int kp);
size_t moe_sb_prep_lds(int kp);
hipError_t launch_moe_sb(MoeSbBatch &b, const ExpertTable &tab, int x_per_slot, int topk,
                         const MoeRoute &route, int32_t *work, int32_t *nwork, int32_t *sorted,
                         int max_work, int ydt, hipStream_t s);

}  // namespace svq
