// Grouped mixture-of-experts product of libsvq for gfx950 (more slots than
// the per-slot GEMV takes).
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability".  Each expert matrix is a separately coded SVQ matrix (Fig. 2
// caption: signs, direction index and quantized radius per 8-weight
// subvector, split chosen per matrix); weights are rebuilt on demand inside
// the product (Fig. 1 / Fig. 5 captions) against the subvector's eight
// reordered activations (Fig. 6 caption).  The routing itself (top-k slots
// per token, slot q = t*topk + j) is this library's convention.
//
// The slots are sorted by expert into work items (each expert's rows split
// evenly into items of at most MOE_SB_ROWS rows): up to MOE_FUSED_MAX_SLOTS
// slots by every block of the prep launch for itself, beyond that by the
// separate moe_route_kernel.  Then two launches per call:
//
// * moe_sb_prep_kernel, block (work item, row group g of 16 rows): the
//   group's input rows are staged whole in LDS, then gathered through the
//   expert's permutation into bf16 fragments in the 16x16x32 MFMA order of
//   the small-batch path: unit u, fragment f = 4ci + q, lane L holds row
//   16g + (L & 15), the eight slots of code column 16ci + 4(L >> 4) + q.
//   Only the item's G = ceil(rows / 16) groups are written.
//
// * moe_sb_kernel, block (work item, group of MOE_SB_TILES row tiles), three
//   blocks per CU: each code of the expert's tiles is decoded once, straight
//   into a v_mfma_f32_16x16x32_bf16 B operand (the small-batch decode: the
//   expert's 1024-row table of RNE_bf16(R*D) rows, signs by XOR), and
//   multiplied with all G row groups.  The activation fragments stream
//   through a three-slot LDS ring, a quarter unit (fragments 4ci + q) per
//   slot, loaded into registers two slices ahead and written to the ring one
//   slice ahead; the last unit's padded half (k = 768) is skipped.  A wave owns
//   two row tiles and reads each activation fragment once for both.  The
//   block's outputs are staged in LDS and leave as 16-byte row pieces.
//   Blocks are mapped so that the column groups of one item share an XCD
//   (and its L2).
//
// Numerics as the dequant GEMM for many rows: weights RNE_bf16(R*D), bf16
// activations, fp32 accumulation, bf16 (RNE) or fp32 output.
#include <algorithm>
#include <type_traits>

#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

constexpr int MOE_SB_G = MOE_SB_ROWS / 16;    // row groups per work item, at most
constexpr int MOE_SB_TW = 2;                  // row tiles per wave
constexpr int MOE_SB_TILES = 4 * MOE_SB_TW;   // row tiles per block
constexpr int MOE_SB_GROUP_BYTES = 16 * 1024; // one row group of one unit (16 fragments of 1 KB)
constexpr int MOE_SB_SLICE_BYTES = MOE_SB_G * 4 * 1024;  // fragments 4ci + q of one unit, all groups
constexpr int MOE_SB_RING = 3;                // LDS slots of staged slices
constexpr int MOE_SB_PREP_LDS = 128 * 1024;   // staged rows of the prep launch, at most
constexpr int MOE_SB_PREP_THREADS = 1024;
constexpr int MOE_XCDS = 8;  // accelerator complex dies of the device, each with its own L2
// Staged row stride of the prep launch: kp bf16 plus 16 bytes, so that one
// column of 16 rows spans 16 distinct banks (kp is a multiple of 512).
__host__ __device__ __forceinline__ int moe_sb_prep_stride(int kp) { return 2 * kp + 16; }
// LDS: the bf16 table, then the ring of staged slices (three blocks per CU)
constexpr int MOE_SB_OFF_BTAB = 0;
constexpr int MOE_SB_OFF_A = BTAB_BYTES;
constexpr int MOE_SB_SMEM = MOE_SB_OFF_A + MOE_SB_RING * MOE_SB_SLICE_BYTES;
static_assert(3 * MOE_SB_SMEM <= 160 * 1024, "three blocks per CU");
// the output staging (MOE_SB_ROWS rows of 128 f32 columns plus padding) reuses the ring
static_assert(MOE_SB_ROWS * (128 * 4 + 16) <= MOE_SB_RING * MOE_SB_SLICE_BYTES, "output staging fits");
static_assert(MOE_SB_TILES * UNIT_ROWS == 128, "a block covers 128 output columns");


// Activation fragments of work item wi, unit u, row group g.
__host__ __device__ __forceinline__ size_t moe_sb_xa_off(int wi, int units, int u, int g) {
  return (((size_t)wi * units + u) * MOE_SB_G + g) * MOE_SB_GROUP_BYTES;
}

// Routing inside the prep launch (ROUTE): every block sorts the slots by
// expert itself, in the order moe_route_kernel's work list defines (experts
// ascending, each expert's rows split evenly into items of at most
// MOE_SB_ROWS rows) and, within an expert, by slot index, so that all blocks
// of an item find the same rows without talking to each other.  Thread t
// holds the ids of slots t*C .. t*C + C - 1 (C = ceil(S / threads) <=
// MOE_ROUTE_IDS) in registers.
constexpr int MOE_ROUTE_IDS = MOE_FUSED_MAX_SLOTS / MOE_SB_PREP_THREADS;
struct MoeRouteLds {
  int32_t cnt[MAX_EXPERTS];
  int32_t off[MAX_EXPERTS + 1];    // first sorted row of each expert
  int32_t items[MAX_EXPERTS + 1];  // first work item of each expert
  int32_t wsum[2][MAX_EXPERTS / 64];
  int32_t scan[MOE_SB_PREP_THREADS / 64];
  int32_t rows[MOE_SB_ROWS];       // slots of the block's item, in row order
  int32_t expert;
};

// Block (work item, row group g), MOE_SB_PREP_THREADS threads: the group's
// 16 activation rows are staged whole in LDS (rb rows per pass, coalesced
// 16-byte loads when x and ldx allow them; the row stride carries 16 bytes
// of padding so that the 16 rows of one column fall in distinct banks),
// then every fragment piece of every unit is gathered from LDS through the
// expert's permutation.  Wave w writes fragment group q = w & 3 of the units
// u = w >> 2 (mod MOE_SB_PREP_THREADS / 256): lane L owns row 16g + (L & 15)
// and the slots of code column 16ci + 4(L >> 4) + q.  Rows past the item and
// slots past k are zeros.  With ROUTE the block first does the routing
// (above); row group 0 of every item writes the item's work record and
// sorted slots for the product launch, block 0 the item count.
template <bool ROUTE>
__global__ __launch_bounds__(MOE_SB_PREP_THREADS) void moe_sb_prep_kernel(
    MoeSbBatch b, ExpertTable tab, int x_per_slot, int topk, MoeRoute route, int32_t *__restrict__ work,
    int32_t *__restrict__ nwork, int32_t *__restrict__ sorted) {
  constexpr int NT = MOE_SB_PREP_THREADS, USTEP = NT / 256;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ MoeRouteLds R;
  const int pc = blockIdx.y;  // projection
  const MoeSbProj &P = b.p[pc];
  const MoeShape &sh = P.sh;
  const uint16_t *__restrict__ x = P.x;
  const int64_t ldx = P.ldx;
  uint8_t *__restrict__ xa = P.xa;
  const int rb = P.rb, vec = b.vec;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63, s = L >> 4, rl = L & 15;
  const int wi = (int)blockIdx.x / MOE_SB_G, g = (int)blockIdx.x - wi * MOE_SB_G;
  int e, r0, rows;
  if constexpr (ROUTE) {
    const int S = route.slots, E = sh.num_experts;
    const int C = (S + NT - 1) / NT;  // <= MOE_ROUTE_IDS (host check)
    int my[MOE_ROUTE_IDS];
#pragma unroll
    for (int j = 0; j < MOE_ROUTE_IDS; ++j) {
      const int q = tid * C + j;
      my[j] = (j < C && q < S) ? route.ids[q] : -1;
    }
    for (int i = tid; i < E; i += NT) R.cnt[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MOE_ROUTE_IDS; ++j) {
      const int q = tid * C + j;
      if (my[j] >= 0 && my[j] < E) {
        atomicAdd(&R.cnt[my[j]], 1);
      } else if (j < C && q < S && q % (int)gridDim.x == (int)blockIdx.x) {
        // a slot with an id outside [0, E): its output row is zeros
        char *yr = (char *)P.y + (size_t)q * P.ldy * (route.ydt == 0 ? 2 : 4);
        for (int c = 0; c < sh.n; ++c) store_out(yr, (size_t)c, 0.f, route.ydt);
      }
    }
    __syncthreads();
    // exclusive scans of the slot counts and of the items per expert (threads
    // 0 .. MAX_EXPERTS-1, one expert each: within each wave, then the wave
    // totals)
    int cn = 0, it = 0, ci = 0, ii = 0;
    if (tid < MAX_EXPERTS) {
      cn = tid < E ? R.cnt[tid] : 0;
      it = (cn + MOE_SB_ROWS - 1) / MOE_SB_ROWS;
      ci = cn;
      ii = it;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int uc = __shfl_up(ci, d), ui = __shfl_up(ii, d);
        if (L >= d) {
          ci += uc;
          ii += ui;
        }
      }
      if (L == 63) {
        R.wsum[0][w] = ci;
        R.wsum[1][w] = ii;
      }
    }
    __syncthreads();
    if (tid < MAX_EXPERTS) {
      int bc = 0, bi = 0;
      for (int v = 0; v < w; ++v) {
        bc += R.wsum[0][v];
        bi += R.wsum[1][v];
      }
      if (tid < E) {
        R.off[tid] = bc + ci - cn;
        R.items[tid] = bi + ii - it;
      }
      if (tid == E - 1) {
        R.off[E] = bc + ci;
        R.items[E] = bi + ii;
      }
    }
    __syncthreads();
    const int nitems = R.items[E];
    if (pc == 0 && blockIdx.x == 0 && tid == 0) *nwork = nitems;
    if (wi >= nitems) return;  // block-uniform
    if (tid < E && R.items[tid] <= wi && wi < R.items[tid + 1]) R.expert = tid;
    __syncthreads();
    e = R.expert;
    const int n_items = R.items[e + 1] - R.items[e], cnt = R.cnt[e], c = wi - R.items[e];
    const int lo = (int)((int64_t)c * cnt / n_items), hi = (int)((int64_t)(c + 1) * cnt / n_items);
    r0 = R.off[e] + lo;
    rows = hi - lo;
    if (16 * g >= rows) return;  // block-uniform
    // rank of each of the expert's slots among them (slot order): the
    // thread's matches, then a block exclusive scan
    int mine = 0;
#pragma unroll
    for (int j = 0; j < MOE_ROUTE_IDS; ++j) mine += my[j] == e ? 1 : 0;
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (L >= d) incl += u;
    }
    if (L == 63) R.scan[w] = incl;
    __syncthreads();
    int rank = incl - mine;
    for (int v = 0; v < w; ++v) rank += R.scan[v];
#pragma unroll
    for (int j = 0; j < MOE_ROUTE_IDS; ++j) {
      if (my[j] == e) {
        if (rank >= lo && rank < hi) R.rows[rank - lo] = tid * C + j;
        ++rank;
      }
    }
    __syncthreads();
    if (pc == 0 && g == 0) {  // the routing is the same for every projection
      if (tid < rows) sorted[r0 + tid] = R.rows[tid];
      if (tid == 0) {
        work[3 * wi + 0] = e;
        work[3 * wi + 1] = r0;
        work[3 * wi + 2] = r0 + rows;
      }
    }
  } else {
    if (wi >= *nwork) return;  // block-uniform, before any barrier
    e = work[3 * wi];
    r0 = work[3 * wi + 1];
    rows = work[3 * wi + 2] - r0;
    if (16 * g >= rows) return;  // block-uniform
  }
  const int U = sh.units, kp = U * UNIT_SLOTS, k = sh.k;
  const int stride = moe_sb_prep_stride(kp);  // bytes per staged row
  const uint16_t *perm = (const uint16_t *)(tab.base[pc * sh.num_experts + e] + sh.off_perm);
  const int q = w & 3, u0 = w >> 2;
  const int chunks = kp / 8;  // 16-byte pieces of a staged row
  constexpr int BATCH = 4;

  for (int rb0 = 0; rb0 < 16; rb0 += rb) {
    __syncthreads();  // the previous pass's gathers are done
    const int nstage = rb * chunks;
    for (int c0 = 0; c0 < nstage; c0 += BATCH * NT) {
      u4 v[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        v[i] = (u4){0u, 0u, 0u, 0u};
        const int c = c0 + tid + NT * i;
        const int rr = c / chunks, cc = c - rr * chunks, row = 16 * g + rb0 + rr;
        if (c < nstage && row < rows && 8 * cc < k) {
          const int slot = ROUTE ? R.rows[row] : sorted[r0 + row];
          const uint16_t *xr = x + (int64_t)(x_per_slot ? slot : slot / topk) * ldx + 8 * cc;
          if (vec) {
            v[i] = *(const u4 *)xr;  // k is a multiple of 8
          } else {
#pragma unroll
            for (int l = 0; l < 4; ++l) v[i][l] = (uint32_t)xr[2 * l] | ((uint32_t)xr[2 * l + 1] << 16);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int c = c0 + tid + NT * i;
        const int rr = c / chunks, cc = c - rr * chunks;
        if (c < nstage) *(u4 *)(smem + (size_t)rr * stride + 16 * cc) = v[i];
      }
    }
    __syncthreads();
    if (rl < rb0 || rl >= rb0 + rb) continue;  // lane-uniform per pass; no barrier below
    const uint16_t *xrow = (const uint16_t *)(smem + (size_t)(rl - rb0) * stride);
    for (int u = u0; u < U; u += USTEP) {
      u4 pv[4];
#pragma unroll
      for (int ci = 0; ci < 4; ++ci)
        pv[ci] = *(const u4 *)(perm + u * UNIT_SLOTS + 8 * (16 * ci + 4 * s + q));
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const int p0 = u * UNIT_SLOTS + 8 * (16 * ci + 4 * s + q);
        u4 v;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          // perm entries are < k (zero past k), so every read is in the row
          const uint32_t lo = p0 + 2 * l < k ? xrow[pv[ci][l] & 0xFFFFu] : 0u;
          const uint32_t hi = p0 + 2 * l + 1 < k ? xrow[pv[ci][l] >> 16] : 0u;
          v[l] = lo | (hi << 16);
        }
        *(u4 *)(xa + moe_sb_xa_off(wi, U, u, g) + ((size_t)(4 * ci + q) * 64 + L) * 16) = v;
      }
    }
  }
}

// Table rows (RNE_bf16(R*D), 16 bytes by 10-bit index) of the codes
// ci = 0..NCI-1 of fragment group q.
template <int NCI>
__device__ __forceinline__ void moe_reads(const uint8_t *smem, uint32_t Lw, uint32_t H, const SbShifts &sh,
                                          u4 (&D)[4]) {
#pragma unroll
  for (int ci = 0; ci < NCI; ++ci) {
    // byte address (hi << 12) | (lo << 4) of the 16-byte row (hi << 8) | lo
    const uint32_t lo4 = __builtin_amdgcn_ubfe(Lw, 8 * ci, 8) << 4;
    const uint32_t hi = __builtin_amdgcn_ubfe(H, sh.hi[ci], 2);
    D[ci] = *(const u4 *)(smem + MOE_SB_OFF_BTAB + ((hi << 12) | lo4));
  }
}

// The code of fragment f = 4ci + q with its signs: a 64-bit shift of the
// record's sign dwords by 4b0 + ci brings the code's pair signs to bits 15
// and 31 of each dword.
__device__ __forceinline__ u4 moe_signed(const u4 &D, uint64_t S01, uint64_t S23, uint32_t sg) {
  const uint32_t SM = 0x80008000u;
  const uint64_t c01 = S01 << sg, c23 = S23 << sg;
  return (u4){D[0] ^ ((uint32_t)c01 & SM), D[1] ^ ((uint32_t)(c01 >> 32) & SM),
              D[2] ^ ((uint32_t)c23 & SM), D[3] ^ ((uint32_t)(c23 >> 32) & SM)};
}

// Workgroup barrier for the slice loop: this wave's LDS operations are
// complete, then s_barrier.  Outstanding global loads are not waited for:
// each is waited for (by the compiler, per register) where its data is
// used.  The memory clobber keeps every memory access on its side of the
// barrier.
__device__ __forceinline__ void moe_slice_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One block's product over G row groups (see moe_sb_kernel).  The unit
// loop runs in slices i = 4u + q (the fragments 4ci + q of unit u, all
// groups): slice i is multiplied from LDS ring slot i % 3.  Its fragments
// are loaded into registers during slice i - 2 and written to the slot
// during slice i - 1; one barrier per slice.  Codes are requested a whole
// unit ahead, slice by slice, into the registers each slice frees.
//
// Every global load here goes to registers, and the loads of one wave
// complete in the order they were issued, so the wait for a slice's
// fragments leaves the code loads issued after them in flight.  (With
// direct global-to-LDS loads the slice barrier had to wait for every
// outstanding load, codes included: those loads do not complete in order
// with the others, and nothing tracks their data per register.)
template <int G>
__device__ __forceinline__ void moe_sb_block(const MatView &w, int tg, int wi, int r0, int rows,
                                             const int32_t *__restrict__ sorted,
                                             const uint8_t *__restrict__ xa, void *__restrict__ y,
                                             int64_t ldy, int ydt, int yvec, uint8_t *smem) {
  const int U = w.units, NS = 4 * U;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the wave's row tiles (absolute); a tile past the matrix is not used
  // (its loads read the wave's first tile instead)
  const int tbase = tg * MOE_SB_TILES + MOE_SB_TW * wv;
  int tl[MOE_SB_TW];
  bool tv[MOE_SB_TW];
#pragma unroll
  for (int t = 0; t < MOE_SB_TW; ++t) {
    tv[t] = tbase + t < w.n_tiles;
    tl[t] = tv[t] ? tbase + t : min(tbase, w.n_tiles - 1);
  }
  const uint32_t s = lane >> 4, b0 = (lane >> 2) & 3, j = lane & 3;
  const uint32_t rec0 = 16 * s + j;
  const SbOffs offs = {16 * rec0, 16 * rec0 + 4 * b0, 4 * rec0};
  SbShifts shf;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    shf.sg[ci] = 4 * b0 + ci;
    shf.hi[ci] = 8 * b0 + 2 * ci;
  }
  // the record-q part of a unit's codes (what slice q reads): three loads per tile
  auto unit_codes_q = [&](SbCodes &c, int t, int u, int q) __attribute__((always_inline)) {
    const uint8_t *ub = w.base + w.off_codes + ((size_t)tl[t] * U + u) * UNIT_BYTES;
    c.S[q] = __builtin_nontemporal_load((const u4 *)(ub + PLANE_SIGN + 64 * q + offs.S));
    c.L[q] = __builtin_nontemporal_load((const uint32_t *)(ub + PLANE_LOW + 64 * q + offs.L));
    c.H[q] = __builtin_nontemporal_load((const uint32_t *)(ub + PLANE_HIGH + 16 * q + offs.H));
  };
  // slice i: wave wv moves fragment 4 wv + q of each group (G loads of
  // 1 KB per wave) into rA, then from rA into ring slot i % 3
  u4 rA[G];
  auto load_slice = [&](int i) __attribute__((always_inline)) {
    const int u = i >> 2, q = i & 3;
#pragma unroll
    for (int g = 0; g < G; ++g)
      rA[g] = *(const u4 *)(xa + moe_sb_xa_off(wi, U, u, g) + ((size_t)(4 * wv + q) * 64 + lane) * 16);
  };
  auto store_slice = [&](int i) __attribute__((always_inline)) {
    uint8_t *b = smem + MOE_SB_OFF_A + (i % MOE_SB_RING) * MOE_SB_SLICE_BYTES + wv * 1024 + lane * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) *(u4 *)(b + g * 4096) = rA[g];
  };

  // table, slice 0 and the first unit's codes requested first
  u4 bt[4];
  const u4 *gbt = (const u4 *)(w.base + w.off_btab);
#pragma unroll
  for (int i = 0; i < 4; ++i) bt[i] = gbt[tid + 256 * i];
  load_slice(0);
  SbCodes cd[MOE_SB_TW];
#pragma unroll
  for (int t = 0; t < MOE_SB_TW; ++t)
#pragma unroll
    for (int q = 0; q < 3; ++q) unit_codes_q(cd[t], t, 0, q);
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u4 *)(smem + MOE_SB_OFF_BTAB + 16 * (tid + 256 * i)) = bt[i];
  store_slice(0);
  load_slice(1);  // NS >= 4
  // the last record's codes after slice 1's loads, the order every slice
  // keeps: the compiler's wait for slice 1 at the loop head then leaves
  // them in flight (a different order on the way in would make it wait for
  // everything there)
#pragma unroll
  for (int t = 0; t < MOE_SB_TW; ++t) unit_codes_q(cd[t], t, 0, 3);

  f4 C[MOE_SB_TW][G];
#pragma unroll
  for (int t = 0; t < MOE_SB_TW; ++t)
#pragma unroll
    for (int g = 0; g < G; ++g) C[t][g] = (f4){0.f, 0.f, 0.f, 0.f};

  // One slice (unit u, fragment group q) with NCI of the unit's four column
  // groups: code columns 16ci .. 16ci + 15 hold input slots 512u + 128ci on,
  // so when the last unit's real slots end within its first half (k = 768:
  // 512 + 256) its groups 2 and 3 are padding (zero inputs) and are skipped.
  auto slice = [&](int u, auto Q, auto NCI) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value, nci = decltype(NCI)::value;
    const int i = 4 * u + q;
    const int un = min(u + 1, U - 1);
    // every wave's part of slice i is in LDS (written during slice i - 1),
    // and every wave is done with slice i - 2, whose slot (i + 1) % 3 is
    // written now
    moe_slice_barrier();
    if (i + 1 < NS) store_slice(i + 1);
    if (i + 2 < NS) load_slice(i + 2);
    const uint8_t *ab = smem + MOE_SB_OFF_A + (i % MOE_SB_RING) * MOE_SB_SLICE_BYTES;
    u4 D[MOE_SB_TW][4];
#pragma unroll
    for (int t = 0; t < MOE_SB_TW; ++t) moe_reads<nci>(smem, cd[t].L[q], cd[t].H[q], shf, D[t]);
    uint64_t S01[MOE_SB_TW], S23[MOE_SB_TW];
#pragma unroll
    for (int t = 0; t < MOE_SB_TW; ++t) {
      S01[t] = (uint64_t)cd[t].S[q][0] | ((uint64_t)cd[t].S[q][1] << 32);
      S23[t] = (uint64_t)cd[t].S[q][2] | ((uint64_t)cd[t].S[q][3] << 32);
      unit_codes_q(cd[t], t, un, q);
    }
#pragma unroll
    for (int ci = 0; ci < nci; ++ci) {
      u4 A[G];
#pragma unroll
      for (int g = 0; g < G; ++g) A[g] = *(const u4 *)(ab + (4 * g + ci) * 1024 + lane * 16);
#pragma unroll
      for (int t = 0; t < MOE_SB_TW; ++t) {
        const u4 B = moe_signed(D[t][ci], S01[t], S23[t], shf.sg[ci]);
#pragma unroll
        for (int g = 0; g < G; ++g)
          C[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, A[g]),
                                                            __builtin_bit_cast(b8, B), C[t][g], 0, 0, 0);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  const bool half_last = w.k - (U - 1) * UNIT_SLOTS <= UNIT_SLOTS / 2;  // block-uniform
  for (int u = 0; u < U - (half_last ? 1 : 0); ++u) {
    slice(u, I0(), I4());
    slice(u, I1(), I4());
    slice(u, I2(), I4());
    slice(u, I3(), I4());
  }
  if (half_last) {
    slice(U - 1, I0(), I2());
    slice(U - 1, I1(), I2());
    slice(U - 1, I2(), I2());
    slice(U - 1, I3(), I2());
  }

  // The outputs leave through LDS: the block's item rows x its 128 columns
  // n0 + nb (n0 = 128 tg), row stride padded by 16 bytes, then 16-byte pieces
  // of whole rows go to y.  Accumulator element i of lane L is activation
  // row 16g + 4(L >> 4) + i, column 16 (tile within the block) + (L & 15).
  // The output type is a template parameter of the store loops (a test per
  // element left a branch at every store).
  auto epi = [&](auto BF) __attribute__((always_inline)) {
    constexpr bool bf = decltype(BF)::value;
    constexpr int esz = bf ? 2 : 4;
    const int ostride = 128 * esz + 16;
    uint8_t *ob = smem + MOE_SB_OFF_A;
    __syncthreads();  // every wave is done with the staged activations
#pragma unroll
    for (int t = 0; t < MOE_SB_TW; ++t) {
      const int nb = 16 * (MOE_SB_TW * wv + t) + (lane & 15);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint8_t *o = ob + (16 * g + 4 * (int)s + i) * ostride;
          if constexpr (bf) *(uint16_t *)(o + 2 * nb) = f32_to_bf16_bits(C[t][g][i]);
          else *(float *)(o + 4 * nb) = C[t][g][i];
        }
    }
    __syncthreads();
    const int n0 = tg * (MOE_SB_TILES * UNIT_ROWS);
    constexpr int per = 16 / esz;  // elements per piece
    const int pieces = 128 / per, total = rows * pieces;
    constexpr int PER_THREAD = 16 * G * 32 / 256;  // pieces of 16 G rows of f32, per thread
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + 256 * i;
      const int r = c / pieces, pc = c - r * pieces, n = n0 + pc * per;
      if (c >= total || n >= w.n) continue;
      const int slot = sorted[r0 + r];
      const uint8_t *src = ob + r * ostride + pc * 16;
      uint8_t *dst = (uint8_t *)y + ((size_t)slot * ldy + n) * esz;
      if (yvec && n + per <= w.n) {
        *(u4 *)dst = *(const u4 *)src;
      } else {
        for (int e = 0; e < per && n + e < w.n; ++e)
          for (int b = 0; b < esz; ++b) dst[e * esz + b] = src[e * esz + b];
      }
    }
  };
  if (ydt == 0) epi(std::true_type());
  else epi(std::false_type());
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void moe_sb_kernel(
    MoeSbBatch b, ExpertTable tab, const int32_t *__restrict__ work, const int32_t *__restrict__ nwork,
    const int32_t *__restrict__ sorted, int ydt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int pc = blockIdx.y;  // projection
  const MoeSbProj &P = b.p[pc];
  const MoeShape &sh = P.sh;
  const uint8_t *__restrict__ xa = P.xa;
  void *__restrict__ y = P.y;
  const int64_t ldy = P.ldy;
  const int yvec = b.yvec;
  const int tgroups = (sh.n_tiles + MOE_SB_TILES - 1) / MOE_SB_TILES;
  // Blocks are dealt to the XCDs round-robin by index (block b runs on XCD
  // b % MOE_XCDS).  The active (item, column group) pairs are split into
  // MOE_XCDS contiguous shares, share x served by the blocks of XCD x, so an
  // item's column groups re-read its staged activations from one L2.
  const int active = *nwork * tgroups;
  const int share = (active + MOE_XCDS - 1) / MOE_XCDS;
  const int xcd = (int)blockIdx.x % MOE_XCDS, j = (int)blockIdx.x / MOE_XCDS;
  const int l = xcd * share + j;
  if (j >= share || l >= active) return;  // block-uniform, before any barrier
  const int wi = l / tgroups, tg = l - wi * tgroups;
  const int e = work[3 * wi], r0 = work[3 * wi + 1], rows = work[3 * wi + 2] - r0;
  const MatView w = expert_view(sh, tab, pc * sh.num_experts + e);
  switch ((rows + 15) >> 4) {  // block-uniform
    case 1: moe_sb_block<1>(w, tg, wi, r0, rows, sorted, xa, y, ldy, ydt, yvec, smem); break;
    case 2: moe_sb_block<2>(w, tg, wi, r0, rows, sorted, xa, y, ldy, ydt, yvec, smem); break;
    default: moe_sb_block<3>(w, tg, wi, r0, rows, sorted, xa, y, ldy, ydt, yvec, smem); break;
  }
}

size_t moe_sb_xa_bytes(int max_work, int units) { return moe_sb_xa_off(max_work, units, 0, 0); }

// Rows of a group staged per pass of the prep launch: all 16 when they fit
// the LDS budget, fewer for wide inputs (kp <= 65536 keeps it >= 1).
int moe_sb_prep_rb(int kp) {
  return std::max(1, std::min(16, MOE_SB_PREP_LDS / moe_sb_prep_stride(kp)));
}
size_t moe_sb_prep_lds(int kp) { return (size_t)moe_sb_prep_rb(kp) * moe_sb_prep_stride(kp); }

hipError_t launch_moe_sb(MoeSbBatch &b, const ExpertTable &tab, int x_per_slot, int topk,
                         const MoeRoute &route, int32_t *work, int32_t *nwork, int32_t *sorted,
                         int max_work, int ydt, hipStream_t s) {
  if (b.count < 1 || b.count > MOE_BATCH_MAX || (!route.ids && b.count != 1)) return hipErrorInvalidValue;
  size_t prep_lds = 0;
  int tgroups = 1;
  for (int c = 0; c < b.count; ++c) {
    const int kp = b.p[c].sh.units * UNIT_SLOTS;
    b.p[c].rb = moe_sb_prep_rb(kp);
    prep_lds = std::max(prep_lds, moe_sb_prep_lds(kp));
    tgroups = std::max(tgroups, (b.p[c].sh.n_tiles + MOE_SB_TILES - 1) / MOE_SB_TILES);
  }
  const dim3 pgrid(max_work * MOE_SB_G, b.count), pblock(MOE_SB_PREP_THREADS);
  hipError_t e;
  if (route.ids) {
    if (route.slots > MOE_FUSED_MAX_SLOTS || b.p[0].sh.num_experts < 1 || b.p[0].sh.num_experts > MAX_EXPERTS)
      return hipErrorInvalidValue;
    e = allow_smem(moe_sb_prep_kernel<true>, (int)prep_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_sb_prep_kernel<true>, pgrid, pblock, prep_lds, s, b, tab, x_per_slot, topk, route,
                       work, nwork, sorted);
  } else {
    e = allow_smem(moe_sb_prep_kernel<false>, (int)prep_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_sb_prep_kernel<false>, pgrid, pblock, prep_lds, s, b, tab, x_per_slot, topk,
                       route, work, nwork, sorted);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = allow_smem(moe_sb_kernel, MOE_SB_SMEM);
  if (e != hipSuccess) return e;
  // every projection's active pairs fit: the grid covers the widest one
  const int blocks = (max_work * tgroups + MOE_XCDS - 1) / MOE_XCDS * MOE_XCDS;
  hipLaunchKernelGGL(moe_sb_kernel, dim3(blocks, b.count), dim3(256), MOE_SB_SMEM, s, b, tab, work, nwork,
                     sorted, ydt);
  return hipGetLastError();
}

}  // namespace svq
