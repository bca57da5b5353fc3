// Small-batch dequant path of libsvq (EXACT_MAX_M < m <= SB_MAX_M) for
// gfx950.
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability".  A weight subvector is rebuilt on demand from its sign bits,
// direction index and radius index (Fig. 2 caption) inside the product
// (Fig. 1 / Fig. 5 captions) with the subvector's eight reordered
// activations (Fig. 6 caption).  The decoded weight R * D is never rounded:
// the matrix's 1024-row fp16 table (one row per 10-bit direction/radius
// index, built by svq_pack) holds hi and lo with hi + lo = R * D * 2^s
// exactly, and both halves, with the code's signs, are MFMA operands
// against the same fp16 activations (a power-of-two scale per activation
// row and unit, as in the m <= 4 path), so products and their sum are exact
// in the fp32 accumulators; 2^-s and the activation scales are applied to
// the fp32 sums.
//
// At a few activation rows the product is still bound by the code stream
// and by the per-code decode, not by the matrix cores, so the decoded
// weights never go through LDS: one code decodes to exactly two B operands
// of v_mfma_f32_16x16x32_f16 (8 consecutive k of one output column, hi and
// lo), in the lane that loaded it.
//
// 16x16x32 operands: lane L holds A row L & 15 and B column L & 15, both for
// k = 8(L >> 4)..+7; accumulator element i of lane L is row 4(L >> 4) + i,
// column L & 15.  With A = activations (row = activation row m) and
// B = weights (column = output row n of the 16-row tile) one MFMA covers one
// code of each of the 16 rows for four code columns.
//
// Code mapping.  The unit layout (svq_internal.h) gives lane 4b + j the
// codes 4ri + ci at row 4ri + j, code column 16ci + b.  The MFMA needs the
// 16 lanes of each k slice to hold one code column, so here lane
// L = 16s + 4b0 + j takes, for MFMA f = 4ci + q, the code at row 4b0 + j,
// column 16ci + 4s + q: code 4b0 + ci of lane record 16s + 4q + j.  It loads
// those records' bytes directly (for each q: the record's 16 sign bytes, the
// index-low dword b0 and the index-high dword), so no data moves between
// lanes; every byte of the unit is still fetched once per wave (lanes that
// share a record share the address).
//
// Activations: a prep launch writes every matrix's permuted activations in
// fragment order, unit by unit: 16 fragments of 1 KB (f = 4ci + q), lane L's
// 16 bytes = activation row L & 15 at the eight slots of code column
// 16ci + 4(L >> 4) + q, in fp16 after the row's power-of-two scale for the
// unit (largest magnitude scaled into [2^14, 2^15)).  A wave loads the 16
// fragments of its unit once (64 VGPRs) with the unit's inverse scales of
// its four accumulator rows, and reuses them for every row tile it covers.
//
// Work split.  A work item is one coded unit of one row tile.  A block of
// 4 waves owns up to SB_TMAX consecutive row tiles and a K range of units
// (the whole K unless the matrix has more than SB_MAX_RANGE units); its
// items, ordered unit by unit, are cut into 4 contiguous runs of at most
// SB_NMAX items, one per wave, so a wave reloads its activation fragments
// only when its run crosses to the next unit.  A wave streams its run with
// the codes of the next two items in flight and adds each item's 16 x 16
// result into its own LDS slot for the item's tile; after one barrier the
// block sums the four waves' slots in wave order.  For a matrix cut into K
// ranges the block writes fp32 partial tiles, and the last block of a tile
// group to arrive (an arrival counter, cleared by the prep launch) adds
// them in range order and writes the output, so results do not depend on
// timing.
#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

typedef __attribute__((address_space(3))) const u4 sb_lds_u4_t;

// LDS (absolute addresses; these kernels declare no static LDS): the fp16
// split table at 0, then the per-wave tile results, then the arrival flag.
constexpr int SB_OFF_XTAB = 0;
constexpr int SB_OFF_RED = XTAB_BYTES;
constexpr int SB_RED_BYTES = SB_WAVES * SB_TMAX * 1024;
constexpr int SB_OFF_FLAG = SB_OFF_RED + SB_RED_BYTES;
constexpr int SB_SMEM = SB_OFF_FLAG + 16;
static_assert(SB_SMEM <= 64 * 1024, "small-batch LDS");

__device__ __forceinline__ u4 sb_lds(uint32_t addr) { return *(sb_lds_u4_t *)(size_t)addr; }

// Table rows of the four codes (ci = 0..3) of MFMA group q: the hi and lo
// halves of each code's exact split (32-byte rows by 10-bit index).
__device__ __forceinline__ void sb_reads(uint32_t Lw, uint32_t H, const SbShifts &sh, u4 (&Dh)[4],
                                         u4 (&Dl)[4]) {
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const uint32_t lo = __builtin_amdgcn_ubfe(Lw, 8 * ci, 8);
    const uint32_t hi = __builtin_amdgcn_ubfe(H, sh.hi[ci], 2);
    const uint32_t a = SB_OFF_XTAB + ((lo | (hi << 8)) << 5);
    Dh[ci] = sb_lds(a);
    Dl[ci] = sb_lds(a + 16);
  }
}

// Signs of the four codes of group q, then their MFMAs.  A 64-bit shift of
// the record's sign dwords (S1:S0, S3:S2) by 4b0 + ci brings code
// 4b0 + ci's pair signs to bits 15 and 31 of each dword (bits the shift
// carries across the dword boundary land below bit 15 and are masked off).
__device__ __forceinline__ void sb_mul(uint64_t S01, uint64_t S23, const SbShifts &sh,
                                       const u4 (&Dh)[4], const u4 (&Dl)[4], const u4 (&A)[16], int q,
                                       f4 &C) {
  const uint32_t SM = 0x80008000u;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const uint64_t c01 = S01 << sh.sg[ci], c23 = S23 << sh.sg[ci];
    const uint32_t m0 = (uint32_t)c01 & SM, m1 = (uint32_t)(c01 >> 32) & SM;
    const uint32_t m2 = (uint32_t)c23 & SM, m3 = (uint32_t)(c23 >> 32) & SM;
    const u4 wh = {Dh[ci][0] ^ m0, Dh[ci][1] ^ m1, Dh[ci][2] ^ m2, Dh[ci][3] ^ m3};
    const u4 wl = {Dl[ci][0] ^ m0, Dl[ci][1] ^ m1, Dl[ci][2] ^ m2, Dl[ci][3] ^ m3};
    const h8 a = __builtin_bit_cast(h8, A[4 * ci + q]);
    C = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, wh), C, 0, 0, 0);
    C = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, wl), C, 0, 0, 0);
  }
}

// One unit of one row tile: the 16 codes of the lane, 16 MFMAs.
__device__ __forceinline__ f4 sb_item(const SbCodes &c, const u4 (&A)[16], const SbShifts &sh) {
  f4 C0 = {0.f, 0.f, 0.f, 0.f}, C1 = {0.f, 0.f, 0.f, 0.f};
  u4 H0[4], L0[4], H1[4], L1[4];
  auto s01 = [&](int q) { return (uint64_t)c.S[q][0] | ((uint64_t)c.S[q][1] << 32); };
  auto s23 = [&](int q) { return (uint64_t)c.S[q][2] | ((uint64_t)c.S[q][3] << 32); };
  // the table reads of group q + 1 are in flight while group q is multiplied
  sb_reads(c.L[0], c.H[0], sh, H0, L0);
  sb_reads(c.L[1], c.H[1], sh, H1, L1);
  __builtin_amdgcn_sched_barrier(0);
  sb_mul(s01(0), s23(0), sh, H0, L0, A, 0, C0);
  __builtin_amdgcn_sched_barrier(0);
  sb_reads(c.L[2], c.H[2], sh, H0, L0);
  __builtin_amdgcn_sched_barrier(0);
  sb_mul(s01(1), s23(1), sh, H1, L1, A, 1, C1);
  __builtin_amdgcn_sched_barrier(0);
  sb_reads(c.L[3], c.H[3], sh, H1, L1);
  __builtin_amdgcn_sched_barrier(0);
  sb_mul(s01(2), s23(2), sh, H0, L0, A, 2, C0);
  __builtin_amdgcn_sched_barrier(0);
  sb_mul(s01(3), s23(3), sh, H1, L1, A, 3, C1);
  return C0 + C1;
}

typedef __attribute__((address_space(3))) u4 sb_lds_u4w_t;
typedef __attribute__((address_space(3))) float sb_lds_f_t;
typedef __attribute__((address_space(3))) int sb_lds_i_t;

__device__ __forceinline__ const uint8_t *sb_unit(const MatView &w, int t, int u) {
  return w.base + w.off_codes + ((size_t)t * w.units + u) * UNIT_BYTES;
}

__global__ __launch_bounds__(256) void sb_gemm_kernel(SbBatch b) {
  const int jn = find_job(b.starts, b.count);
  const SbJob &J = b.job[jn];
  const MatView &w = J.w;
  const int lb = (int)blockIdx.x - J.block_begin;
  const int g = lb / J.splits, r = lb - g * J.splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = g * J.tiles, tn = min(J.tiles, w.n_tiles - t0);
  const int u0 = r * J.upr, ul = min(J.upr, w.units - u0);
  // this wave's run: items [i0, i0 + nk) of the block, item i = unit
  // u0 + i / tn, tile t0 + i % tn
  const int N = ul * tn;
  const int i0 = wv * N / SB_WAVES, nk = (wv + 1) * N / SB_WAVES - i0;
  const uint32_t s = lane >> 4, b0 = (lane >> 2) & 3, j = lane & 3;
  const uint32_t rec0 = 16 * s + j;
  const SbOffs offs = {16 * rec0, 16 * rec0 + 4 * b0, 4 * rec0};
  SbShifts sh;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    sh.sg[ci] = 4 * b0 + ci;
    sh.hi[ci] = 8 * b0 + 2 * ci;
  }
  const uint32_t slot0 = SB_OFF_RED + wv * SB_TMAX * 1024 + 16 * lane;

  // the bf16 table (requested first), the activation fragments of the
  // run's first unit and the codes of its first two items
  u4 bt[XTAB_BYTES / 4096];
  const u4 *gbt = (const u4 *)(w.base + w.off_xtab);
#pragma unroll
  for (int i = 0; i < XTAB_BYTES / 4096; ++i) bt[i] = gbt[tid + 256 * i];
  __builtin_amdgcn_sched_barrier(0);
  u4 A[16];
  f4 xsc;  // inverse activation scales of the lane's accumulator rows 4s..4s+3
  SbCodes cd[2];
  int ui = i0 / tn, ti = i0 - ui * tn;  // unit and tile of item k (relative)
  {
    // unconditional (a wave without items loads item i0 < N anyway), so
    // that only the table loads are waited for before the barrier
    const u4 *xa = (const u4 *)(J.xa + (size_t)(u0 + ui) * SB_XA_UNIT_BYTES) + lane;
#pragma unroll
    for (int f = 0; f < 16; ++f) A[f] = xa[64 * f];
    xsc = *(const f4 *)(J.xs + (size_t)(u0 + ui) * 16 + 4 * s);
    cd[0] = sb_load_codes(sb_unit(w, t0 + ti, u0 + ui), offs);
    const int i1 = min(i0 + 1, N - 1), u1 = i1 / tn;
    cd[1] = sb_load_codes(sb_unit(w, t0 + i1 - u1 * tn, u0 + u1), offs);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < SB_TMAX; ++t)
    *(sb_lds_u4w_t *)(size_t)(slot0 + t * 1024) = (u4){0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < XTAB_BYTES / 4096; ++i)
    *(sb_lds_u4w_t *)(size_t)(SB_OFF_XTAB + 16 * (tid + 256 * i)) = bt[i];
  __syncthreads();

#pragma unroll
  for (int k = 0; k < SB_NMAX; ++k) {
    if (k >= nk) break;
    if (k > 0 && ti == 0) {
      // the run enters the next unit
      const u4 *xa = (const u4 *)(J.xa + (size_t)(u0 + ui) * SB_XA_UNIT_BYTES) + lane;
#pragma unroll
      for (int f = 0; f < 16; ++f) A[f] = xa[64 * f];
      xsc = *(const f4 *)(J.xs + (size_t)(u0 + ui) * 16 + 4 * s);
    }
    const f4 C = sb_item(cd[k & 1], A, sh) * xsc;
    if (k + 2 < nk) {
      const int i2 = i0 + k + 2, u2 = i2 / tn;
      cd[k & 1] = sb_load_codes(sb_unit(w, t0 + i2 - u2 * tn, u0 + u2), offs);
    }
    sb_lds_u4w_t *sl = (sb_lds_u4w_t *)(size_t)(slot0 + ti * 1024);
    *sl = __builtin_bit_cast(u4, __builtin_bit_cast(f4, *sl) + C);
    if (++ti == tn) {
      ti = 0;
      ++ui;
    }
  }
  __syncthreads();

  // sum of the four waves' slots of each tile, in wave order.  Thread tid
  // takes output row n = tid & 15 of the tile for activation row
  // m = tid >> 4: accumulator element m & 3 of lane 16(m >> 2) + n.
  const int m = tid >> 4, nn = tid & 15;
  const uint32_t eoff = SB_OFF_RED + 256 * (m >> 2) + 16 * nn + 4 * (m & 3);
  float acc[SB_TMAX];
#pragma unroll
  for (int t = 0; t < SB_TMAX; ++t) {
    acc[t] = 0.f;
#pragma unroll
    for (int ww = 0; ww < SB_WAVES; ++ww)
      acc[t] += *(sb_lds_f_t *)(size_t)(eoff + (ww * SB_TMAX + t) * 1024);
  }
  if (J.splits > 1) {
    // Partial tiles for the range, then the arrival count of the group.
    // The partials are written and read as device-scope atomics (coherent
    // between the XCDs' L2 caches without writing back or invalidating
    // them, which a device-scope fence does), and every partial store has
    // completed (vmcnt 0, then the barrier) before the count is raised.
    float *pt = J.part + ((size_t)t0 * J.splits + r) * 256 + tid;
#pragma unroll
    for (int t = 0; t < SB_TMAX; ++t)
      if (t < tn)
        __hip_atomic_store(pt + (size_t)t * J.splits * 256, acc[t], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const int prev = __hip_atomic_fetch_add(J.cnt + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *(sb_lds_i_t *)(size_t)SB_OFF_FLAG = prev == J.splits - 1 ? 1 : 0;
    }
    __syncthreads();
    if (*(sb_lds_i_t *)(size_t)SB_OFF_FLAG == 0) return;
    // all partials of a batch of 8 ranges are requested before any is added
    const float *pa = J.part + (size_t)t0 * J.splits * 256 + tid;
#pragma unroll
    for (int t = 0; t < SB_TMAX; ++t) acc[t] = 0.f;
    for (int r0 = 0; r0 < J.splits; r0 += 8) {
      float v[SB_TMAX][8];
#pragma unroll
      for (int t = 0; t < SB_TMAX; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = min(r0 + e, J.splits - 1), tt = min(t, tn - 1);
          v[t][e] = __hip_atomic_load(pa + ((size_t)tt * J.splits + rr) * 256, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
      for (int t = 0; t < SB_TMAX; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (r0 + e < J.splits) acc[t] += v[t][e];
    }
  }
  if (m >= b.m) return;
#pragma unroll
  for (int t = 0; t < SB_TMAX; ++t) {
    const int n = (t0 + t) * UNIT_ROWS + nn;
    if (t < tn && n < w.n) store_out(J.y, (size_t)m * J.ldy + n, acc[t] * J.xinv, b.ydt);
  }
  (void)j;
}

// Prep: the permuted activations of every job in fragment order (see the
// file comment), rows >= m and slots >= k zero; block u of a job writes the
// 16 fragments of unit u, thread tid the 16-byte pieces of fragments
// 4 (tid >> 6) .. + 3 for lane tid & 63 (activation row tid & 15).  Each
// activation row's largest magnitude over the unit (512 slots) sets its
// power-of-two scale 2^e (max * 2^e in [2^14, 2^15)): a bf16 value of at
// least 2^-31 times the maximum is then exact in fp16.  2^-e goes to
// xs[16u + row].  The first block of a job also clears the job's arrival
// counters.
__global__ __launch_bounds__(256) void sb_prep_kernel(SbBatch b) {
  __shared__ float s_max[4][16];
  const int jn = find_job(b.prep_starts, b.count);
  const SbJob &J = b.job[jn];
  const MatView &w = J.w;
  const int u = (int)blockIdx.x - J.prep_begin;
  const int tid = threadIdx.x, wv = tid >> 6, L = tid & 63;
  if (u == 0 && J.cnt)
    for (int i = tid; i < J.groups; i += 256) J.cnt[i] = 0;
  const int m = L & 15, s = L >> 4;
  float v[4][8];
  float mx = 0.f;
#pragma unroll
  for (int ff = 0; ff < 4; ++ff) {
    const int f = 4 * wv + ff, ci = f >> 2, q = f & 3;
    const int p0 = u * UNIT_SLOTS + 8 * (16 * ci + 4 * s + q);
#pragma unroll
    for (int l = 0; l < 8; ++l) v[ff][l] = 0.f;
    if (m < b.m && p0 < w.k) {
      // perm is zero padded to the unit width, so every index is < k
      const u4 pv = *(const u4 *)(w.base + w.off_perm + 2 * (size_t)p0);
      const uint16_t *xr = J.x + (int64_t)m * J.ldx;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const float lo = bf16_bits_to_f32(xr[pv[l] & 0xFFFFu]), hi = bf16_bits_to_f32(xr[pv[l] >> 16]);
        v[ff][2 * l] = p0 + 2 * l < w.k ? lo : 0.f;
        v[ff][2 * l + 1] = p0 + 2 * l + 1 < w.k ? hi : 0.f;
      }
    }
#pragma unroll
    for (int l = 0; l < 8; ++l) mx = fmaxf(mx, fabsf(v[ff][l]));
  }
  // row maximum: the lanes of one row (m, m + 16, m + 32, m + 48), then the waves
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (L < 16) s_max[wv][L] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_max[0][m], s_max[1][m]), fmaxf(s_max[2][m], s_max[3][m]));
  const int e = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
  for (int ff = 0; ff < 4; ++ff) {
    const int f = 4 * wv + ff;
    u4 h;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const _Float16 lo = (_Float16)ldexpf(v[ff][2 * l], e), hi = (_Float16)ldexpf(v[ff][2 * l + 1], e);
      h[l] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *(u4 *)(J.xa + ((size_t)u * 16 + f) * 1024 + 16 * L) = h;
  }
  if (tid < 16) J.xs[(size_t)u * 16 + tid] = ldexpf(1.f, -e);
}

hipError_t launch_sb(SbBatch &b, int prep_blocks, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(sb_prep_kernel, dim3(prep_blocks), dim3(256), 0, s, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sb_gemm_kernel, dim3(blocks), dim3(256), SB_SMEM, s, b);
  return hipGetLastError();
}

}  // namespace svq
