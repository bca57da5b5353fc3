// Prefill dequant-GEMM of libsvq (m >= PREFILL_MIN_M) for gfx950.
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability".  Weights are rebuilt on demand (Fig. 1 and Fig. 5 captions)
// from sign bits, a direction index and a quantized radius (Fig. 2 caption)
// and multiply reordered activations (Fig. 6 caption); at prefill sizes the
// product is a dense contraction, so the decoded tile feeds the matrix cores.
//
// One launch covers every matrix of a call ("jobs", longest k first).  A
// block computes a P_BM x P_BN output tile (activation rows x weight rows)
// over K in steps of P_BK = 64 permuted slots (8 codes per weight row).  The
// decoded weight tile of each step, RNE_bf16(R*D) with the signs applied,
// goes through LDS (two stages: the next step's decode overlaps the current
// step's MFMAs, one barrier per step).  The activations never touch LDS: a
// prep launch writes the permuted activations in MFMA fragment order (see
// prefill_prep_kernel), so each wave loads its A fragments straight into
// registers with fully coalesced 1 KB loads, one step ahead.  Four waves in
// a 2 x 2 grid each own a 128 x 128 tile: 16 accumulators of
// v_mfma_f32_32x32x16_bf16 (held in accumulation registers; this
// translation unit is built without the VGPR-form MFMA option of the
// exact-path kernels).  B fragments of the next 16-wide k substep are read
// while the current one's MFMAs run.
//
// 32x32x16 operands: lane L holds row L & 31 of a 32-row fragment and
// k = 8(L >> 5)..+7; accumulator element e of lane L is row
// (e & 3) + 8(e >> 2) + 4(L >> 5), column L & 31.
//
// Decode mapping (unit layout in svq_internal.h): K-step t of a unit covers
// code columns 8t..8t+7, i.e. ci = t >> 1 and b in 8(t & 1) + [0, 8).
// Thread tau handles, for row tiles (tau >> 5) and (tau >> 5) + 8, lane
// record 4b + j (b = 8(t & 1) + ((tau & 31) >> 2), j = tau & 3): its four
// codes 4*ri + ci sit in rows 4*ri + j, column b - 8(t & 1) of the step.  A
// thread needs four records per unit (two row tiles x two halves); those of
// the next unit are loaded during the last two steps of the current one.
#include <type_traits>

#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

constexpr int P_BN = 256, P_BK = 64;
constexpr int P_ROW = P_BK * 2;                  // 128 bytes per LDS row
constexpr int P_B = P_BN * P_ROW;                // weight tile, 32 KB
constexpr int P_STAGE = P_B;
constexpr int P_OFF_BTAB = 2 * P_STAGE;
constexpr int P_SMEM = P_OFF_BTAB + BTAB_BYTES;  // 80 KB
static_assert(P_SMEM <= 160 * 1024, "prefill LDS exceeds a workgroup's 160 KB");

// Fragment order of the permuted activations xb (per job, m_pad x Kp bf16):
// the 1 KB block F(rb, s, ks) holds, for 32-row block rb, K-step s and k
// substep ks, lane L's eight values (row 32rb + (L & 31), slots
// 64s + 16ks + 8(L >> 5) + 0..7) at bytes 16L..16L+15 -- exactly one
// 32x32x16 A fragment -- and the blocks are ordered (rb, s, ks).
__device__ __forceinline__ size_t xb_frag_offset(int r, int p, int S) {
  const int rb = r >> 5, s = p >> 6, ks = (p >> 4) & 3, L = (r & 31) + 32 * ((p >> 3) & 1);
  return ((((size_t)rb * S + s) * 4 + ks) * 64 + L) * 8 + (p & 7);
}

// LDS tiles hold rows of 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ swz(r).  With swz(r) = (r >> 1) & 7 the 16 consecutive rows a
// fragment read touches at one chunk fall in 16 distinct bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r >> 1) & 7u; }

// Decode the four codes of column group CI of one lane record: table rows
// first (all reads before any write: the writes could alias them), then the
// signed rows into the weight tile.  Row of code ri: row0 + 4*ri; chunk bl.
template <int CI>
__device__ __forceinline__ void p_decode(const ItemCodes &c, const uint8_t *s_btab, uint8_t *tile,
                                         int row0, int bl, u4 (&v)[4]) {
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    const int i = 4 * ri + CI;
    const uint32_t idx = ((c.L[ri] >> (8 * CI)) & 0xFFu) | (((c.H >> (2 * i)) & 3u) << 8);
    v[ri] = *(const u4 *)(s_btab + 16 * idx);
  }
}
// Sign carrier S << I, computed where it is used: as plain C the 128
// carriers of a unit are all computed at its start and spilled.
template <int I>
__device__ __forceinline__ uint32_t carrier(uint32_t S) {
  if (I == 0) return S;
  uint32_t r;
  asm volatile("v_lshlrev_b32 %0, %1, %2" : "=v"(r) : "i"(I), "v"(S));
  return r;
}

template <int CI>
__device__ __forceinline__ void p_store(const ItemCodes &c, uint8_t *tile, int row0, int bl,
                                        u4 (&v)[4]) {
  const uint32_t SM = 0x80008000u;
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    const int i = 4 * ri + CI;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t cr;
      switch (ri) {
        case 0: cr = carrier<CI>(c.S[q]); break;
        case 1: cr = carrier<4 + CI>(c.S[q]); break;
        case 2: cr = carrier<8 + CI>(c.S[q]); break;
        default: cr = carrier<12 + CI>(c.S[q]); break;
      }
      v[ri][q] ^= cr & SM;
    }
    const int r = row0 + 4 * ri;
    *(u4 *)(tile + r * P_ROW + ((bl ^ swz(r)) << 4)) = v[ri];
  }
}

// BM = 256: four waves in a 2 x 2 grid of 128 x 128 tiles, one block per CU.
// BM = 64 (activation row counts below 256): four waves side by side, each
// 64 x 64, with a register budget for two blocks per CU.
template <int BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BM == 256 ? 1 : 2, BM == 256 ? 1 : 2)))
void prefill_batched_kernel(PrefillBatch b) {
  constexpr int WM = BM == 256 ? 2 : 1, WN = 4 / WM;  // wave grid
  constexpr int TM = BM / WM, TN = P_BN / WN;         // wave tile
  constexpr int NI = TM / 32, NJ = TN / 32;           // 32 x 32 accumulator blocks
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int jn = 0;
  while (jn + 1 < b.count && (int)blockIdx.x >= b.job[jn + 1].block_begin) ++jn;
  const PrefillJob &J = b.job[jn];
  const MatView &w = J.w;
  // Blocks are dealt to the 8 XCDs round-robin (block i on XCD i % 8) and
  // each XCD has its own L2: with m-tile = local % tiles_m, the blocks that
  // share one 256-row activation tile run on the same XCD (when tiles_m
  // divides 8 or is a multiple of it and jobs start on multiples of 8), so
  // that tile is fetched into one L2 and reused there.
  const int local = (int)blockIdx.x - J.block_begin;
  if (local >= J.tiles_n * J.tiles_m * J.splits) return;  // padding block (uniform, before any barrier)
  const int mt = local % J.tiles_m, nt = (local / J.tiles_m) % J.tiles_n;
  const int sp = local / (J.tiles_m * J.tiles_n);  // K split: units [u0, u1)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / WN, wn = wv % WN;
  const int U = w.units, Kp = U * UNIT_SLOTS;
  const int u0 = sp * J.units_per_split, u1 = min(U, u0 + J.units_per_split);
  const int rt0 = nt * (P_BN / UNIT_ROWS);
  const int m0 = mt * BM;

  uint8_t *s_btab = smem + P_OFF_BTAB;
  for (int j = tid; j < 1024; j += 256) ((u4 *)s_btab)[j] = ((const u4 *)(w.base + w.off_btab))[j];

  // A fragments of the wave: 32-row blocks rb = m0/32 + NI*wm + i; step s,
  // substep ks at a_ptr[i] + s * 2048 + ks * 512 elements (one 1 KB block)
  const int S = Kp / P_BK;
  const uint16_t *a_ptr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
    a_ptr[i] = J.xb + ((size_t)((m0 >> 5) + NI * wm + i) * S * 4 * 64 + lane) * 8;
  // weight tile: row tiles rtl and rtl + 8 (clamped to the matrix; rows past
  // n are decoded from the last tile and never stored)
  const int rtl = tid >> 5, bl = (tid & 31) >> 2, jr = tid & 3;
  const int rtA = min(rt0 + rtl, w.n_tiles - 1), rtB = min(rt0 + rtl + 8, w.n_tiles - 1);
  const uint8_t *codesA = w.base + w.off_codes + (size_t)rtA * U * UNIT_BYTES;
  const uint8_t *codesB = w.base + w.off_codes + (size_t)rtB * U * UNIT_BYTES;
  const int rec0 = 4 * bl + jr, rec1 = rec0 + 32;
  const int rowA = rtl * UNIT_ROWS + jr;
  const int rowB = rowA + 8 * UNIT_ROWS;

  f16x C[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) C[i][j] = (f16x){};

  // records of the current unit: [row tile A/B][half 0/1]
  const size_t cu0 = (size_t)u0 * UNIT_BYTES;
  ItemCodes r00 = load_item(codesA + cu0, rec0), r01 = load_item(codesA + cu0, rec1);
  ItemCodes r10 = load_item(codesB + cu0, rec0), r11 = load_item(codesB + cu0, rec1);
  // A fragments of the first step: af[ks][i]
  u4 af[4][NI];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int i = 0; i < NI; ++i) af[ks][i] = *(const u4 *)(a_ptr[i] + (size_t)u0 * 8 * 2048 + ks * 512);
  __syncthreads();  // btab
  {
    u4 va[4], vb[4];
    p_decode<0>(r00, s_btab, smem, rowA, bl, va);
    p_decode<0>(r10, s_btab, smem, rowB, bl, vb);
    p_store<0>(r00, smem, rowA, bl, va);
    p_store<0>(r10, smem, rowB, bl, vb);
  }
  __syncthreads();

  // B fragment rows: 32j + (lane & 31) of the wave's weight rows; the chunk
  // of k substep ks is 2ks + (lane >> 5), stored at that ^ swz(row), and
  // swz(row) = ((lane & 31) >> 1) & 7 for every fragment
  const int sl = ((lane & 31) >> 1) & 7, hl = lane >> 5;
  const int b_frag = (TN * wn + (lane & 31)) * P_ROW;

  for (int u = u0; u < u1; ++u) {
    // records of the next unit (the last unit reloads itself): half 0 is
    // first needed by step 7's decode and loaded at step 6, after the
    // current half 0 was last used; half 1 is loaded at step 7
    const size_t nu = (size_t)min(u + 1, u1 - 1) * UNIT_BYTES;
    ItemCodes n00, n01, n10, n11;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t == 6) {
        n00 = load_item(codesA + nu, rec0);
        n10 = load_item(codesB + nu, rec0);
      }
      if (t == 7) {
        n01 = load_item(codesA + nu, rec1);
        n11 = load_item(codesB + nu, rec1);
      }
      // One K-step is one branch-free region: the next step's A fragment
      // loads (clamped on the last step: a harmless reload), table reads,
      // signed stores and B fragment reads are interleaved with this step's
      // 64 MFMAs (sched_group_barrier), so they run in the MFMA shadow.
      const int sn = min(u * 8 + t + 1, 8 * u1 - 1);
      const uint8_t *cur = smem + (t & 1) * P_STAGE;
      uint8_t *nxt = smem + ((t + 1) & 1) * P_STAGE;
      u4 va[4], vb[4];
      u4 bf[2][NJ];
      {
        const int pos = ((hl ^ sl) << 4);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[0][j] = *(const u4 *)(cur + b_frag + j * 32 * P_ROW + pos);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < P_BK / 16; ++ks) {
        const int c = ks & 1;
        if (ks + 1 < P_BK / 16) {
          const int pos = (((2 * (ks + 1) + hl) ^ sl) << 4);
#pragma unroll
          for (int j = 0; j < NJ; ++j) bf[c ^ 1][j] = *(const u4 *)(cur + b_frag + j * 32 * P_ROW + pos);
        }
        if (ks == 0) {
          switch (t) {  // table rows of the next step's decode
            case 0: p_decode<0>(r01, s_btab, nxt, rowA, bl, va); p_decode<0>(r11, s_btab, nxt, rowB, bl, vb); break;
            case 1: p_decode<1>(r00, s_btab, nxt, rowA, bl, va); p_decode<1>(r10, s_btab, nxt, rowB, bl, vb); break;
            case 2: p_decode<1>(r01, s_btab, nxt, rowA, bl, va); p_decode<1>(r11, s_btab, nxt, rowB, bl, vb); break;
            case 3: p_decode<2>(r00, s_btab, nxt, rowA, bl, va); p_decode<2>(r10, s_btab, nxt, rowB, bl, vb); break;
            case 4: p_decode<2>(r01, s_btab, nxt, rowA, bl, va); p_decode<2>(r11, s_btab, nxt, rowB, bl, vb); break;
            case 5: p_decode<3>(r00, s_btab, nxt, rowA, bl, va); p_decode<3>(r10, s_btab, nxt, rowB, bl, vb); break;
            case 6: p_decode<3>(r01, s_btab, nxt, rowA, bl, va); p_decode<3>(r11, s_btab, nxt, rowB, bl, vb); break;
            default: p_decode<0>(n00, s_btab, nxt, rowA, bl, va); p_decode<0>(n10, s_btab, nxt, rowB, bl, vb); break;
          }
        }
        if (ks == 1) {
          switch (t) {
            case 0: p_store<0>(r01, nxt, rowA, bl, va); break;
            case 1: p_store<1>(r00, nxt, rowA, bl, va); break;
            case 2: p_store<1>(r01, nxt, rowA, bl, va); break;
            case 3: p_store<2>(r00, nxt, rowA, bl, va); break;
            case 4: p_store<2>(r01, nxt, rowA, bl, va); break;
            case 5: p_store<3>(r00, nxt, rowA, bl, va); break;
            case 6: p_store<3>(r01, nxt, rowA, bl, va); break;
            default: p_store<0>(n00, nxt, rowA, bl, va); break;
          }
        }
        if (ks == 2) {
          switch (t) {
            case 0: p_store<0>(r11, nxt, rowB, bl, vb); break;
            case 1: p_store<1>(r10, nxt, rowB, bl, vb); break;
            case 2: p_store<1>(r11, nxt, rowB, bl, vb); break;
            case 3: p_store<2>(r10, nxt, rowB, bl, vb); break;
            case 4: p_store<2>(r11, nxt, rowB, bl, vb); break;
            case 5: p_store<3>(r10, nxt, rowB, bl, vb); break;
            case 6: p_store<3>(r11, nxt, rowB, bl, vb); break;
            default: p_store<0>(n10, nxt, rowB, bl, vb); break;
          }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            C[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, af[ks][i]),
                                                              __builtin_bit_cast(b8, bf[c][j]),
                                                              C[i][j], 0, 0, 0);
        // the next step's A fragments of this substep, into the registers
        // these MFMAs just read
#pragma unroll
        for (int i = 0; i < NI; ++i) af[ks][i] = *(const u4 *)(a_ptr[i] + (size_t)sn * 2048 + ks * 512);
        // Interleave: the next substep's B fragment reads (and, in substep
        // 0, the table reads) first, then MFMAs alternating with the A
        // loads and the step's vector work and stores.
        if (ks + 1 < P_BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, NJ, 0);  // DS reads
        if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // table reads
#pragma unroll
        for (int g = 0; g < NI * NJ / 2; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
          if (g == NI * NJ / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x020, NI, 0);  // VMEM reads (A)
          if (ks == 1 || ks == 2) {
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU (signs)
            if (g & 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    }
    r00 = n00;
    r01 = n01;
    r10 = n10;
    r11 = n11;
  }

  // Epilogue through LDS (the weight stages are free now): each wave turns
  // its TM x TN accumulator tile into output-type rows in a private 16 KB
  // region, as many 32-row blocks per pass as fit, and writes them back as
  // whole 16-byte pieces of consecutive output columns.
  __syncthreads();
  {
    uint8_t *s_c = smem + wv * 16384;
    // destination: y, or this split's fp32 partial tile (summed by the
    // reduce launch) when K is split
    const bool split = J.splits > 1;
    void *const ybase = split ? (void *)(J.part + (size_t)sp * J.m_pad * J.n_pad) : J.y;
    const int64_t yld = split ? J.n_pad : J.ldy;
    const int nlim = split ? J.n_pad : w.n;
    const bool yv = split || b.yvec;
    const bool bf = !split && b.ydt == 0;
    const int esz = bf ? 2 : 4;
    const int ipp = min(NI, 16384 / (32 * TN * esz));  // 32-row blocks per pass
    const int cpr = TN * esz / 16;                      // 16-byte pieces per row
    const int per = 16 / esz;                           // columns per piece
#pragma unroll
    for (int i0 = 0; i0 < NI; ++i0) {
      if (i0 % ipp != 0) continue;
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        if (ii >= ipp || i0 + ii >= NI) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 32 * ii + (e & 3) + 8 * (e >> 2) + 4 * (lane >> 5), c = 32 * j + (lane & 31);
            const float val = C[i0 + ii][j][e];
            if (bf) ((uint16_t *)s_c)[r * TN + c] = f32_to_bf16_bits(val);
            else ((float *)s_c)[r * TN + c] = val;
          }
      }
      __syncthreads();
      for (int q = lane; q < 32 * ipp * cpr; q += 64) {
        const int r = q / cpr, ch = q % cpr;
        const int mm = m0 + TM * wm + 32 * i0 + r;
        const int n0 = rt0 * UNIT_ROWS + TN * wn + ch * per;
        if (mm >= J.m) continue;
        const u4 v = *(const u4 *)(s_c + r * TN * esz + ch * 16);
        char *dst = (char *)ybase + ((size_t)mm * yld + n0) * esz;
        if (yv && n0 + per <= nlim) {
          *(u4 *)dst = v;
        } else {
          for (int l = 0; l < per; ++l) {
            if (n0 + l >= nlim) break;
            if (bf) ((uint16_t *)dst)[l] = (uint16_t)(v[l >> 1] >> (16 * (l & 1)));
            else ((uint32_t *)dst)[l] = v[l];
          }
        }
      }
      __syncthreads();
    }
  }
}

// Sum of the K-split partial tiles of every split job, in split order:
// y[row][n] = sum_s part[s][row][n], four columns per thread.
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillBatch b) {
  int jn = 0;
  while (jn + 1 < b.count && (int)blockIdx.x >= b.job[jn + 1].red_begin) ++jn;
  const PrefillJob &J = b.job[jn];
  if (J.splits <= 1) return;
  const int per_row = (J.w.n + 1023) / 1024;  // blocks per output row
  const int lb = (int)blockIdx.x - J.red_begin;
  const int row = lb / per_row, n = (lb % per_row) * 1024 + 4 * (int)threadIdx.x;
  if (row >= J.m || n >= J.w.n) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < J.splits; ++sp) {
    const float4 v = *(const float4 *)(J.part + ((size_t)sp * J.m_pad + row) * J.n_pad + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const float o[4] = {acc.x, acc.y, acc.z, acc.w};
  for (int l = 0; l < 4 && n + l < J.w.n; ++l) store_out(J.y, (size_t)row * J.ldy + n + l, o[l], b.ydt);
}

hipError_t launch_prefill_reduce(PrefillBatch &b, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(prefill_reduce_kernel, dim3(blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

// Prep for the prefill launch: the permuted activations of every job in
// fragment order (xb_frag_offset), rows >= m and slots >= k zero.  A block
// takes `rpb` consecutive activation rows of one job and one of the job's
// prep_csplit ranges of 8-slot chunks (several when the rows alone give few
// blocks); it stages the live rows in LDS (rpb * k bf16), and thread tau
// handles row tau % rpb and every (256 / rpb)-th chunk of the range, so the
// rpb threads of one chunk write rpb * 16 contiguous bytes.
template <bool XVEC>
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillBatch b, int rpb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_rows[];
  int jn = 0;
  while (jn + 1 < b.count && (int)blockIdx.x >= b.job[jn + 1].prep_begin) ++jn;
  const PrefillJob &J = b.job[jn];
  const MatView &w = J.w;
  const int K = w.k, Kp = w.units * UNIT_SLOTS, S = Kp / P_BK;
  const int lb = (int)blockIdx.x - J.prep_begin;
  const int r0 = (lb / J.prep_csplit) * rpb, cs = lb % J.prep_csplit;
  const int nch = Kp / 8, cpb = (nch + J.prep_csplit - 1) / J.prep_csplit;
  const int c_lo = cs * cpb, c_hi = min(nch, c_lo + cpb);
  const int nlive = max(0, min(rpb, J.m - r0));  // rows of the group below m
  const int tid = threadIdx.x;
  // Stage the live rows (rows >= m are written as zeros below), LDS row
  // stride k + 8: the rpb threads of one chunk read one column of rpb rows,
  // and the 16-byte pad puts those rows in different banks.  Eight 16-byte
  // loads per thread are in flight at a time.
  const int ks_ = K + 8;
  if (XVEC) {
    const int n8 = K / 8, tot = nlive * n8;
    constexpr int B = 8;
    for (int q0 = tid; q0 < tot; q0 += 256 * B) {
      u4 v[B];
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const int q = min(q0 + 256 * bb, tot - 1);
        const int rr = q / n8, c = q - rr * n8;
        v[bb] = *(const u4 *)(J.x + (int64_t)min(r0 + rr, J.m - 1) * J.ldx + 8 * c);
      }
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const int q = q0 + 256 * bb;
        if (q < tot) {
          const int rr = q / n8, c = q - rr * n8;
          *(u4 *)(s_rows + (size_t)rr * ks_ + 8 * c) = v[bb];
        }
      }
    }
  } else {
    for (int rr = 0; rr < nlive; ++rr) {
      const uint16_t *xr = J.x + (int64_t)(r0 + rr) * J.ldx;
      uint16_t *dst = s_rows + (size_t)rr * ks_;
      for (int j = tid; j < K; j += 256) dst[j] = xr[j];
    }
  }
  __syncthreads();
  const uint16_t *perm = (const uint16_t *)(w.base + w.off_perm);
  const int rr = tid % rpb, r = r0 + rr;
  const uint16_t *row = s_rows + (size_t)rr * ks_;
  const bool live = r < J.m;
  // eight chunks at a time: their permutation vectors are loaded together
  const int cstep = 256 / rpb;
  for (int cb = c_lo + tid / rpb; cb < c_hi; cb += 8 * cstep) {
    u4 pv[8];
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
      pv[bb] = *(const u4 *)(perm + 8 * min(cb + bb * cstep, c_hi - 1));
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const int c = cb + bb * cstep;
      if (c >= c_hi) break;
      // perm is zero padded to the unit width, so every index is < k
      u4 v;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const uint32_t lo = live && 8 * c + 2 * l < K ? row[pv[bb][l] & 0xFFFFu] : 0u;
        const uint32_t hi = live && 8 * c + 2 * l + 1 < K ? row[pv[bb][l] >> 16] : 0u;
        v[l] = lo | (hi << 16);
      }
      *(u4 *)(J.xb + xb_frag_offset(r, 8 * c, S)) = v;
    }
  }
}

// LDS of a prep block: rpb staged rows of k + 8 values.
static size_t prep_lds(int rpb, int k_max) { return (size_t)rpb * (k_max + 8) * 2; }

int prefill_prep_rows(int k_max) {
  int rpb = 8;
  while (rpb > 1 && prep_lds(rpb, k_max) > GV_LDS_LIMIT) rpb /= 2;
  return rpb;
}

hipError_t launch_prefill_prep(PrefillBatch &b, int blocks, int rpb, int k_max, bool xvec,
                               hipStream_t s) {
  const size_t lds = prep_lds(rpb, k_max);
  if (lds > GV_LDS_LIMIT) return hipErrorInvalidValue;
  hipError_t e = xvec ? allow_smem(prefill_prep_kernel<true>, lds) : allow_smem(prefill_prep_kernel<false>, lds);
  if (e != hipSuccess) return e;
  if (xvec)
    hipLaunchKernelGGL(prefill_prep_kernel<true>, dim3(blocks), dim3(256), lds, s, b, rpb);
  else
    hipLaunchKernelGGL(prefill_prep_kernel<false>, dim3(blocks), dim3(256), lds, s, b, rpb);
  return hipGetLastError();
}

int prefill_bm(int m) { return m >= PREFILL_MIN_M ? 256 : 64; }

int prefill_m_pad(int m) {
  const int bm = prefill_bm(m);
  return ((m + bm - 1) / bm) * bm;
}

int prefill_tiles_n(int n_tiles) { return (n_tiles + P_BN / UNIT_ROWS - 1) / (P_BN / UNIT_ROWS); }

hipError_t launch_prefill_batched(PrefillBatch &b, int bm, int blocks, hipStream_t s) {
  if (bm == 256) {
    hipError_t e = allow_smem(prefill_batched_kernel<256>, P_SMEM);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_batched_kernel<256>, dim3(blocks), dim3(256), P_SMEM, s, b);
  } else {
    hipError_t e = allow_smem(prefill_batched_kernel<64>, P_SMEM);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_batched_kernel<64>, dim3(blocks), dim3(256), P_SMEM, s, b);
  }
  return hipGetLastError();
}

}  // namespace svq
