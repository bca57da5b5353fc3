// HIP kernels of libsvq for gfx950 (CDNA4).
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability" (SAGE).  A weight subvector is rebuilt on demand as
// radius * signs * direction (SAGE Fig. 2 caption) inside the product
// (Fig. 1 / Fig. 5 captions), against the subvector's eight reordered
// activations (Fig. 6 caption).  The pages' own kernel (Fig. 6: a 64-row
// mma loop over half-groups on an RTX 4090) is prior art only; these kernels
// are organised around the MI355X matrix cores and 64-wide wavefronts.
//
// Two decode-and-multiply schemes share the coded-unit layout described in
// svq_internal.h:
//
// * Exact (m <= 4, this file).  The 8 signed fp16 direction values of a
//   code are MFMA B operands as they come out of LDS (sign flips are exact),
//   4 values each for two chained v_mfma_f32_4x4x4_16b_f16; the activations
//   (fp16 after an exact power-of-two scale) are the A operands, so the MFMA
//   returns, in the very lane that decoded the code, the code's 8-term dot
//   product per activation row.  The radius multiply is then applied per
//   code in fp32 (fp16 radius x fp32 dot, fused multiply-add), so the
//   decoded weight R*D is never rounded.
// * bf16 (m > 4, svq_small.hip and svq_prefill.hip).  A code decodes to 8
//   bf16 weights RNE_bf16(R*D) with its signs from a 1024-row table (one row
//   per direction/radius index): straight into a v_mfma_f32_16x16x32_bf16
//   operand up to m = 16, through an LDS weight tile for
//   v_mfma_f32_32x32x16_bf16 above.
#include <cstring>
#include <type_traits>

#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

// ---------------------------------------------------------------------------
// Exact path (m <= 4): two launches.
// ---------------------------------------------------------------------------
//
// Gather launch: one wave per (matrix, activation row a, coded unit u).  Lane
// c takes code column c of the unit (permuted slots 8c .. 8c+7; Fig. 6
// caption: a subvector multiplies eight reordered activations), loads the
// eight activations x[a][perm[p]] and the wave writes the unit's fp16 copy
// with a power-of-two scale 2^e (max|x_au| * 2^e in [2^14, 2^15)).  A bf16
// value has 8 significant bits, so its scaled copy is exact down to a
// scaled magnitude of 2^-17 (the fp16 subnormal quantum is 2^-24), i.e. for
// every |x| >= 2^-31 * max|x_au|; smaller values round to fp16 subnormals.
// 2^-e is stored beside the copy and undone once per (row tile, unit) in
// fp32.
//
// Main launch: a block of 4 waves owns R consecutive 16-row tiles of one
// matrix and all of its K; the block's R*U coded units are split evenly
// between the waves in tile-major order (a wave's range may cross a tile
// boundary: its partial sums are flushed to LDS at every tile end).  One work
// item is one coded unit (16 rows x 64 codes, 2304 contiguous bytes, 36 per
// lane) together with the lane's four 16-byte activation fragments and the
// unit's scales, all loaded straight into registers GV_PIPE items ahead.
// MFMA mapping (v_mfma_f32_4x4x4_16b_f16: 16 blocks of 4 lanes, lane 4b + j):
//   B: lane 4b + j holds 4 signed direction values of its code (one half of
//      the code's 8), column j of block b;
//   A: lane 4b + j holds the matching 4 scaled activations of activation row
//      j (rows >= m repeat row 0), row j of block b; all four lanes of a
//      block share the code column;
//   C: lane 4b + j receives, for activation row a, the dot product of its
//      own code's half with row a; two chained halves give the code's 8-term
//      dot product.
// The radius multiply R[r] * dot is an fp32 FMA per code, so R*D is never
// rounded.
//
// Direction rows are read from LDS at random (one row per code), which is
// the main loop's most frequent LDS access.  A ds_read_b128 serves 16 lanes
// per pass, one 16-byte bank group each, so the table is stored C times,
// lane-interleaved: copy c of row d sits at d*16C + c*16 and lane l reads
// copy l % C.  With C = 16 (bd <= 7) the 16 lanes of a pass always hit 16
// different bank groups; the 256-row tables of bd = 8 keep C = 8 (32 KB, so
// that four blocks fit in a compute unit), two lanes per bank group.

#ifndef SVQ_GV_PIPE
#define SVQ_GV_PIPE 2
#endif
// Work items whose loads are in flight per wave.
constexpr int GV_PIPE = SVQ_GV_PIPE;
// lane-interleaved copies of a direction table of 2^bd rows (at most 32 KB)
// LDS (absolute addresses, see lds_u4): radius by 10-bit index, then the
// direction copies (2^bd rows of 256 bytes), then the cross-wave partial sums
// [R][GV_WAVES][4][4][4][M] fp32 at GemvBatch::red_off.

// Maximum over the 64 lanes of a non-negative float (returned in every
// lane): DPP row shifts within the 16-lane rows, row broadcasts across rows,
// then lane 63.
__device__ __forceinline__ float wave_max(float v) {
  int b = __builtin_bit_cast(int, v);  // non-negative floats order as ints
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x111, 0xF, 0xF, false));  // row_shr:1
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x112, 0xF, 0xF, false));  // row_shr:2
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x114, 0xF, 0xF, false));  // row_shr:4
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x118, 0xF, 0xF, false));  // row_shr:8
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x142, 0xA, 0xF, false));  // row_bcast:15
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
}

// (byte k of v) << SH in one VALU op (SDWA source select).
template <int K, int SH>
__device__ __forceinline__ uint32_t byte_shl(uint32_t v) {
  uint32_t r;
  if (K == 0)
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(v), "i"(SH));
  else if (K == 1)
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(v), "i"(SH));
  else if (K == 2)
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(v), "i"(SH));
  else
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(v), "i"(SH));
  return r;
}

// Byte 1 of dst := (byte k of v) & mask, the other bytes of dst kept (SDWA
// destination select with preserve): one VALU op turns a code's low index
// byte into the address of its direction row in the lane's table copy.
template <int K>
__device__ __forceinline__ void byte_and_to_b1(uint32_t &dst, uint32_t mask, uint32_t v) {
  if (K == 0)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_0"
        : "+v"(dst) : "v"(mask), "v"(v));
  else if (K == 1)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_1"
        : "+v"(dst) : "v"(mask), "v"(v));
  else if (K == 2)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_2"
        : "+v"(dst) : "v"(mask), "v"(v));
  else
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_3"
        : "+v"(dst) : "v"(mask), "v"(v));
}

// 64-bit left shift by a constant in one VALU op (the compiler otherwise
// splits it into a shift and a funnel shift).
template <int SH>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  if (SH == 0) return v;
  uint64_t r;
  asm("v_lshlrev_b64 %0, %2, %1" : "=v"(r) : "v"(v), "i"(SH));
  return r;
}

// Reads from the start of dynamic LDS by absolute address.  The exact-path
// kernels declare no static LDS, so dynamic LDS begins at address 0 (checked
// by the launcher) and the table offsets go straight into the instruction's
// address and offset fields.
typedef __attribute__((address_space(3))) const u4 lds_u4_t;
typedef __attribute__((address_space(3))) const _Float16 lds_f16_t;
__device__ __forceinline__ u4 lds_u4(uint32_t addr) { return *(lds_u4_t *)(size_t)addr; }
__device__ __forceinline__ _Float16 lds_f16(uint32_t addr) { return *(lds_f16_t *)(size_t)addr; }

// Gather of one block: activation row xr (K bf16) is staged in LDS with
// coalesced loads while each wave loads the permutation vector of its unit
// u0 + w (one memory round trip for both); then wave w writes the unit's
// permuted fp16 copy (64 x 16 bytes at xg_row + u * 1 KB, lane c = code
// column c) with its exact power-of-two scale (see the gather launch above),
// and 2^-e to xs_row[4u].  xvec: xr is 16-byte aligned.
constexpr int GV_STAGE_BATCH = 8;  // staging loads in flight per thread
__device__ __forceinline__ void gather_block(const uint16_t *__restrict__ perm,
                                             const uint16_t *__restrict__ xr, int K, int U, int u0,
                                             bool xvec, uint8_t *__restrict__ xg_row,
                                             float *__restrict__ xs_row, uint8_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = min(u0 + wv, U - 1);  // clamped: every wave reaches the barrier
  const int p0 = u * UNIT_SLOTS + 8 * lane;
  const u4 pv = __builtin_nontemporal_load((const u4 *)(perm + p0));
  uint16_t *s_x = (uint16_t *)smem;
  if (xvec) {
    const int n8 = K / 8;
    for (int base = 0; base < n8; base += 256 * GV_STAGE_BATCH) {
      u4 v[GV_STAGE_BATCH];
#pragma unroll
      for (int g = 0; g < GV_STAGE_BATCH; ++g) {
        const int idx = base + g * 256 + tid;
        v[g] = ((const u4 *)xr)[min(idx, n8 - 1)];
      }
#pragma unroll
      for (int g = 0; g < GV_STAGE_BATCH; ++g) {
        const int idx = base + g * 256 + tid;
        if (idx < n8) ((u4 *)s_x)[idx] = v[g];
      }
    }
  } else {
    for (int base = 0; base < K; base += 256 * 2 * GV_STAGE_BATCH) {
      uint16_t v[2 * GV_STAGE_BATCH];
#pragma unroll
      for (int g = 0; g < 2 * GV_STAGE_BATCH; ++g) v[g] = xr[min(base + g * 256 + tid, K - 1)];
#pragma unroll
      for (int g = 0; g < 2 * GV_STAGE_BATCH; ++g)
        if (base + g * 256 + tid < K) s_x[base + g * 256 + tid] = v[g];
    }
  }
  __syncthreads();
  if (u0 + wv >= U) return;  // wave-uniform, after the only barrier
  float v[8], mx = 0.f;
#pragma unroll
  for (int l = 0; l < 4; ++l) {  // perm is zero padded to the unit width: every channel < K
    v[2 * l] = (p0 + 2 * l < K) ? bf16_bits_to_f32(s_x[pv[l] & 0xFFFFu]) : 0.f;
    v[2 * l + 1] = (p0 + 2 * l + 1 < K) ? bf16_bits_to_f32(s_x[pv[l] >> 16]) : 0.f;
  }
#pragma unroll
  for (int l = 0; l < 8; ++l) mx = fmaxf(mx, fabsf(v[l]));
  mx = wave_max(mx);
  const int e = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
  u4 h;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const _Float16 lo = (_Float16)ldexpf(v[2 * l], e), hi = (_Float16)ldexpf(v[2 * l + 1], e);
    h[l] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  ((u4 *)(xg_row + (size_t)u * GV_XG_UNIT_BYTES))[lane] = h;
  if (lane == 0) xs_row[4 * u] = ldexpf(1.f, -e);
}

// Gather launch of the dense path: block = (job, activation row a, group of
// 4 units), wave = unit.  The launch ends with 8 blocks per job (one per XCD:
// blocks go to the XCDs round-robin) that only read the job's direction and
// radius tables, so that the main launch finds them near.
__global__ __launch_bounds__(256) void gemv_gather_kernel(GemvBatch b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  if ((int)blockIdx.x >= b.touch_begin) {
    const int jt = ((int)blockIdx.x - b.touch_begin) >> 3;
    if (jt < b.count) {
      const MatView &w = b.job[jt].w;
      const u4 d = ((const u4 *)(w.base + w.off_dtab))[threadIdx.x];
      const u2 r = ((const u2 *)(w.base + w.off_rtab))[threadIdx.x];
      asm volatile("" ::"v"(d), "v"(r));  // keeps the loads
    }
    return;
  }
  const int j = find_job(b.gather_starts, b.count);
  const GemvJob &jb = b.job[j];
  const int U = jb.w.units, groups = (U + GV_WAVES - 1) / GV_WAVES;
  const int local = (int)blockIdx.x - b.gather_starts.first[j];
  const int a = local / groups, u0 = (local - a * groups) * GV_WAVES;
  if (a >= b.m) return;  // block-uniform, before the barrier
  gather_block((const uint16_t *)(jb.w.base + jb.w.off_perm), jb.x + (int64_t)a * jb.ldx, jb.w.k, U,
               u0, b.xvec != 0, jb.xg + (size_t)a * U * GV_XG_UNIT_BYTES, jb.xs + a, smem);
}

// Activation fragments of one item, one per column group.  With a single
// activation row the four lanes of an MFMA block need the same 16 bytes, so
// each lane holds one dword of them (4 registers per item instead of 16) and
// the block's lanes exchange them (DPP quad broadcasts) when the item is
// used.
template <int M>
struct GvAct {
  u4 A[4];
  template <int CI>
  __device__ __forceinline__ u4 get() const { return A[CI]; }
};
template <>
struct GvAct<1> {
  uint32_t q[4];
  template <int CI>
  __device__ __forceinline__ u4 get() const {
    const int v = (int)q[CI];
    return (u4){(uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x00, 0xF, 0xF, false),
                (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false),
                (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false),
                (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false)};
  }
};

// One work item in registers: the lane's 36 code bytes, its activation
// fragments and the unit's scales (one per activation row).
template <int M>
struct GvItem {
  ItemCodes c;
  GvAct<M> act;
  float sc[M];
};

// Item f of a block (flat unit index, tile-major from the block's first
// tile; u = f mod U): codes at codes + f*UNIT_BYTES, activations of unit u.
template <int M>
__device__ __forceinline__ GvItem<M> load_gv_item(const uint8_t *codes, const uint8_t *xa,
                                                  const float *xs, int f, int u, int lane) {
  GvItem<M> it;
  it.c = load_item<true>(codes + (size_t)f * UNIT_BYTES, lane);
  if constexpr (M == 1) {
#pragma unroll
    for (int ci = 0; ci < 4; ++ci)
      it.act.q[ci] = *(const uint32_t *)(xa + (size_t)u * GV_XG_UNIT_BYTES + 256 * ci + 4 * (lane & 3));
  } else {
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) it.act.A[ci] = *(const u4 *)(xa + (size_t)u * GV_XG_UNIT_BYTES + 256 * ci);
  }
#pragma unroll
  for (int a = 0; a < M; ++a) it.sc[a] = xs[4 * u + a];
  return it;
}

// Sum over the four lanes of each 16-lane row that share lane & 3 (DPP row
// rotations); every such lane receives the sum.
__device__ __forceinline__ float row_sum4(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  return v;
}

// Direction-row address parts: index bits, log2 of the row stride (16
// bytes per copy), the lane's copy offset.
struct DirAddr {
  uint32_t bd, rs, loff;
};

// Table reads of the four codes of column group ci: direction rows (signs
// not yet applied) from the lane's table copy, and radii.
template <int CI>
__device__ __forceinline__ void gemv_group_reads(const ItemCodes &c, const DirAddr &da,
                                                 uint32_t (&dad)[4], u4 (&D)[4], _Float16 (&R)[4]) {
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    const int i = 4 * ri + CI;
    // direction index * row stride + copy * 16
    dad[ri] = (__builtin_amdgcn_ubfe(c.L[ri], 8 * CI, da.bd) << da.rs) | da.loff;
    const uint32_t lo2 = byte_shl<CI, 1>(c.L[ri]);  // low index byte * 2
    const int sh = 9 - 2 * i;
    const uint32_t hs = sh >= 0 ? c.H << sh : c.H >> -sh;
    const uint32_t idx2 = (hs & 0x600u) | lo2;      // 10-bit index * 2
    D[ri] = lds_u4(GV_OFF_D + dad[ri]);
    R[ri] = lds_f16(GV_OFF_RTAB + idx2);
  }
}

// Sign carriers of code i (see the sign plane): bits 15 and 31 of c[j] are
// the signs of pair j.
template <int I>
__device__ __forceinline__ void sign_carriers(uint64_t S01, uint64_t S23, uint32_t (&cr)[4]) {
  const uint64_t c01 = shl64<I>(S01), c23 = shl64<I>(S23);
  cr[0] = (uint32_t)c01;
  cr[1] = (uint32_t)(c01 >> 32);
  cr[2] = (uint32_t)c23;
  cr[3] = (uint32_t)(c23 >> 32);
}

// Decode-and-multiply of the four codes of column group ci (see the mapping
// above): tmp[ri][a] += R * dot(code, activation row a).  The four codes go
// through each phase together (signs, first-half MFMAs, second-half MFMAs,
// radius FMAs), so that independent MFMAs cover each other's latency.
template <int M, int CI, typename RT>
__device__ __forceinline__ void gemv_group_mul(uint64_t S01, uint64_t S23, const u4 &A,
                                              const u4 (&Din)[4], const RT (&R)[4],
                                              float (&tmp)[4][M]) {
  const uint32_t SM = 0x80008000u;
  const h4 A0 = __builtin_bit_cast(h4, (u2){A[0], A[1]});
  const h4 A1 = __builtin_bit_cast(h4, (u2){A[2], A[3]});
  u4 D[4];
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    uint32_t cr[4];
    switch (ri) {
      case 0: sign_carriers<CI>(S01, S23, cr); break;
      case 1: sign_carriers<4 + CI>(S01, S23, cr); break;
      case 2: sign_carriers<8 + CI>(S01, S23, cr); break;
      default: sign_carriers<12 + CI>(S01, S23, cr); break;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) D[ri][j] = Din[ri][j] ^ (cr[j] & SM);
  }
  f4 C[4];
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
    C[ri] = __builtin_amdgcn_mfma_f32_4x4x4f16(A0, __builtin_bit_cast(h4, (u2){D[ri][0], D[ri][1]}),
                                               (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
    C[ri] = __builtin_amdgcn_mfma_f32_4x4x4f16(A1, __builtin_bit_cast(h4, (u2){D[ri][2], D[ri][3]}),
                                               C[ri], 0, 0, 0);
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    const float Rf = (float)R[ri];
#pragma unroll
    for (int a = 0; a < M; ++a) tmp[ri][a] = __builtin_fmaf(Rf, C[ri][a], tmp[ri][a]);
  }
  // materialise the partial sums here: left alone, instruction selection
  // sinks every radius FMA of the item to its end and keeps all 16 MFMA
  // results live
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int a = 0; a < M; ++a) asm volatile("" : "+v"(tmp[ri][a]));
}

// One work item: the lane's 16 codes, column group by column group, with
// the table reads of the next group issued before the current one is used.
template <int M>
__device__ __forceinline__ void gemv_item(const GvItem<M> &it, const DirAddr &dmask, uint32_t (&dad0)[4],
                                          uint32_t (&dad1)[4], float (&tmp)[4][M]) {
  const ItemCodes &c = it.c;
  const uint64_t S01 = (uint64_t)c.S[0] | ((uint64_t)c.S[1] << 32);
  const uint64_t S23 = (uint64_t)c.S[2] | ((uint64_t)c.S[3] << 32);
  u4 D0[4], D1[4];
  _Float16 R0[4], R1[4];
  // phases are kept in this order (scheduling barriers): the reads of group
  // g + 1 are in flight while group g is decoded and multiplied
  gemv_group_reads<0>(c, dmask, dad0, D0, R0);
  gemv_group_reads<1>(c, dmask, dad1, D1, R1);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 0>(S01, S23, it.act.template get<0>(), D0, R0, tmp);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_reads<2>(c, dmask, dad0, D0, R0);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 1>(S01, S23, it.act.template get<1>(), D1, R1, tmp);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_reads<3>(c, dmask, dad1, D1, R1);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 2>(S01, S23, it.act.template get<2>(), D0, R0, tmp);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 3>(S01, S23, it.act.template get<3>(), D1, R1, tmp);
}

// Main launch, one block: tiles t0 .. t0+Reff-1 of matrix w (U units each),
// activations gathered at xg / xs (row a of unit u at xg + (a*U + u) * 1 KB).
template <int M>
__device__ void gemv_main_block(const MatView &w, const uint8_t *__restrict__ xg,
                                const float *__restrict__ xs, void *__restrict__ y, int64_t ldy,
                                int ydt, int t0, int Reff, int red_off, uint8_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int U = w.units, F = Reff * U;
  // the wave's items: flat units f = wv + k*GV_WAVES < F, k < n_items (the
  // block's waves step through its units side by side, so that at any time
  // they read neighbouring units)
  static_assert(GV_WAVES == 4, "gv_wave_items assumes 4 waves per block");
  const int n_items = gv_wave_items(F, wv);
  const uint8_t *codes = w.base + w.off_codes + (size_t)t0 * U * UNIT_BYTES;
  // lane 4b + j reads activation row j (row 0 when j >= M) of code column
  // 16*ci + b of each unit
  const int jl = lane & 3, bl = lane >> 2;
  const uint8_t *xa = xg + (size_t)(jl < M ? jl : 0) * U * GV_XG_UNIT_BYTES + 16 * bl;

  // Tables first, and their LDS copies written before any code is
  // requested: at the start of a launch every block asks for its tables at
  // once, and behind the code stream of the blocks already running they
  // would wait for the whole queue.
  const int bd = w.bd, rows = 1 << bd;
  const u4 drow = ((const u4 *)(w.base + w.off_dtab))[tid & (rows - 1)];
  const u2 rrow = ((const u2 *)(w.base + w.off_rtab))[tid];
  // LDS: radius table, 16 lane-interleaved copies of the direction table
  // (each thread writes copies of row tid mod 2^bd; the copy index rotates
  // with the row so that the lanes of one store hit different bank groups),
  // zeroed partial sums [R][GV_WAVES][4 lane rows][j][ri][M] (tile, wave,
  // 16-lane row of the wave, then output row 4*ri + j of the tile)
  float *s_red = (float *)(smem + red_off);
  for (int o = tid; o < Reff * GV_WAVES * 64 * M; o += 256) s_red[o] = 0.f;
  ((u2 *)(smem + GV_OFF_RTAB))[tid] = rrow;
  const int copies = gv_copies(bd);
  for (int e = tid; e < rows * copies; e += 256) {
    const int row = e & (rows - 1), cp = ((e >> bd) + row) & (copies - 1);
    *(u4 *)(smem + GV_OFF_D + (row * copies + cp) * 16) = drow;
  }

  __syncthreads();  // before the code requests: a wave may stall while issuing them

  // The first GV_PIPE items, all unconditional (clamped indexes) and in the
  // order of the main loop's refills (scheduling barriers), which keeps its
  // wait counts exact.
  GvItem<M> ring[GV_PIPE];
  int fl = wv, ul = wv % U;  // next item to load and its unit
#pragma unroll
  for (int s = 0; s < GV_PIPE; ++s) {
    const bool in = fl < F;
    __builtin_amdgcn_sched_barrier(0);
    ring[s] = load_gv_item<M>(codes, xa, xs, gv_load_flat(fl, F), in ? ul : U - 1, lane);
    __builtin_amdgcn_sched_barrier(0);
    fl += GV_WAVES;
    for (ul += GV_WAVES; ul >= U; ul -= U) {}
  }

  DirAddr dmask;
  dmask.bd = (uint32_t)bd;
  dmask.rs = copies == 16 ? 8u : 7u;
  dmask.loff = (uint32_t)(lane & (copies - 1)) << 4;
  uint32_t dad0[4], dad1[4];  // direction addresses
  float acc[4][M];
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int a = 0; a < M; ++a) acc[ri][a] = 0.f;

  auto step = [&](const GvItem<M> &it) __attribute__((always_inline)) {
    // items are scheduled one at a time: interleaving several items only
    // raises register pressure
    __builtin_amdgcn_sched_barrier(0);
    float tmp[4][M];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int a = 0; a < M; ++a) tmp[ri][a] = 0.f;
    gemv_item<M>(it, dmask, dad0, dad1, tmp);
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int ri = 0; ri < 4; ++ri) acc[ri][a] = __builtin_fmaf(tmp[ri][a], it.sc[a], acc[ri][a]);
  };
  // partial sums of tile tl (block-local): sum over the 4 code columns of
  // each 16-lane row that share j, then every lane stores its row's sums
  // (the four lanes of equal j store equal values to one place: no lane
  // mask, no cross-row traffic; the rows meet in the final sum)
  auto flush = [&](int tl) __attribute__((always_inline)) {
    float *dst = s_red + (((tl * GV_WAVES + wv) * 4 + (lane >> 4)) * 4 + (lane & 3)) * 4 * M;
    float v[4 * M];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int a = 0; a < M; ++a) {
        v[ri * M + a] = row_sum4(acc[ri][a]);
        acc[ri][a] = 0.f;
      }
#pragma unroll
    for (int q = 0; q < M; ++q) ((u4 *)dst)[q] = (u4){__builtin_bit_cast(uint32_t, v[4 * q]),
                                                    __builtin_bit_cast(uint32_t, v[4 * q + 1]),
                                                    __builtin_bit_cast(uint32_t, v[4 * q + 2]),
                                                    __builtin_bit_cast(uint32_t, v[4 * q + 3])};
  };

  // Items k = 0 .. n_items-1 (ring slot k % GV_PIPE).  While GV_PIPE more
  // items follow, each processed slot is refilled at once (unconditional
  // loads); the last GV_PIPE items have no refills.  The partial sums are
  // flushed whenever the next item lies in another tile.
  int k = 0, t = wv / U, u = wv % U;  // tile and unit of item k
  auto advance = [&]() __attribute__((always_inline)) {
    const int t_now = t;
    for (u += GV_WAVES; u >= U; u -= U) ++t;
    ++k;
    if (k == n_items || t != t_now) flush(t_now);
  };
  while (k + GV_PIPE < n_items) {
#pragma unroll
    for (int s = 0; s < GV_PIPE; ++s) {
      step(ring[s]);
      // item k + GV_PIPE exists for s = 0 only when the loop is entered;
      // a refill past the wave's run reads the block's last item instead
      // (never used), so every address stays inside the matrix
      const bool in = fl < F;
      ring[s] = load_gv_item<M>(codes, xa, xs, gv_load_flat(fl, F), in ? ul : U - 1, lane);
      fl += GV_WAVES;
      for (ul += GV_WAVES; ul >= U; ul -= U) {}
      advance();
    }
  }
#pragma unroll
  for (int s = 0; s < GV_PIPE; ++s) {
    if (k < n_items) {
      step(ring[s]);
      advance();
    }
  }
  __syncthreads();
  for (int o = tid; o < Reff * 16 * M; o += 256) {
    const int t = o / (16 * M), rem = o - t * 16 * M, row = rem / M, a = rem - row * M;
    const int ri = row >> 2, j = row & 3;
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < GV_WAVES * 4; ++p) sum += s_red[((t * GV_WAVES * 4 + p) * 4 + j) * 4 * M + ri * M + a];
    const int n = (t0 + t) * 16 + row;
    if (n < w.n) store_out(y, (size_t)a * ldy + n, sum, ydt);
  }
}

template <int M>
__global__ __launch_bounds__(256) void gemv_batched_kernel(GemvBatch b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int j = find_job(b.starts, b.count);
  const GemvJob &jb = b.job[j];
  const int t0 = ((int)blockIdx.x - b.starts.first[j]) * jb.R;
  const int Reff = min(jb.R, jb.w.n_tiles - t0);
  gemv_main_block<M>(jb.w, jb.xg, jb.xs, jb.y, jb.ldy, b.ydt, t0, Reff, b.red_off, smem);
}


// The exact-path kernels address their LDS tables from 0 (see lds_u4), which
// holds when they declare no static LDS.
template <typename Kern>
static hipError_t check_no_static_lds(Kern k) {
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, (const void *)k);
  if (e != hipSuccess) return e;
  return attr.sharedSizeBytes == 0 ? hipSuccess : hipErrorInvalidKernelFile;
}

template <int M>
static hipError_t launch_gemv_m(GemvBatch &b, int blocks, size_t smem, hipStream_t s) {
  static const hipError_t lds_ok = check_no_static_lds(gemv_batched_kernel<M>);
  if (lds_ok != hipSuccess) return lds_ok;
  hipError_t e = allow_smem(gemv_batched_kernel<M>, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemv_batched_kernel<M>), dim3(blocks), dim3(256), smem, s, b);
  return hipGetLastError();
}

hipError_t launch_gemv_batched(GemvBatch &b, int gather_blocks, int k_max, int blocks, size_t smem,
                               hipStream_t s) {
  const size_t gsmem = align256((size_t)k_max * 2);
  hipError_t e = allow_smem(gemv_gather_kernel, gsmem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemv_gather_kernel, dim3(gather_blocks), dim3(256), gsmem, s, b);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (b.m) {
    case 1: return launch_gemv_m<1>(b, blocks, smem, s);
    case 2: return launch_gemv_m<2>(b, blocks, smem, s);
    case 3: return launch_gemv_m<3>(b, blocks, smem, s);
    default: return launch_gemv_m<4>(b, blocks, smem, s);
  }
}

// ---------------------------------------------------------------------------
// Exact path, m = 1: one fused launch (gather + scale + decode-and-multiply).
// ---------------------------------------------------------------------------
//
// With a single activation row the gather costs less inside the block than
// as a launch of its own.  A block owns R <= GF_MAX_R consecutive 16-row
// tiles of one matrix and all of its K; its R x U items (unit u of tile t,
// tile-major, which is their order in memory) are cut into 4 equal runs,
// one per wave, and a wave flushes its sums to its LDS slot of a tile when
// its run leaves the tile.  Prologue: the block
// stages the activation row in LDS and gathers the permuted slots unit by
// unit, with the exact per-unit power-of-two scale described above.  Main
// loop: the same work items and MFMA mapping as the main launch of m = 2..4,
// with the activations read from LDS and the tables in one of the two modes
// below.
constexpr int GF_PRE_UNITS = 5;    // permutation vectors prefetched per wave (gather)
constexpr int GF_STAGE_BATCH = 5;  // 16-byte activation loads per thread per staging pass
// Tables, per block by the matrix's bd (a template parameter):
// * direction rows, lane-interleaved copies so that the lanes of one
//   ds_read_b128 pass spread over the bank groups: bd <= 7: 16 copies at a
//   256-byte row stride (copy c of row d at d*256 + 16c, lane l reads copy
//   l & 15: the 16 lanes of a pass hit 16 different bank groups; the row
//   address is one SDWA op); bd = 8: 8 copies at a 128-byte stride (32 KB,
//   written over the staging row once the gather is done; two lanes of a
//   pass share a bank group);
// * radii: the 2^(10-bd) values in fp32, one copy per lane (R[r] of lane l
//   at r*256 + 4l: every lane reads its own bank, so the read never
//   conflicts).  The address r*256 + 4l is formed in at most three ops from
//   the code planes: the low index byte's top 8 - bd bits go into byte 1 of
//   a register whose byte 0 holds 4l (SDWA destination select), the two
//   high index bits are shifted into place and or-ed in.
// LDS map: gf_lds (svq_internal.h).

// Table reads of the four codes of column group ci: direction rows (signs
// not yet applied) and radii.
// byte 1 of dst := (byte K of v) >> SH, the other bytes kept
template <int K, int SH>
__device__ __forceinline__ void byte_shr_to_b1(uint32_t &dst, uint32_t v) {
  if (K == 0)
    asm("v_lshrrev_b32_sdwa %0, %2, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_0"
        : "+v"(dst) : "v"(v), "i"(SH));
  else if (K == 1)
    asm("v_lshrrev_b32_sdwa %0, %2, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_1"
        : "+v"(dst) : "v"(v), "i"(SH));
  else if (K == 2)
    asm("v_lshrrev_b32_sdwa %0, %2, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_2"
        : "+v"(dst) : "v"(v), "i"(SH));
  else
    asm("v_lshrrev_b32_sdwa %0, %2, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_3"
        : "+v"(dst) : "v"(v), "i"(SH));
}

typedef __attribute__((address_space(3))) const float lds_f32_t;
__device__ __forceinline__ float lds_f32(uint32_t addr) { return *(lds_f32_t *)(size_t)addr; }

// (16-bit word W of v) << SH in one VALU op (SDWA source select).
template <int W, int SH>
__device__ __forceinline__ uint32_t word_shl(uint32_t v) {
  uint32_t r;
  if (W == 0)
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
        : "=v"(r) : "v"(v), "i"(SH));
  else
    asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(r) : "v"(v), "i"(SH));
  return r;
}

typedef __attribute__((address_space(3))) const uint16_t lds_u16_t;
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// The two staged bf16 values one dword of permutation entries names:
// x[c0] in bits 0..15, x[c1] in bits 16..31 (c0, c1: the dword's low and
// high entries; the staging row starts at the constant STAGE).
template <int STAGE>
__device__ __forceinline__ uint32_t stage_pair(uint32_t pv) {
  const uint32_t lo = *(lds_u16_t *)(size_t)(STAGE + word_shl<0, 1>(pv));
  const uint32_t hi = *(lds_u16_t *)(size_t)(STAGE + word_shl<1, 1>(pv));
  return lo | (hi << 16);
}

// Elementwise max of the magnitudes of two packed bf16 pairs, as 16-bit
// integers (finite bf16 magnitudes order as their bit patterns).
__device__ __forceinline__ uint32_t pk_absmax(uint32_t m, uint32_t p) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, m),
                                                                __builtin_bit_cast(us2, p & 0x7FFF7FFFu)));
}

// dad: direction addresses (bd <= 7: byte 0 = the lane's copy * 16, byte 1
// rewritten per code); rad: radius addresses (bd <= 7: byte 0 = 4 * lane,
// byte 1 rewritten per code); loff: the lane's copy offset (bd = 8) and 4 * lane.
template <int CI, int BD>
__device__ __forceinline__ void gf_group_reads(const ItemCodes &c, uint32_t (&dad)[4], uint32_t (&rad)[4],
                                               uint32_t loff, uint32_t lane4, u4 (&D)[4], float (&R)[4]) {
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    const int i = 4 * ri + CI;
    uint32_t raddr;
    if constexpr (BD <= 7) {
      byte_and_to_b1<CI>(dad[ri], (1u << BD) - 1u, c.L[ri]);  // direction * 256 + copy * 16
      byte_shr_to_b1<CI, BD>(rad[ri], c.L[ri]);                 // radius bits of the low byte, * 256
      // the two high index bits, r bits 8-BD..9-BD, to address bits 16-BD..17-BD
      const int sh = 16 - BD - 2 * i;  // unrolled: a constant
      const uint32_t hs = sh >= 0 ? c.H << sh : c.H >> -sh;
      raddr = (hs & (3u << (16 - BD))) | rad[ri];
      D[ri] = lds_u4(gf_off_d(BD) + dad[ri]);
    } else {
      // direction * 128 + copy * 16; radius = the two high index bits
      const uint32_t d128 = byte_shl<CI, 7>(c.L[ri]);
      const int sh = 8 - 2 * i;  // unrolled: a constant
      const uint32_t hs = sh >= 0 ? c.H << sh : c.H >> -sh;
      raddr = (hs & 0x300u) | lane4;
      D[ri] = lds_u4(gf_off_d(BD) + (d128 | loff));
    }
    R[ri] = lds_f32(GF_OFF_R + raddr);
  }
}

// One work item: the lane's 16 codes, column group by column group, with
// the table reads of the next group issued before the current one is used.
template <int M, int BD>
__device__ __forceinline__ void gf_item(const ItemCodes &c, const uint8_t *xu, uint32_t (&dad0)[4],
                                        uint32_t (&dad1)[4], uint32_t (&rad0)[4], uint32_t (&rad1)[4],
                                        uint32_t loff, uint32_t lane4, float (&tmp)[4][M]) {
  const uint64_t S01 = (uint64_t)c.S[0] | ((uint64_t)c.S[1] << 32);
  const uint64_t S23 = (uint64_t)c.S[2] | ((uint64_t)c.S[3] << 32);
  u4 D0[4], D1[4];
  float R0[4], R1[4];
  // phases are kept in this order (scheduling barriers): the reads of group
  // g + 1 are in flight while group g is decoded and multiplied
  u4 A0 = *(const u4 *)(xu);
  gf_group_reads<0, BD>(c, dad0, rad0, loff, lane4, D0, R0);
  u4 A1 = *(const u4 *)(xu + 256);
  gf_group_reads<1, BD>(c, dad1, rad1, loff, lane4, D1, R1);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 0>(S01, S23, A0, D0, R0, tmp);
  __builtin_amdgcn_sched_barrier(0);
  A0 = *(const u4 *)(xu + 512);
  gf_group_reads<2, BD>(c, dad0, rad0, loff, lane4, D0, R0);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 1>(S01, S23, A1, D1, R1, tmp);
  __builtin_amdgcn_sched_barrier(0);
  A1 = *(const u4 *)(xu + 768);
  gf_group_reads<3, BD>(c, dad1, rad1, loff, lane4, D1, R1);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 2>(S01, S23, A0, D0, R0, tmp);
  __builtin_amdgcn_sched_barrier(0);
  gemv_group_mul<M, 3>(S01, S23, A1, D1, R1, tmp);
}

// XVEC: every activation row starts 16-byte aligned (vector staging loads).
// BD: the matrix's direction bits (table layout, see above).
template <int M, bool XVEC, int BD>
__device__ void gemv_fused_block(const MatView &w, const uint16_t *__restrict__ x, int64_t ldx,
                                 void *__restrict__ y, int64_t ldy, int ydt, int rt0, int R,
                                 int Reff, uint8_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int U = w.units, Kp = U * UNIT_SLOTS, K = w.k;
  constexpr int rows = 1 << BD;
  const GfLds L = gf_lds(BD, K, U, M, R);
  float *s_scale = (float *)(smem + L.scale);             // [U][M] 2^-e per unit
  float *s_red = (float *)(smem + L.red);                 // [GF_MAX_R][W][4][M][4]
  uint16_t *s_xp = (uint16_t *)(smem + L.xp);             // [M][Kp] fp16
  uint16_t *s_stage = (uint16_t *)(smem + L.stage);       // [K] bf16
  const int n8 = K / 8;

  // this wave's work: items [i_begin, i_end) of the block's Reff x U items
  // (item i = unit i % U of tile rt0 + i / U, at codes0 + i units)
  const int n_items = Reff * U;
  const int i_begin = gf_wave_begin(n_items, GV_WAVES, wv);
  const int i_end = gf_wave_begin(n_items, GV_WAVES, wv + 1);
  const uint8_t *codes0 = w.base + w.off_codes + (size_t)rt0 * U * UNIT_BYTES;
  // this wave's share of the gather: units [g_lo, g_hi]
  const int gper = (U + GV_WAVES - 1) >> 2;
  const int g_lo = wv * gper, g_hi = min(U, g_lo + gper) - 1;

  // Global loads of the prologue, all unconditional (clamped addresses) so
  // that the wait counts stay exact, in the order they are needed: tables,
  // permutation vectors of the wave's gather units and the first staging
  // pass of every activation row; the codes follow once row 0 is staged.
  const u4 drow = ((const u4 *)(w.base + w.off_dtab))[tid & (rows - 1)];
  // radii for the lane-copy table: entry e = r * 64 + lane, R[r] at 10-bit
  // index r << BD of the packed radius table
  constexpr int nrad = 1 << (10 - BD);
  _Float16 rv[(nrad * 64 + 255) / 256];
  const _Float16 *rtab = (const _Float16 *)(w.base + w.off_rtab);
#pragma unroll
  for (int q = 0; q < (nrad * 64 + 255) / 256; ++q) rv[q] = rtab[((tid + 256 * q) >> 6) << BD];
  const uint16_t *perm = (const uint16_t *)(w.base + w.off_perm);
  u4 pvec[GF_PRE_UNITS];
#pragma unroll
  for (int j = 0; j < GF_PRE_UNITS; ++j)
    pvec[j] = *(const u4 *)(perm + min(g_lo + j, U - 1) * UNIT_SLOTS + 8 * lane);
  u4 xv[M][GF_STAGE_BATCH];
  if (XVEC) {
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int b = 0; b < GF_STAGE_BATCH; ++b)
        xv[a][b] = ((const u4 *)(x + (int64_t)a * ldx))[min(tid + 256 * b, n8 - 1)];
  }
  ItemCodes ring[GV_PIPE];
  int ul = i_begin;  // next item to load
  // every (tile, wave) slot of the tile sums starts at zero: a wave adds
  // only the tiles its run touches
  for (int e = tid; e < R * GV_WAVES * 4 * M * 4; e += 256) s_red[e] = 0.f;
#pragma unroll
  for (int q = 0; q < (nrad * 64 + 255) / 256; ++q)
    if (tid + 256 * q < nrad * 64) ((float *)(smem + GF_OFF_R))[tid + 256 * q] = (float)rv[q];
  if constexpr (BD <= 7) {
    // 16 copies of each row; the copy index rotates with the row so that the
    // lanes of one store hit different bank groups
    for (int e = tid; e < rows * 16; e += 256) {
      const int row = e & (rows - 1), cp = ((e >> BD) + row) & 15;
      *(u4 *)(smem + gf_off_d(BD) + (row * 16 + cp) * 16) = drow;
    }
  }

  // fp16 copy of gathered unit uu of activation row a with its exact
  // power-of-two scale: 2^e with max|x_unit| * 2^e in [2^14, 2^15), i.e.
  // e = 14 - ilogb(max) = 15 - (frexp exponent of max).  pr: the lane's
  // eight slots as packed bf16 pairs; mxb: bf16 bits of the unit's largest
  // magnitude.
  auto gather_store = [&](int a, int uu, const uint32_t (&pr)[4], uint32_t mxb) __attribute__((always_inline)) {
    const float mxw = bf16_bits_to_f32(mxb);
    const int e = mxw > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mxw) : 0;
    u4 h;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const _Float16 lo = (_Float16)ldexpf(bf16_bits_to_f32(pr[l] & 0xFFFFu), e);
      const _Float16 hi = (_Float16)ldexpf(__builtin_bit_cast(float, pr[l] & 0xFFFF0000u), e);
      h[l] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    ((u4 *)(s_xp + (size_t)a * Kp))[64 * uu + lane] = h;
    if (lane == 0) s_scale[uu * M + a] = ldexpf(1.f, -e);
  };
  // The lane's eight slots of unit uu (permutation entries pv) as packed
  // bf16 pairs, and their largest magnitude per pair half.  k is a multiple
  // of 8, so a lane's eight slots are all inside k or all padding (zeros).
  auto gather_pairs = [&](const u4 &pv, int uu, uint32_t (&pr)[4]) __attribute__((always_inline)) {
    const bool valid = uu * UNIT_SLOTS + 8 * lane < K;
    uint32_t m2 = 0;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const uint32_t p = stage_pair<gf_off_stage(BD)>(pv[l]);
      pr[l] = valid ? p : 0u;
      m2 = pk_absmax(m2, pr[l]);
    }
    return max(m2 & 0xFFFFu, m2 >> 16);
  };
  auto wave_max_bits = [](uint32_t b) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint32_t, wave_max(__builtin_bit_cast(float, b)));
  };

  // One activation row at a time: stage it in LDS, then every wave gathers
  // the permuted slots of its gather units and converts them to fp16 with
  // their per-unit scale.  (Unrolled: xv is indexed by the row.)
#pragma unroll
  for (int a = 0; a < M; ++a) {
    const uint16_t *xr = x + (int64_t)a * ldx;
    if (a > 0) __syncthreads();  // previous row's gathers are done
    if (XVEC) {
#pragma unroll
      for (int b = 0; b < GF_STAGE_BATCH; ++b) {
        const int j = tid + 256 * b;
        if (j < n8) ((u4 *)s_stage)[j] = xv[a][b];
      }
      for (int j = tid + 256 * GF_STAGE_BATCH; j < n8; j += 256) ((u4 *)s_stage)[j] = ((const u4 *)xr)[j];
    } else {
      for (int j = tid; j < K; j += 256) s_stage[j] = xr[j];
    }
    if (a == 0) {
      // The codes of the first GV_PIPE items are requested only now: while
      // the HBM queues are still empty the activations arrive quickly, and
      // the code latency then overlaps the gather.
#pragma unroll
      for (int s = 0; s < GV_PIPE; ++s) {
        const int lu = gf_load_unit(ul, i_end);
        const uint8_t *ub = lu >= 0 ? codes0 + (size_t)lu * UNIT_BYTES : w.base;
        ring[s] = load_item<true>(ub, lane);
        ++ul;
      }
    }
    __syncthreads();
    // The wave's first GF_PRE_UNITS gather units side by side (unrolled, so
    // that their LDS reads and wave reductions overlap), two at a time and
    // the remaining three together when the wave has them; slots past the
    // wave's units read a clamped unit and store nothing.
    const int npre = min(g_hi - g_lo + 1, GF_PRE_UNITS);  // may be <= 0
    auto gather_group = [&](auto J0, auto NJ) __attribute__((always_inline)) {
      constexpr int j0 = decltype(J0)::value, nj = decltype(NJ)::value;
      uint32_t pr[nj][4], mx[nj];
#pragma unroll
      for (int jj = 0; jj < nj; ++jj) mx[jj] = gather_pairs(pvec[j0 + jj], g_lo + j0 + jj, pr[jj]);
#pragma unroll
      for (int jj = 0; jj < nj; ++jj) mx[jj] = wave_max_bits(mx[jj]);
#pragma unroll
      for (int jj = 0; jj < nj; ++jj)
        if (j0 + jj < npre) gather_store(a, g_lo + j0 + jj, pr[jj], mx[jj]);
    };
    static_assert(GF_PRE_UNITS == 5, "gather groups cover 2 + 3 units");
    if (npre > 0) gather_group(std::integral_constant<int, 0>(), std::integral_constant<int, 2>());
    if (npre > 2) gather_group(std::integral_constant<int, 2>(), std::integral_constant<int, 3>());
    // units beyond the prefetched ones (k > 4 * GF_PRE_UNITS * 512 only)
    for (int uu = g_lo + GF_PRE_UNITS; uu <= g_hi; ++uu) {
      const u4 pv = *(const u4 *)(perm + uu * UNIT_SLOTS + 8 * lane);
      uint32_t pr[4];
      const uint32_t mxb = gather_pairs(pv, uu, pr);
      gather_store(a, uu, pr, wave_max_bits(mxb));
    }
  }
  if constexpr (BD == 8) {
    // the 8 direction copies go over the staging row, now that every gather
    // has read it
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = tid, cp = (q + row) & 7;
      *(u4 *)(smem + gf_off_d(BD) + row * 128 + cp * 16) = drow;
    }
  }
  __syncthreads();  // gathered activations, scales and tables are visible

  // lane 4b + j reads activation row j (row 0 when j >= M) of code column
  // 16*ci + b of the current unit
  const int jl = lane & 3, bl = lane >> 2;
  const uint8_t *xa = (const uint8_t *)(s_xp + (size_t)(jl < M ? jl : 0) * Kp) + 16 * bl;
  float acc[4][M];
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
#pragma unroll
    for (int a = 0; a < M; ++a) acc[ri][a] = 0.f;
  const uint32_t lane4 = (uint32_t)lane << 2;
  const uint32_t loff = (uint32_t)(lane & 7) << 4;  // bd = 8: the lane's copy
  uint32_t dad0[4], dad1[4];  // bd <= 7: byte 0 = the lane's copy * 16
  uint32_t rad0[4], rad1[4];  // bd <= 7: byte 0 = 4 * lane
#pragma unroll
  for (int ri = 0; ri < 4; ++ri) {
    dad0[ri] = dad1[ri] = (uint32_t)(lane & 15) << 4;
    rad0[ri] = rad1[ri] = lane4;
  }

  auto step = [&](const ItemCodes &c, int u) __attribute__((always_inline)) {
    // items are scheduled one at a time: interleaving several items only
    // raises register pressure past the occupancy target
    __builtin_amdgcn_sched_barrier(0);
    float tmp[4][M];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
      for (int a = 0; a < M; ++a) tmp[ri][a] = 0.f;
    gf_item<M, BD>(c, xa + (size_t)u * (UNIT_CODES * 16), dad0, dad1, rad0, rad1, loff, lane4, tmp);
#pragma unroll
    for (int a = 0; a < M; ++a) {
      const float sc = s_scale[u * M + a];
#pragma unroll
      for (int ri = 0; ri < 4; ++ri) acc[ri][a] = __builtin_fmaf(tmp[ri][a], sc, acc[ri][a]);
    }
  };

  // The wave's sums of tile t: over the 16 code columns of each lane group
  // (lanes with equal j) into the (t, wave) slot, then cleared.
  auto flush = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
#pragma unroll
      for (int a = 0; a < M; ++a) {
        float v = acc[ri][a];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 4) s_red[(((t * GV_WAVES + wv) * 4 + ri) * M + a) * 4 + lane] = v;
        acc[ri][a] = 0.f;
      }
    }
  };

  // Items of the wave: i_begin .. i_end-1 (slot (i - i_begin) % GV_PIPE),
  // unit cu of tile ct.  While a later chunk exists, every processed slot
  // is refilled at once (unconditional loads, dummy address past the end);
  // the last chunk has no refills.
  int i = i_begin;
  int ct = i_begin / U, cu = i_begin - ct * U;
  auto advance = [&]() __attribute__((always_inline)) {
    ++i;
    if (++cu == U) {
      flush(ct);
      ++ct;
      cu = 0;
    }
  };
  while (i + GV_PIPE < i_end) {
#pragma unroll
    for (int s = 0; s < GV_PIPE; ++s) {
      step(ring[s], cu);
      advance();
      const int lu = gf_load_unit(ul, i_end);
      const uint8_t *ub = lu >= 0 ? codes0 + (size_t)lu * UNIT_BYTES : w.base;
      ring[s] = load_item<true>(ub, lane);
      ++ul;
    }
  }
#pragma unroll
  for (int s = 0; s < GV_PIPE; ++s) {
    if (i < i_end) {
      step(ring[s], cu);
      advance();
    }
  }
  if (cu != 0) flush(ct);  // the run ends inside a tile

  // sum over the waves of each tile, in wave order
  __syncthreads();
  for (int o = tid; o < Reff * 16 * M; o += 256) {
    const int t = o / (16 * M), a = (o / 16) % M, row = o & 15;
    const int ri = row >> 2, j = row & 3;
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < GV_WAVES; ++p) sum += s_red[(((t * GV_WAVES + p) * 4 + ri) * M + a) * 4 + j];
    const int n = (rt0 + t) * 16 + row;
    if (n < w.n) store_out(y, (size_t)a * ldy + n, sum, ydt);
  }
}

// Occupancy: three 256-thread blocks per CU at m = 1 (the tables, activations
// and staging row of a 2560..9728-wide matrix fit 3x in LDS); at m >= 2 the
// permuted activation rows already limit LDS to one or two blocks per CU, so
// the register budget is relaxed accordingly.
#define SVQ_GEMV_OCCUPANCY(M) \
  __attribute__((amdgpu_waves_per_eu((M) == 1 ? 3 : ((M) == 2 ? 2 : 1))))
// Occupancy: three 256-thread blocks per CU (the tables, activations and
// staging row of a 2560..9728-wide matrix fit 3x in LDS).
template <bool XVEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void gemv_fused_kernel(GemvBatch b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int j = find_job(b.starts, b.count);
  const GemvJob &jb = b.job[j];
  const int rt0 = ((int)blockIdx.x - b.starts.first[j]) * jb.R;
  const int Reff = min(jb.R, jb.w.n_tiles - rt0);
  if (jb.w.bd >= 8)
    gemv_fused_block<1, XVEC, 8>(jb.w, jb.x, jb.ldx, jb.y, jb.ldy, b.ydt, rt0, jb.R, Reff, smem);
  else if (jb.w.bd == 7)
    gemv_fused_block<1, XVEC, 7>(jb.w, jb.x, jb.ldx, jb.y, jb.ldy, b.ydt, rt0, jb.R, Reff, smem);
  else
    gemv_fused_block<1, XVEC, 6>(jb.w, jb.x, jb.ldx, jb.y, jb.ldy, b.ydt, rt0, jb.R, Reff, smem);
}


template <bool XVEC>
static hipError_t launch_fused_x(GemvBatch &b, int blocks, size_t smem, hipStream_t s) {
  static const hipError_t lds_ok = check_no_static_lds(gemv_fused_kernel<XVEC>);
  if (lds_ok != hipSuccess) return lds_ok;
  hipError_t e = allow_smem(gemv_fused_kernel<XVEC>, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemv_fused_kernel<XVEC>), dim3(blocks), dim3(256), smem, s, b);
  return hipGetLastError();
}

hipError_t launch_gemv_fused(GemvBatch &b, int blocks, size_t smem, hipStream_t s) {
  return b.xvec ? launch_fused_x<true>(b, blocks, smem, s) : launch_fused_x<false>(b, blocks, smem, s);
}

// ---------------------------------------------------------------------------
// Mixture of experts (grouped form; routing is not on the pages and follows
// the usual top-k slot convention: slot q = t*topk + j)
// ---------------------------------------------------------------------------

// Per-slot fused GEMV (one activation row per slot): block (row-tile group,
// slot, projection), matrix = the slot's expert of that projection.
template <bool XVEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void moe_gemv_kernel(
    MoeGemvBatch mb, ExpertTable tab, const int32_t *__restrict__ ids, int x_per_slot, int topk, int ydt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int c = blockIdx.z;  // projection
  const MoeShape &sh = mb.sh[c];
  const int R = mb.R[c];
  const int rt0 = blockIdx.x * R;
  if (rt0 >= sh.n_tiles) return;  // block-uniform: the grid covers the widest projection
  const int q = blockIdx.y;
  const int e = ids[q];
  char *yq = (char *)mb.y[c] + (size_t)q * mb.ldy[c] * (ydt == 0 ? 2 : 4);
  if (e < 0 || e >= sh.num_experts) {  // block-uniform: the slot is skipped, its rows are zero
    for (int r = rt0 * 16 + (int)threadIdx.x; r < min(sh.n, (rt0 + R) * 16); r += 256)
      store_out(yq, (size_t)r, 0.f, ydt);
    return;
  }
  // projection c's experts are entries c * E .. c * E + E - 1 of the table
  const MatView w = expert_view(sh, tab, c * sh.num_experts + e);
  const int src = x_per_slot ? q : q / topk;
  const uint16_t *xr = mb.x[c] + (int64_t)src * mb.ldx[c];
  const int reff = min(R, w.n_tiles - rt0);
  if (w.bd >= 8)
    gemv_fused_block<1, XVEC, 8>(w, xr, mb.ldx[c], yq, mb.ldy[c], ydt, rt0, R, reff, smem);
  else if (w.bd == 7)
    gemv_fused_block<1, XVEC, 7>(w, xr, mb.ldx[c], yq, mb.ldy[c], ydt, rt0, R, reff, smem);
  else
    gemv_fused_block<1, XVEC, 6>(w, xr, mb.ldx[c], yq, mb.ldy[c], ydt, rt0, R, reff, smem);
}

// Routing for the grouped GEMM: counting sort of slots by expert and a list
// of work items (expert, first sorted row, end row), at most 16*BMT rows
// each.  Single block of 1024 threads.
//   ws_counts[E], ws_offsets[E+1], ws_sorted[S], ws_work[3*max_work], ws_nwork[1]
// Slots whose id is outside [0, E) are left out of the sort, and their output
// rows (n values each, y of type ydt with row stride ldy) are written as zeros.
__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t *__restrict__ ids, int S,
                                                         int E, int rows_per_item,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ sorted,
                                                         int32_t *__restrict__ work,
                                                         int32_t *__restrict__ nwork, void *y,
                                                         int64_t ldy, int n, int ydt) {
  __shared__ int32_t s_cnt[MAX_EXPERTS];
  __shared__ int32_t s_off[MAX_EXPERTS + 1];
  __shared__ int32_t s_fill[MAX_EXPERTS];
  __shared__ int32_t s_items[MAX_EXPERTS + 1];
  __shared__ int32_t s_wsum[2][MAX_EXPERTS / 64];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int q = t; q < S; q += 1024) {
    const int e = ids[q];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  // exclusive scans of the slot counts and of the work items per expert
  // (threads 0 .. MAX_EXPERTS-1, one expert each: a scan within each wave,
  // then the wave totals)
  int c = 0, it = 0, ci = 0, ii = 0;
  if (t < MAX_EXPERTS) {
    c = t < E ? s_cnt[t] : 0;
    it = (c + rows_per_item - 1) / rows_per_item;
    ci = c;
    ii = it;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int uc = __shfl_up(ci, d), ui = __shfl_up(ii, d);
      if ((t & 63) >= d) {
        ci += uc;
        ii += ui;
      }
    }
    if ((t & 63) == 63) {
      s_wsum[0][t >> 6] = ci;
      s_wsum[1][t >> 6] = ii;
    }
  }
  __syncthreads();
  if (t < MAX_EXPERTS) {
    int bc = 0, bi = 0;
    for (int w = 0; w < (t >> 6); ++w) {
      bc += s_wsum[0][w];
      bi += s_wsum[1][w];
    }
    if (t < E) {
      s_off[t] = bc + ci - c;
      s_items[t] = bi + ii - it;
      s_fill[t] = 0;
    }
    if (t == E - 1) {
      s_off[E] = bc + ci;
      s_items[E] = bi + ii;
      *nwork = bi + ii;
    }
  }
  __syncthreads();
  for (int e = t; e < E; e += 1024) counts[e] = s_cnt[e];
  for (int e = t; e <= E; e += 1024) offsets[e] = s_off[e];
  for (int q = t; q < S; q += 1024) {
    const int e = ids[q];
    if (e >= 0 && e < E) {
      const int pos = s_off[e] + atomicAdd(&s_fill[e], 1);
      sorted[pos] = q;
    } else {
      for (int c = 0; c < n; ++c) store_out((char *)y + (size_t)q * ldy * (ydt == 0 ? 2 : 4), (size_t)c, 0.f, ydt);
    }
  }
  // an expert's rows split into its work items as evenly as possible (sizes
  // differ by at most one, each <= rows_per_item)
  for (int e = t; e < E; e += 1024) {
    const int n_items = s_items[e + 1] - s_items[e], cnt = s_off[e + 1] - s_off[e];
    for (int c = 0; c < n_items; ++c) {
      const int wi = s_items[e] + c;
      work[3 * wi + 0] = e;
      work[3 * wi + 1] = s_off[e] + (int)((int64_t)c * cnt / n_items);
      work[3 * wi + 2] = s_off[e] + (int)((int64_t)(c + 1) * cnt / n_items);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------


// ---------------------------------------------------------------------------
// MoE launcher.  Workspace layout depends on the path:
//   exact (m*topk <= MOE_EXACT_MAX_SLOTS): none (one fused per-slot launch
//            for all projections of the call)
//   grouped: counts[E], offsets[E+1], sorted[S], work[3*max_work], nwork,
//            fragment-ordered activations (moe_sb_xa_bytes); the routing
//            is done by the prep launch up to MOE_FUSED_MAX_SLOTS slots
//            (counts and offsets unused), by moe_route_kernel beyond.  Up to
//            MOE_FUSED_MAX_SLOTS one prep and one product launch serve every
//            projection of the call (one fragment area each, after the
//            shared routing tables); beyond, the projections run one after
//            another on the same workspace (its size is the largest any of
//            them needs).
// ---------------------------------------------------------------------------
constexpr int MOE_EXACT_MAX_SLOTS = 64;

// Layout of one projection's experts (all share n, k and the region
// offsets; bd may differ, and lives in the expert table).
static MoeShape moe_shape(const svq_handle *experts, int32_t E) {
  const svq_handle &h0 = experts[0];
  MoeShape sh;
  sh.off_dtab = (uint32_t)h0.off_dtab;
  sh.off_rtab = (uint32_t)h0.off_rtab;
  sh.off_btab = (uint32_t)h0.off_btab;
  sh.off_xtab = (uint32_t)h0.off_xtab;
  sh.off_perm = (uint32_t)h0.off_perm;
  sh.off_codes = h0.off_codes;
  sh.n = h0.n;
  sh.k = h0.k;
  sh.n_tiles = h0.n_tiles;
  sh.units = h0.units;
  sh.num_experts = E;
  return sh;
}

// The grouped path for `count` projections in one prep and one product
// launch (count > 1 only with the routing inside the prep launch).
// Workspace: the routing tables, then each projection's staged activations.
static hipError_t launch_moe_grouped(const svq_handle *const *experts, int count, int32_t E,
                                     const void *const *x, const int64_t *ldx, int32_t x_per_slot,
                                     const int32_t *ids, int S, int32_t topk, void *const *y,
                                     const int64_t *ldy, int ydt, void *ws, size_t ws_bytes,
                                     hipStream_t s, size_t *need) {
  const int rows_per_item = MOE_SB_ROWS;
  const int max_work = (S + rows_per_item - 1) / rows_per_item + E;
  size_t off = 0;
  const size_t o_counts = off;
  off += align256((size_t)E * 4);
  const size_t o_offsets = off;
  off += align256((size_t)(E + 1) * 4);
  const size_t o_sorted = off;
  off += align256((size_t)S * 4);
  const size_t o_work = off;
  off += align256((size_t)max_work * 12);
  const size_t o_nwork = off;
  off += 256;
  size_t o_xb[MOE_BATCH_MAX];
  for (int c = 0; c < count; ++c) {
    o_xb[c] = off;
    off += align256(moe_sb_xa_bytes(max_work, experts[c][0].units));
  }
  *need = off;
  if (!ws) return hipSuccess;
  if (ws_bytes < *need) return hipErrorInvalidValue;
  uint8_t *base = (uint8_t *)ws;
  int32_t *counts = (int32_t *)(base + o_counts), *offsets = (int32_t *)(base + o_offsets);
  int32_t *sorted = (int32_t *)(base + o_sorted), *work = (int32_t *)(base + o_work);
  int32_t *nwork = (int32_t *)(base + o_nwork);
  MoeSbBatch b;
  std::memset(&b, 0, sizeof(b));
  ExpertTable tab;
  std::memset(&tab, 0, sizeof(tab));
  b.count = count;
  b.vec = 1;
  b.yvec = 1;
  const int esz = ydt == 0 ? 2 : 4;
  for (int c = 0; c < count; ++c) {
    b.p[c].sh = moe_shape(experts[c], E);
    b.p[c].x = (const uint16_t *)x[c];
    b.p[c].ldx = ldx[c];
    b.p[c].xa = base + o_xb[c];
    b.p[c].y = y[c];
    b.p[c].ldy = ldy[c];
    if (!((uintptr_t)x[c] % 16 == 0 && ldx[c] % 8 == 0)) b.vec = 0;
    if (!((uintptr_t)y[c] % 16 == 0 && (ldy[c] * esz) % 16 == 0)) b.yvec = 0;
    for (int e = 0; e < E; ++e) {
      tab.base[c * E + e] = (const uint8_t *)experts[c][e].dev;
      tab.bd[c * E + e] = (uint8_t)experts[c][e].bd;
    }
  }
  MoeRoute route;
  route.ids = nullptr;
  route.slots = S;
  route.ydt = ydt;
  if (S <= MOE_FUSED_MAX_SLOTS) {
    route.ids = ids;  // the prep launch does the routing
  } else {
    if (count != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(1024), 0, s, ids, S, E, rows_per_item, counts,
                       offsets, sorted, work, nwork, y[0], ldy[0], b.p[0].sh.n, ydt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_moe_sb(b, tab, x_per_slot, topk, route, work, nwork, sorted, max_work, ydt, s);
}

hipError_t launch_moe(const svq_handle *const *experts, int32_t count, int32_t E, const void *const *x,
                      const int64_t *ldx, int32_t x_per_slot, const int32_t *ids, int64_t m,
                      int32_t topk, void *const *y, const int64_t *ldy, int ydt, void *ws,
                      size_t ws_bytes, hipStream_t s, size_t *need) {
  const int S = (int)(m * topk);
  if (count < 1 || count > MOE_BATCH_MAX || count * E > MAX_EXPERTS) return hipErrorInvalidValue;
  if (S > MOE_EXACT_MAX_SLOTS) {
    // one prep and one product launch for all projections while the prep
    // does the routing; beyond, each projection with its own routing launch
    if (S <= MOE_FUSED_MAX_SLOTS)
      return launch_moe_grouped(experts, count, E, x, ldx, x_per_slot, ids, S, topk, y, ldy, ydt, ws,
                                ws_bytes, s, need);
    size_t most = 0;
    for (int c = 0; c < count; ++c) {
      size_t nc = 0;
      const hipError_t e =
          launch_moe_grouped(&experts[c], 1, E, ws ? &x[c] : nullptr, ws ? &ldx[c] : nullptr, x_per_slot,
                             ids, S, topk, ws ? &y[c] : nullptr, ws ? &ldy[c] : nullptr, ydt, ws, ws_bytes,
                             s, &nc);
      if (e != hipSuccess) return e;
      most = nc > most ? nc : most;
    }
    *need = most;
    return hipSuccess;
  }
  *need = 256;
  if (!ws) return hipSuccess;
  MoeGemvBatch mb;
  std::memset(&mb, 0, sizeof(mb));
  ExpertTable tab;
  std::memset(&tab, 0, sizeof(tab));
  bool xvec = true;
  size_t smem = 0;
  int gx = 1;
  for (int c = 0; c < count; ++c) {
    const MoeShape sh = moe_shape(experts[c], E);
    // row tiles per block: about 5 units per wave to amortise the gather,
    // while the launch keeps >= 256 blocks
    constexpr int ITEMS_PER_WAVE = 5;
    int R = sh.units <= ITEMS_PER_WAVE ? 4 : (sh.units <= 2 * ITEMS_PER_WAVE ? 2 : 1);
    while (R > 1 && ((sh.n_tiles + R - 1) / R) * S < 256) R /= 2;
    for (int e = 0; e < E; ++e) {
      tab.base[c * E + e] = (const uint8_t *)experts[c][e].dev;
      tab.bd[c * E + e] = (uint8_t)experts[c][e].bd;
      const size_t b = gemv_fused_smem_bytes(sh.k, sh.units, experts[c][e].bd, R);
      smem = b > smem ? b : smem;
    }
    mb.sh[c] = sh;
    mb.x[c] = (const uint16_t *)x[c];
    mb.ldx[c] = ldx[c];
    mb.y[c] = y[c];
    mb.ldy[c] = ldy[c];
    mb.R[c] = R;
    if (((((uintptr_t)x[c]) | ((uintptr_t)ldx[c] * 2)) & 15) != 0) xvec = false;
    const int g = (sh.n_tiles + R - 1) / R;
    gx = g > gx ? g : gx;
  }
  if (smem > GV_LDS_LIMIT) return hipErrorInvalidValue;
  static const hipError_t lds_ok_t = check_no_static_lds(moe_gemv_kernel<true>);
  static const hipError_t lds_ok_f = check_no_static_lds(moe_gemv_kernel<false>);
  if ((xvec ? lds_ok_t : lds_ok_f) != hipSuccess) return xvec ? lds_ok_t : lds_ok_f;
  hipError_t e = xvec ? allow_smem(moe_gemv_kernel<true>, smem) : allow_smem(moe_gemv_kernel<false>, smem);
  if (e != hipSuccess) return e;
  const dim3 grid(gx, S, count);
  if (xvec)
    hipLaunchKernelGGL(moe_gemv_kernel<true>, grid, dim3(256), smem, s, mb, tab, ids, x_per_slot, topk, ydt);
  else
    hipLaunchKernelGGL(moe_gemv_kernel<false>, grid, dim3(256), smem, s, mb, tab, ids, x_per_slot, topk, ydt);
  return hipGetLastError();
}

}  // namespace svq
