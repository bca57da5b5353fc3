// Device-side helpers shared by the kernel translation units of libsvq.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "svq_internal.h"

namespace svq {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN): gfx950
// converts in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// y[i] = v as bf16 (ydt 0, RNE) or fp32 (ydt 1).
__device__ __forceinline__ void store_out(void *y, size_t i, float v, int ydt) {
  if (ydt == 0) ((uint16_t *)y)[i] = f32_to_bf16_bits(v);
  else ((float *)y)[i] = v;
}

// The 36 code bytes one lane record holds (16 codes, see the unit layout).
struct ItemCodes {
  u4 S, L;
  uint32_t H;
};

// Lane record `rec` of the coded unit at ub.  NT: non-temporal loads, for
// codes that are read exactly once (a streaming hint; on MI355X it raises
// the HBM rate of a launch that streams all of its codes about twofold).
template <bool NT = false>
__device__ __forceinline__ ItemCodes load_item(const uint8_t *ub, int rec) {
  ItemCodes c;
  if constexpr (NT) {
    c.S = __builtin_nontemporal_load((const u4 *)(ub + PLANE_SIGN + 16 * rec));
    c.L = __builtin_nontemporal_load((const u4 *)(ub + PLANE_LOW + 16 * rec));
    c.H = __builtin_nontemporal_load((const uint32_t *)(ub + PLANE_HIGH + 4 * rec));
  } else {
    c.S = *(const u4 *)(ub + PLANE_SIGN + 16 * rec);
    c.L = *(const u4 *)(ub + PLANE_LOW + 16 * rec);
    c.H = *(const uint32_t *)(ub + PLANE_HIGH + 4 * rec);
  }
  return c;
}

// Record-crossing code loads of the 16x16x32 MFMA paths (small batch and
// grouped MoE).  Lane L = 16s + 4b0 + j takes, for MFMA f = 4ci + q, the
// code at row 4b0 + j, column 16ci + 4s + q of a unit: code 4b0 + ci of
// lane record 16s + 4q + j.
// The code bytes one lane needs for one unit:
// for each q, the 16 sign bytes, index-low dword b0 and index-high dword of
// lane record 16s + 4q + j.
struct SbCodes {
  u4 S[4];
  uint32_t L[4], H[4];
};

// Lane offsets of those bytes within a unit, for q = 0: record 16s + j
// (the records of q > 0 lie 4q records further).
struct SbOffs {
  uint32_t S, L, H;
};

__device__ __forceinline__ SbCodes sb_load_codes(const uint8_t *ub, const SbOffs &o) {
  SbCodes c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c.S[q] = __builtin_nontemporal_load((const u4 *)(ub + PLANE_SIGN + 64 * q + o.S));
    c.L[q] = __builtin_nontemporal_load((const uint32_t *)(ub + PLANE_LOW + 64 * q + o.L));
    c.H[q] = __builtin_nontemporal_load((const uint32_t *)(ub + PLANE_HIGH + 16 * q + o.H));
  }
  return c;
}

// Per-lane shift amounts of code 4b0 + ci (ci = 0..3): sign carriers
// (S << (4b0 + ci) brings the code's pair signs to bits 15 and 31) and the
// index-high bits (at 8b0 + 2ci of the record's high dword).
struct SbShifts {
  uint32_t sg[4], hi[4];
};

// The job of a batched launch that owns this block (see JobStarts): the
// number of later job starts at or below blockIdx.x.
__device__ __forceinline__ int find_job(const JobStarts &st, int count) {
  const int blk = (int)blockIdx.x;
  int j = 0;
#pragma unroll
  for (int t = 1; t < GV_MAX_JOBS; ++t) j += (t < count && blk >= st.first[t]) ? 1 : 0;
  return j;
}

// Matrix view of expert e of a MoE projection.
__device__ __forceinline__ MatView expert_view(const MoeShape &sh, const ExpertTable &tab, int e) {
  MatView v;
  v.base = tab.base[e];
  v.off_dtab = sh.off_dtab;
  v.off_rtab = sh.off_rtab;
  v.off_btab = sh.off_btab;
  v.off_xtab = sh.off_xtab;
  v.off_perm = sh.off_perm;
  v.off_codes = sh.off_codes;
  v.n = sh.n;
  v.k = sh.k;
  v.bd = tab.bd[e];
  v.n_tiles = sh.n_tiles;
  v.units = sh.units;
  return v;
}

// Opt a kernel into more than 64 KB of dynamic LDS.
template <typename Kern>
static hipError_t allow_smem(Kern k, size_t bytes) {
  if (bytes > 64 * 1024)
    return hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
  return hipSuccess;
}

}  // namespace svq
