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
// * Exact (m <= 4).  The 8 signed fp16 direction values of a code are an
//   MFMA B operand as they come out of LDS (sign flips are exact), the
//   activations (fp16 after an exact power-of-two scale) sit in a
//   block-diagonal A operand, so v_mfma_f32_16x16x32_f16 returns, in the very
//   lane that decoded the code, the code's 8-term dot product per activation
//   row.  The radius multiply is then applied per code in fp32 (fp16 radius
//   x fp32 dot, fused multiply-add), so the decoded weight R*D is never
//   rounded.
// * bf16 (m > 4).  A code decodes to 8 bf16 weights RNE_bf16(R*D) with its
//   signs from a 1024-row table (one row per direction/radius index), which
//   is the B operand of v_mfma_f32_16x16x32_bf16; activations are the
//   A operand.
#include "svq_internal.h"
#include "../../include/svq.h"

namespace svq {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void *y, size_t i, float v, int ydt) {
  if (ydt == 0) ((uint16_t *)y)[i] = f32_to_bf16_bits(v);
  else ((float *)y)[i] = v;
}

// Apply the 8 sign bits of code i (carried in S, see svq_internal.h) to the
// 8 fp16/bf16 values in D: the sign bit of every 16-bit half is bit 15/31.
__device__ __forceinline__ u4 apply_signs(u4 D, u4 S, int i) {
  const uint32_t M = 0x80008000u;
  D[0] ^= (S[0] << i) & M;
  D[1] ^= (S[1] << i) & M;
  D[2] ^= (S[2] << i) & M;
  D[3] ^= (S[3] << i) & M;
  return D;
}

// 10-bit index of code i from the two index planes.
__device__ __forceinline__ uint32_t code_index(u4 L, uint32_t H, int i) {
  uint32_t lo = (L[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  return lo | (((H >> (2 * i)) & 3u) << 8);
}

// ---------------------------------------------------------------------------
// Exact path (m <= 4), fused: gather + scale + decode-and-multiply in one
// kernel.
// ---------------------------------------------------------------------------
//
// A block owns R consecutive 16-row tiles of one matrix and all of its K.
// Prologue: the block stages each activation row in LDS, and its 4 waves
// gather the permuted slots (Fig. 6 caption: a subvector multiplies eight
// reordered activations) unit by unit.  Each 512-slot unit u gets its own
// exact power-of-two scale 2^e_u with max|x_u| * 2^e_u in [2^14, 2^15), so
// the fp16 copy is exact for every bf16 value above 2^-17 * max|x_u|; the
// scale is undone once per (row tile, unit) in fp32.
//
// Main loop: work item t = rt*U + u (row tile rt, unit u) goes to wave
// t mod 4.  The item's 2304 code bytes are contiguous and prefetched one
// item ahead.  MFMA mapping for K-block i of the unit (4 codes):
//   B[k][n]: lane L holds the signed direction row of its code (row n =
//            L & 15, code group q = L >> 4), k = 8q..8q+7.
//   A[m][k]: m = 4q' + a; lane L holds A[L & 15][k-group L >> 4], which is
//            non-zero only on the "diagonal" lanes (L & 15) >> 2 == L >> 4,
//            where it is the 8 scaled activations of code 4i + q for
//            activation row a = L & 3 (read from LDS under the exec mask,
//            so the other lanes keep their zeros).
//   C[m][n]: lane L receives rows 4q + a of column L & 15: the dot products
//            of exactly the code it decoded, one per activation row.
// The radius multiply R[r] * dot is an fp32 FMA per code; R*D is never
// rounded.  Partial sums meet in LDS at the end of the block.

constexpr int GV_WAVES = 4;
constexpr int GV_MAX_R = 4;
// LDS: direction table (GV_REP copies interleaved: row b, copy j at
// b*16*GV_REP + 16*j; lane L reads copy L % GV_REP), radius table, unit
// scales, cross-wave partial sums, then the permuted activations and the
// staging row.
constexpr int GV_REP = 1;
constexpr int GV_DTAB_BYTES = 256 * 16 * GV_REP;
constexpr int GV_OFF_RTAB = GV_DTAB_BYTES;
constexpr int GV_OFF_MAX = GV_OFF_RTAB + 256;
constexpr int GV_OFF_RED = GV_OFF_MAX + 128 * 4 * 4;  // [U <= 128][M <= 4] scales
constexpr int GV_SMEM_FIXED = GV_OFF_RED + 4096;
constexpr int GV_PRE_UNITS = 5;   // permutation vectors prefetched per wave
constexpr int GV_STAGE_BATCH = 5; // x loads in flight per thread while staging

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

template <int M>
__device__ void gemv_fused_block(const MatView &w, const uint16_t *__restrict__ x, int64_t ldx,
                                 void *__restrict__ y, int64_t ldy, int ydt, int rt0, int R,
                                 uint8_t *smem) {
  u4 *s_dtab = (u4 *)smem;
  _Float16 *s_rtab = (_Float16 *)(smem + GV_OFF_RTAB);
  float *s_scale = (float *)(smem + GV_OFF_MAX);          // [U][M] 2^-e per unit
  float *s_red = (float *)(smem + GV_OFF_RED);            // [W][GV_MAX_R][M][16]
  uint16_t *s_xp = (uint16_t *)(smem + GV_SMEM_FIXED);    // [M][Kp] fp16
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int U = w.units, Kp = U * UNIT_SLOTS, K = w.k;
  uint16_t *s_stage = s_xp + (size_t)M * Kp;              // [K] bf16
  const int items = R * U;
  const uint8_t *codes0 = w.base + w.off_codes + (size_t)rt0 * U * UNIT_BYTES;
  // wave wv owns the contiguous run of work items [t_begin, t_end) in
  // unit-major order t = u*R + rt
  const int per = (items + GV_WAVES - 1) / GV_WAVES;
  const int t_begin = wv * per;
  const int t_end = min(items, t_begin + per);

  // Global loads of the prologue are issued first, in the order they are
  // needed (vmcnt counts in order): the direction table row of this thread,
  // the permutation vectors of the wave's units, the first activation row,
  // and only then the first work item's codes, whose HBM latency overlaps
  // the rest of the prologue.
  const int u_lo = t_begin / R, u_hi = t_end > t_begin ? (t_end - 1) / R : u_lo - 1;
  const u4 drow = ((const u4 *)(w.base + w.off_dtab))[tid];
  const uint16_t *perm = (const uint16_t *)(w.base + w.off_perm);
  u4 pvec[GV_PRE_UNITS];
#pragma unroll
  for (int j = 0; j < GV_PRE_UNITS; ++j) {
    const int uu = u_lo + j;
    pvec[j] = uu <= u_hi ? *(const u4 *)(perm + uu * UNIT_SLOTS + 8 * lane) : (u4){0u, 0u, 0u, 0u};
  }
  const int n8 = K / 8;
  const bool x_vec = ((((uintptr_t)x) | ((uintptr_t)ldx * 2)) & 15) == 0;
  u4 xv[GV_STAGE_BATCH];
  if (x_vec) {
#pragma unroll
    for (int b = 0; b < GV_STAGE_BATCH; ++b) {
      const int j = tid + 256 * b;
      xv[b] = j < n8 ? ((const u4 *)x)[j] : (u4){0u, 0u, 0u, 0u};
    }
  }
  u4 S = (u4){0u, 0u, 0u, 0u}, L = S;
  uint32_t H = 0;
  int u = u_lo, rt = t_begin - u_lo * R;
  if (t_begin < t_end) {
    const uint8_t *ub = codes0 + (size_t)(rt * U + u) * UNIT_BYTES;
    S = *(const u4 *)(ub + PLANE_SIGN + 16 * lane);
    L = *(const u4 *)(ub + PLANE_LOW + 16 * lane);
    H = *(const uint32_t *)(ub + PLANE_HIGH + 4 * lane);
  }
#pragma unroll
  for (int j = 0; j < GV_REP; ++j) s_dtab[tid * GV_REP + j] = drow;
  if (tid < 16) s_rtab[tid] = ((const _Float16 *)(w.base + w.off_rtab))[tid];

  // The units this wave multiplies: its items t in [t_begin, t_end) are
  // unit-major, so they cover units u_lo..u_hi.

  // One activation row at a time: stage it in LDS (one barrier), then every
  // wave gathers the permuted slots of its own units (Fig. 6 "reordered
  // activations") and converts them to fp16 with a per-unit scale 2^e,
  // chosen so that max|x_unit| * 2^e lies in [2^14, 2^15): exact for every
  // bf16 value above 2^-17 of the unit's maximum.  Waves that share a unit
  // write identical values.
  for (int a = 0; a < M; ++a) {
    const uint16_t *xr = x + (int64_t)a * ldx;
    if (a > 0) __syncthreads();  // previous row's gathers are done
    if (x_vec) {
      for (int j0 = tid; j0 < n8; j0 += 256 * GV_STAGE_BATCH) {
        if (a > 0 || j0 != tid) {
#pragma unroll
          for (int b = 0; b < GV_STAGE_BATCH; ++b) {
            const int j = j0 + 256 * b;
            xv[b] = j < n8 ? ((const u4 *)xr)[j] : (u4){0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
        for (int b = 0; b < GV_STAGE_BATCH; ++b) {
          const int j = j0 + 256 * b;
          if (j < n8) ((u4 *)s_stage)[j] = xv[b];
        }
      }
    } else {
      for (int j = tid; j < K; j += 256) s_stage[j] = xr[j];
    }
    __syncthreads();
    for (int uu = u_lo; uu <= u_hi; ++uu) {
      const int p0 = uu * UNIT_SLOTS + 8 * lane;
      u4 pv;
      const int j = uu - u_lo;
      if (j < GV_PRE_UNITS) {
        pv = pvec[0];
#pragma unroll
        for (int jj = 1; jj < GV_PRE_UNITS; ++jj)
          if (jj == j) pv = pvec[jj];
      } else {
        pv = *(const u4 *)(perm + p0);
      }
      float v[8];
      float mx = 0.f;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const uint32_t c0 = pv[l] & 0xFFFFu, c1 = pv[l] >> 16;
        // perm is zero padded to the unit width, so c0, c1 < K always
        const float g0 = bf16_bits_to_f32(s_stage[c0]), g1 = bf16_bits_to_f32(s_stage[c1]);
        v[2 * l] = (p0 + 2 * l < K) ? g0 : 0.f;
        v[2 * l + 1] = (p0 + 2 * l + 1 < K) ? g1 : 0.f;
        mx = fmaxf(mx, fmaxf(fabsf(v[2 * l]), fabsf(v[2 * l + 1])));
      }
      mx = wave_max(mx);
      const int e = mx > 0.f ? 14 - ilogbf(mx) : 0;
      u4 h;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const _Float16 lo = (_Float16)ldexpf(v[2 * l], e), hi = (_Float16)ldexpf(v[2 * l + 1], e);
        h[l] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      ((u4 *)(s_xp + (size_t)a * Kp))[64 * uu + lane] = h;
      if (lane == 0) s_scale[uu * M + a] = ldexpf(1.f, -e);
    }
  }
  // the gathered activations of a unit are read back only by the wave that
  // wrote them (or an identical copy): a wave-level fence suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int q = lane >> 4;
  const int bd = w.bd;
  float acc[GV_MAX_R][M];
#pragma unroll
  for (int r = 0; r < GV_MAX_R; ++r)
#pragma unroll
    for (int a = 0; a < M; ++a) acc[r][a] = 0.f;
  u4 A[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) A[i] = (u4){0u, 0u, 0u, 0u};

  // Diagonal lanes of the block-diagonal A operand: (L & 15) >> 2 == L >> 4.
  //  M == 1: four K-blocks i = 4g + j (j = 0..3) are chained into one C;
  //          lane 20q + j carries code 4i + q of K-block j, so C row 4q + j
  //          of lane L (q = L >> 4) is the dot of the code that lane decoded
  //          for K-block 4g + j.
  //  M > 1:  one C per K-block; lane 20q + a carries row a of code 4i + q,
  //          and C row 4q + a is that code's dot for activation row a.
  const bool diag = (((lane & 15) >> 2) == q) && (M == 1 || (lane & 3) < M);
  const int a_lane = M == 1 ? 0 : (lane & 3);
  const int j_lane = lane & 3;  // M == 1: which K-block of the group
  const u4 *xa = (const u4 *)(s_xp + (size_t)(diag ? a_lane : 0) * Kp) + q;
  const u4 *dtab_l = s_dtab + (lane & (GV_REP - 1));  // this lane's replica

  for (int t = t_begin; t < t_end; ++t) {
    // prefetch the next item's codes
    int un = u, rn = rt + 1;
    if (rn == R) {
      rn = 0;
      ++un;
    }
    u4 S2 = S, L2 = L;
    uint32_t H2 = H;
    if (t + 1 < t_end) {
      const uint8_t *ub = codes0 + (size_t)(rn * U + un) * UNIT_BYTES;
      S2 = *(const u4 *)(ub + PLANE_SIGN + 16 * lane);
      L2 = *(const u4 *)(ub + PLANE_LOW + 16 * lane);
      H2 = *(const uint32_t *)(ub + PLANE_HIGH + 4 * lane);
    }
    float tmp[M];
#pragma unroll
    for (int a = 0; a < M; ++a) tmp[a] = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (M == 1) {
        // lane 20q + j feeds only K-block 4g + j of the group; every other
        // lane keeps zeros in A[j]
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (diag && j_lane == j) A[j] = xa[64 * u + 4 * (4 * g + j)];
      } else if (diag) {
#pragma unroll
        for (int j = 0; j < 4; ++j) A[j] = xa[64 * u + 16 * g + 4 * j];
      }
      if (M == 1) {
        f4 C = (f4){0.f, 0.f, 0.f, 0.f};
        float Rv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          const uint32_t idx = code_index(L, H, i);
          const u4 D = apply_signs(dtab_l[(idx & 0xFFu) * GV_REP], S, i);
          C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, A[j]),
                                                     __builtin_bit_cast(h8, D), C, 0, 0, 0);
          Rv[j] = (float)s_rtab[idx >> bd];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) tmp[0] = __builtin_fmaf(Rv[j], C[j], tmp[0]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          const uint32_t idx = code_index(L, H, i);
          const u4 D = apply_signs(dtab_l[(idx & 0xFFu) * GV_REP], S, i);
          const f4 C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, A[j]),
                                                              __builtin_bit_cast(h8, D),
                                                              (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          const float Rv = (float)s_rtab[idx >> bd];
#pragma unroll
          for (int a = 0; a < M; ++a) tmp[a] = __builtin_fmaf(Rv, C[a], tmp[a]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < M; ++a) {
      const float sc = s_scale[u * M + a];
#pragma unroll
      for (int r = 0; r < GV_MAX_R; ++r)
        if (r == rt) acc[r][a] = __builtin_fmaf(tmp[a], sc, acc[r][a]);
    }
    S = S2;
    L = L2;
    H = H2;
    u = un;
    rt = rn;
  }

#pragma unroll
  for (int r = 0; r < GV_MAX_R; ++r) {
#pragma unroll
    for (int a = 0; a < M; ++a) {
      float v = acc[r][a];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) s_red[((wv * GV_MAX_R + r) * M + a) * 16 + lane] = v;
    }
  }
  __syncthreads();
  for (int o = tid; o < R * M * 16; o += 256) {
    const int r = o / (M * 16), a = (o / 16) % M, row = o & 15;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < GV_WAVES; ++j) sum += s_red[((j * GV_MAX_R + r) * M + a) * 16 + row];
    const int n = (rt0 + r) * 16 + row;
    if (n < w.n) store_out(y, (size_t)a * ldy + n, sum, ydt);
  }
}

template <int M>
__global__ __launch_bounds__(256) void gemv_batched_kernel(GemvBatch b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int j = 0;
  while (j + 1 < b.count && (int)blockIdx.x >= b.job[j + 1].block_begin) ++j;
  const GemvJob &jb = b.job[j];
  const int rt0 = ((int)blockIdx.x - jb.block_begin) * jb.R;
  const int R = min(jb.R, jb.w.n_tiles - rt0);
  gemv_fused_block<M>(jb.w, jb.x, jb.ldx, jb.y, jb.ldy, b.ydt, rt0, R, smem);
}

size_t gemv_smem_bytes(int m, int k_max, int units_max) {
  return (size_t)GV_SMEM_FIXED + (size_t)m * units_max * UNIT_SLOTS * 2 + (size_t)k_max * 2;
}

template <typename Kern>
static hipError_t allow_smem(Kern k, size_t bytes) {
  if (bytes > 64 * 1024)
    return hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
  return hipSuccess;
}

hipError_t launch_gemv_batched(GemvBatch &b, int blocks, size_t smem, hipStream_t s) {
  hipError_t e = hipSuccess;
  switch (b.m) {
    case 1:
      e = allow_smem(gemv_batched_kernel<1>, smem);
      if (e == hipSuccess) hipLaunchKernelGGL(gemv_batched_kernel<1>, dim3(blocks), dim3(256), smem, s, b);
      break;
    case 2:
      e = allow_smem(gemv_batched_kernel<2>, smem);
      if (e == hipSuccess) hipLaunchKernelGGL(gemv_batched_kernel<2>, dim3(blocks), dim3(256), smem, s, b);
      break;
    case 3:
      e = allow_smem(gemv_batched_kernel<3>, smem);
      if (e == hipSuccess) hipLaunchKernelGGL(gemv_batched_kernel<3>, dim3(blocks), dim3(256), smem, s, b);
      break;
    default:
      e = allow_smem(gemv_batched_kernel<4>, smem);
      if (e == hipSuccess) hipLaunchKernelGGL(gemv_batched_kernel<4>, dim3(blocks), dim3(256), smem, s, b);
      break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------

// Block-level: xo[p] = xr[perm[p]] (bf16), zero for p >= k.  The row is
// staged in LDS (s_row, K entries) when stage != 0.  blockDim.x == 256.
__device__ void prep_bf16_row(const uint16_t *__restrict__ perm, int K, int Kp,
                              const uint16_t *__restrict__ xr, uint16_t *__restrict__ xo,
                              uint16_t *s_row, int stage) {
  if (stage) {
    for (int j = threadIdx.x; j < K; j += 256) s_row[j] = xr[j];
    __syncthreads();
    for (int p = threadIdx.x; p < Kp; p += 256) xo[p] = p < K ? s_row[perm[p]] : (uint16_t)0;
  } else {
    for (int p = threadIdx.x; p < Kp; p += 256) xo[p] = p < K ? xr[perm[p]] : (uint16_t)0;
  }
}

__global__ __launch_bounds__(256) void prep_bf16_kernel(MatView w, const uint16_t *__restrict__ x,
                                                         int64_t ldx, int m, uint16_t *__restrict__ xb,
                                                         int stage) {
  extern __shared__ uint16_t s_row[];
  const int r = blockIdx.x;
  const int Kp = w.units * UNIT_SLOTS;
  uint16_t *xo = xb + (size_t)r * Kp;
  if (r >= m) {
    for (int p = threadIdx.x; p < Kp; p += 256) xo[p] = 0;
    return;
  }
  prep_bf16_row((const uint16_t *)(w.base + w.off_perm), w.k, Kp, x + (int64_t)r * ldx, xo, s_row,
                stage);
}

// GEMM tile: wave wv of the block owns row tile rt (16 output rows) and BMT
// 16-row activation tiles starting at activation row m0 of xb (rows Kp
// apart).  Each decoded code (B operand) is reused across the BMT activation
// tiles.  Output row mm (m0 <= mm < m_end) goes to y row out_row(mm).
template <int BMT, typename RowMap>
__device__ void gemm_bf16_tile(const MatView &w, int rt, const uint16_t *__restrict__ xb, int m0,
                               int m_end, void *__restrict__ y, int64_t ldy, int ydt,
                               const u4 *s_btab, RowMap out_row) {
  const int lane = threadIdx.x & 63;
  const int Kp = w.units * UNIT_SLOTS;
  const uint8_t *tile = w.base + w.off_codes + (size_t)rt * w.units * UNIT_BYTES;
  const u4 *xrow = (const u4 *)(xb + (size_t)(m0 + (lane & 15)) * Kp) + (lane >> 4);
  const size_t xstride = (size_t)16 * Kp / 8;  // 16 rows, in u4 units

  f4 C[BMT];
#pragma unroll
  for (int t = 0; t < BMT; ++t) C[t] = (f4){0.f, 0.f, 0.f, 0.f};

  for (int u = 0; u < w.units; ++u) {
    const uint8_t *ub = tile + (size_t)u * UNIT_BYTES;
    const u4 S = *(const u4 *)(ub + PLANE_SIGN + 16 * lane);
    const u4 L = *(const u4 *)(ub + PLANE_LOW + 16 * lane);
    const uint32_t H = *(const uint32_t *)(ub + PLANE_HIGH + 4 * lane);
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const uint32_t idx = code_index(L, H, i);
      const u4 B = apply_signs(s_btab[idx], S, i);
#pragma unroll
      for (int t = 0; t < BMT; ++t) {
        const u4 A = xrow[t * xstride + 64 * u + 4 * i];
        C[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, A),
                                                       __builtin_bit_cast(b8, B), C[t], 0, 0, 0);
      }
    }
  }
  const int n = rt * 16 + (lane & 15);
  if (n >= w.n) return;
#pragma unroll
  for (int t = 0; t < BMT; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = m0 + 16 * t + 4 * (lane >> 4) + j;
      if (mm < m_end) store_out(y, (size_t)out_row(mm) * ldy + n, C[t][j], ydt);
    }
  }
}

struct IdentityRows {
  __device__ int operator()(int mm) const { return mm; }
};

template <int BMT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(MatView w, const uint16_t *__restrict__ xb,
                                                        int m, void *__restrict__ y, int64_t ldy,
                                                        int ydt) {
  __shared__ u4 s_btab[1024];
  const u4 *btab_g = (const u4 *)(w.base + w.off_btab);
  for (int j = threadIdx.x; j < 1024; j += 256) s_btab[j] = btab_g[j];
  __syncthreads();
  const int rt = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rt >= w.n_tiles) return;
  gemm_bf16_tile<BMT>(w, rt, xb, blockIdx.y * 16 * BMT, m, y, ldy, ydt, s_btab, IdentityRows{});
}

// ---------------------------------------------------------------------------
// Mixture of experts (grouped form; routing is not on the pages and follows
// the usual top-k slot convention: slot q = t*topk + j)
// ---------------------------------------------------------------------------

__device__ __forceinline__ MatView expert_view(const MoeShape &sh, const ExpertTable &tab, int e) {
  MatView v;
  v.base = tab.base[e];
  v.off_dtab = sh.off_dtab;
  v.off_rtab = sh.off_rtab;
  v.off_btab = sh.off_btab;
  v.off_perm = sh.off_perm;
  v.off_codes = sh.off_codes;
  v.n = sh.n;
  v.k = sh.k;
  v.bd = tab.bd[e];
  v.n_tiles = sh.n_tiles;
  v.units = sh.units;
  return v;
}

// Per-slot fused GEMV (one activation row per slot): block (row group, slot),
// matrix = the slot's expert.
__global__ __launch_bounds__(256) void moe_gemv_kernel(MoeShape sh, ExpertTable tab,
                                                       const int32_t *__restrict__ ids,
                                                       const uint16_t *__restrict__ x, int64_t ldx,
                                                       int x_per_slot, int topk,
                                                       void *__restrict__ y, int64_t ldy, int ydt,
                                                       int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int q = blockIdx.y;
  const MatView w = expert_view(sh, tab, ids[q]);
  const int src = x_per_slot ? q : q / topk;
  const int rt0 = blockIdx.x * R;
  const int Reff = min(R, w.n_tiles - rt0);
  char *yq = (char *)y + (size_t)q * ldy * (ydt == 0 ? 2 : 4);
  gemv_fused_block<1>(w, x + (int64_t)src * ldx, ldx, yq, ldy, ydt, rt0, Reff, smem);
}

// Routing for the grouped GEMM: counting sort of slots by expert and a list
// of work items (expert, first sorted row, end row), at most 16*BMT rows
// each.  Single block of 1024 threads.
//   ws_counts[E], ws_offsets[E+1], ws_sorted[S], ws_work[3*max_work], ws_nwork[1]
__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t *__restrict__ ids, int S,
                                                         int E, int rows_per_item,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ sorted,
                                                         int32_t *__restrict__ work,
                                                         int32_t *__restrict__ nwork) {
  __shared__ int32_t s_cnt[MAX_EXPERTS];
  __shared__ int32_t s_off[MAX_EXPERTS + 1];
  __shared__ int32_t s_fill[MAX_EXPERTS];
  __shared__ int32_t s_items[MAX_EXPERTS + 1];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int q = t; q < S; q += 1024) atomicAdd(&s_cnt[ids[q]], 1);
  __syncthreads();
  if (t == 0) {
    int off = 0, items = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = off;
      s_items[e] = items;
      off += s_cnt[e];
      items += (s_cnt[e] + rows_per_item - 1) / rows_per_item;
      s_fill[e] = 0;
    }
    s_off[E] = off;
    s_items[E] = items;
    *nwork = items;
  }
  __syncthreads();
  for (int e = t; e < E; e += 1024) counts[e] = s_cnt[e];
  for (int e = t; e <= E; e += 1024) offsets[e] = s_off[e];
  for (int q = t; q < S; q += 1024) {
    const int e = ids[q];
    const int pos = s_off[e] + atomicAdd(&s_fill[e], 1);
    sorted[pos] = q;
  }
  for (int e = t; e < E; e += 1024) {
    const int n_items = s_items[e + 1] - s_items[e];
    for (int c = 0; c < n_items; ++c) {
      const int wi = s_items[e] + c;
      const int r0 = s_off[e] + c * rows_per_item;
      work[3 * wi + 0] = e;
      work[3 * wi + 1] = r0;
      work[3 * wi + 2] = min(r0 + rows_per_item, s_off[e + 1]);
    }
  }
}

// bf16 grouped preparation: sorted row j holds slot sorted[j]'s activations
// permuted by its expert's permutation.
__global__ __launch_bounds__(256) void moe_prep_bf16_kernel(MoeShape sh, ExpertTable tab,
                                                             const uint16_t *__restrict__ x,
                                                             int64_t ldx, int x_per_slot, int topk,
                                                             const int32_t *__restrict__ ids,
                                                             const int32_t *__restrict__ sorted,
                                                             uint16_t *__restrict__ xb, int stage) {
  extern __shared__ uint16_t s_row[];
  const int j = blockIdx.x;
  const int q = sorted[j];
  const int e = ids[q];
  const int src = x_per_slot ? q : q / topk;
  const int Kp = sh.units * UNIT_SLOTS;
  prep_bf16_row((const uint16_t *)(tab.base[e] + sh.off_perm), sh.k, Kp, x + (int64_t)src * ldx,
                xb + (size_t)j * Kp, s_row, stage);
}

struct SortedRows {
  const int32_t *sorted;
  __device__ int operator()(int mm) const { return sorted[mm]; }
};

template <int BMT>
__global__ __launch_bounds__(256) void moe_gemm_bf16_kernel(MoeShape sh, ExpertTable tab,
                                                            const int32_t *__restrict__ work,
                                                            const int32_t *__restrict__ nwork,
                                                            const int32_t *__restrict__ sorted,
                                                            const uint16_t *__restrict__ xb,
                                                            void *__restrict__ y, int64_t ldy,
                                                            int ydt) {
  __shared__ u4 s_btab[1024];
  const int wi = blockIdx.y;
  if (wi >= *nwork) return;
  const int e = work[3 * wi + 0], r0 = work[3 * wi + 1], r1 = work[3 * wi + 2];
  const MatView w = expert_view(sh, tab, e);
  const u4 *btab_g = (const u4 *)(w.base + w.off_btab);
  for (int j = threadIdx.x; j < 1024; j += 256) s_btab[j] = btab_g[j];
  __syncthreads();
  const int rt = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rt >= w.n_tiles) return;
  gemm_bf16_tile<BMT>(w, rt, xb, r0, r1, y, ldy, ydt, s_btab, SortedRows{sorted});
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_prep_bf16(const MatView &w, const uint16_t *x, int64_t ldx, int m, int m_pad,
                            uint16_t *xb, hipStream_t s) {
  const int stage = w.k <= 32768 ? 1 : 0;
  const size_t lds = stage ? (size_t)w.k * 2 : 0;
  hipLaunchKernelGGL(prep_bf16_kernel, dim3(m_pad), dim3(256), lds, s, w, x, ldx, m, xb, stage);
  return hipGetLastError();
}

constexpr int GEMM_BMT = 4;  // 64 activation rows per block

hipError_t launch_gemm_bf16(const MatView &w, const uint16_t *xb, int m, int m_pad, void *y,
                            int64_t ldy, int ydt, hipStream_t s) {
  dim3 grid((w.n_tiles + 3) / 4, m_pad / (16 * GEMM_BMT)), block(256);
  hipLaunchKernelGGL(gemm_bf16_kernel<GEMM_BMT>, grid, block, 0, s, w, xb, m, y, ldy, ydt);
  return hipGetLastError();
}

int gemm_m_pad(int m) { return ((m + 16 * GEMM_BMT - 1) / (16 * GEMM_BMT)) * (16 * GEMM_BMT); }

// ---------------------------------------------------------------------------
// MoE launcher.  Workspace layout depends on the path:
//   exact (m*topk <= MOE_EXACT_MAX_SLOTS): xw[S][Kp] fp16, escale[S]
//   bf16: counts[E], offsets[E+1], sorted[S], work[3*max_work], nwork,
//         xb[S + 16*BMT][Kp] bf16
// ---------------------------------------------------------------------------
constexpr int MOE_EXACT_MAX_SLOTS = 64;

hipError_t launch_moe(const svq_handle *experts, int32_t E, const void *x, int64_t ldx,
                      int32_t x_per_slot, const int32_t *ids, int64_t m, int32_t topk, void *y,
                      int64_t ldy, int ydt, void *ws, size_t ws_bytes, hipStream_t s, size_t *need) {
  const int S = (int)(m * topk);
  const svq_handle &h0 = experts[0];
  MoeShape sh;
  sh.off_dtab = (uint32_t)h0.off_dtab;
  sh.off_rtab = (uint32_t)h0.off_rtab;
  sh.off_btab = (uint32_t)h0.off_btab;
  sh.off_perm = (uint32_t)h0.off_perm;
  sh.off_codes = h0.off_codes;
  sh.n = h0.n;
  sh.k = h0.k;
  sh.n_tiles = h0.n_tiles;
  sh.units = h0.units;
  sh.num_experts = E;
  const size_t Kp = (size_t)sh.units * UNIT_SLOTS;
  ExpertTable tab;
  for (int e = 0; e < MAX_EXPERTS; ++e) {
    tab.base[e] = e < E ? (const uint8_t *)experts[e].dev : nullptr;
    tab.bd[e] = e < E ? (uint8_t)experts[e].bd : 0;
  }
  const uint16_t *xp = (const uint16_t *)x;
  if (S <= MOE_EXACT_MAX_SLOTS) {
    *need = 256;
    if (!ws) return hipSuccess;
    const int R = 1;
    const size_t smem = gemv_smem_bytes(1, sh.k, sh.units);
    hipError_t e = allow_smem(moe_gemv_kernel, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_gemv_kernel, dim3((sh.n_tiles + R - 1) / R, S), dim3(256), smem, s, sh,
                       tab, ids, xp, ldx, x_per_slot, topk, y, ldy, ydt, R);
    return hipGetLastError();
  }
  const int rows_per_item = 16 * GEMM_BMT;
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
  const size_t o_xb = off;
  off += align256((size_t)(S + rows_per_item) * Kp * 2);
  *need = off;
  if (!ws) return hipSuccess;
  if (ws_bytes < *need) return hipErrorInvalidValue;
  uint8_t *b = (uint8_t *)ws;
  int32_t *counts = (int32_t *)(b + o_counts), *offsets = (int32_t *)(b + o_offsets);
  int32_t *sorted = (int32_t *)(b + o_sorted), *work = (int32_t *)(b + o_work);
  int32_t *nwork = (int32_t *)(b + o_nwork);
  uint16_t *xb = (uint16_t *)(b + o_xb);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(1024), 0, s, ids, S, E, rows_per_item, counts,
                     offsets, sorted, work, nwork);
  const int stage = sh.k <= 32768 ? 1 : 0;
  hipLaunchKernelGGL(moe_prep_bf16_kernel, dim3(S), dim3(256), stage ? (size_t)sh.k * 2 : 0, s, sh,
                     tab, xp, ldx, x_per_slot, topk, ids, (const int32_t *)sorted, xb, stage);
  hipLaunchKernelGGL(moe_gemm_bf16_kernel<GEMM_BMT>, dim3((sh.n_tiles + 3) / 4, max_work), dim3(256),
                     0, s, sh, tab, (const int32_t *)work, (const int32_t *)nwork,
                     (const int32_t *)sorted, (const uint16_t *)xb, y, ldy, ydt);
  return hipGetLastError();
}

}  // namespace svq
