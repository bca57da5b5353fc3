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
// Exact path
// ---------------------------------------------------------------------------

// Block-level: permute one activation row (gather, Fig. 6 "reordered
// activations"), scale it by 2^e with e chosen so that max|x| * 2^e lies in
// [2^14, 2^15) (exact for every bf16 value above 2^-17 * max), convert to
// fp16.  Slots >= k are zero.  blockDim.x == 256.
__device__ void prep_exact_row(const uint16_t *__restrict__ perm, int K, int Kp,
                               const uint16_t *__restrict__ xr, uint16_t *__restrict__ xo,
                               int32_t *__restrict__ esc, float *red4) {
  float mx = 0.f;
  for (int j = threadIdx.x; j < K; j += 256) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(xr[j])));
  for (int off = 32; off; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
  const int e = mx > 0.f ? 14 - ilogbf(mx) : 0;
  for (int p = threadIdx.x; p < Kp; p += 256) {
    float v = p < K ? bf16_bits_to_f32(xr[perm[p]]) : 0.f;
    _Float16 h = (_Float16)ldexpf(v, e);
    xo[p] = __builtin_bit_cast(uint16_t, h);
  }
  if (threadIdx.x == 0) *esc = e;
}

__global__ __launch_bounds__(256) void prep_exact_kernel(MatView w, const uint16_t *__restrict__ x,
                                                          int64_t ldx, uint16_t *__restrict__ xw,
                                                          int32_t *__restrict__ escale) {
  __shared__ float red4[4];
  const int a = blockIdx.x;
  const int Kp = w.units * UNIT_SLOTS;
  prep_exact_row((const uint16_t *)(w.base + w.off_perm), w.k, Kp, x + (int64_t)a * ldx,
                 xw + (size_t)a * Kp, escale + a, red4);
}

// GEMV of one 16-row tile for m <= 4 activation rows.  The block's W waves
// take the tile's coded units round-robin and meet in LDS at the end.
//
// MFMA mapping for K-block i of unit u (4 codes, 32 permuted slots):
//   B[k][n]: lane L holds the signed direction row of its code (row n =
//            L & 15, code group q = L >> 4), k = 8q..8q+7.
//   A[m][k]: m = 4q' + a selects code group q' and activation row a; lane L
//            holds A[L & 15][k-group L >> 4], non-zero only when
//            (L & 15) >> 2 == L >> 4 ("diagonal" lanes), where it is the
//            8 scaled activations of code (4i + q) for row a = L & 3.
//   C[m][n]: lane L receives rows 4q + a (a = 0..3) of column L & 15, i.e.
//            exactly the dot products of the code it decoded, one per
//            activation row.
// xw rows are Kp = units*512 fp16 apart; output row a goes to y + a*ldy.
template <int M>
__device__ void gemv_exact_tile(const MatView &w, int rt, const uint16_t *__restrict__ xw,
                                const int32_t *__restrict__ escale, void *__restrict__ y,
                                int64_t ldy, int ydt, u4 *s_dtab, _Float16 *s_rtab,
                                float (*s_red)[EXACT_MAX_M][16]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, W = blockDim.x >> 6;
  const u4 *dtab_g = (const u4 *)(w.base + w.off_dtab);
  for (int j = tid; j < 256; j += blockDim.x) s_dtab[j] = dtab_g[j];
  if (tid < 16) s_rtab[tid] = ((const _Float16 *)(w.base + w.off_rtab))[tid];
  __syncthreads();

  const int q = lane >> 4;
  const int a_lane = lane & 3;
  const bool diag = (((lane & 15) >> 2) == q) && (a_lane < M);
  const int Kp = w.units * UNIT_SLOTS;
  const u4 *xa = (const u4 *)(xw + (size_t)(diag ? a_lane : 0) * Kp) + q;
  const int bd = w.bd;
  const uint8_t *tile = w.base + w.off_codes + (size_t)rt * w.units * UNIT_BYTES;

  float acc[M];
#pragma unroll
  for (int a = 0; a < M; ++a) acc[a] = 0.f;
  u4 A[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) A[i] = (u4){0u, 0u, 0u, 0u};

  for (int u = wv; u < w.units; u += W) {
    const uint8_t *ub = tile + (size_t)u * UNIT_BYTES;
    const u4 S = *(const u4 *)(ub + PLANE_SIGN + 16 * lane);
    const u4 L = *(const u4 *)(ub + PLANE_LOW + 16 * lane);
    const uint32_t H = *(const uint32_t *)(ub + PLANE_HIGH + 4 * lane);
    if (diag) {
#pragma unroll
      for (int i = 0; i < 16; ++i) A[i] = xa[64 * u + 4 * i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t idx = code_index(L, H, i);
      const u4 D = apply_signs(s_dtab[idx & 0xFFu], S, i);
      const f4 C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, A[i]),
                                                          __builtin_bit_cast(h8, D),
                                                          (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float R = (float)s_rtab[idx >> bd];
#pragma unroll
      for (int a = 0; a < M; ++a) acc[a] = __builtin_fmaf(R, C[a], acc[a]);
    }
  }
#pragma unroll
  for (int a = 0; a < M; ++a) {
    acc[a] += __shfl_xor(acc[a], 16);
    acc[a] += __shfl_xor(acc[a], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int a = 0; a < M; ++a) s_red[wv][a][lane] = acc[a];
  }
  __syncthreads();
  if (tid < 16 * M) {
    const int a = tid >> 4, r = tid & 15;
    float s = 0.f;
    for (int j = 0; j < W; ++j) s += s_red[j][a][r];
    s = ldexpf(s, -escale[a]);
    const int n = rt * 16 + r;
    if (n < w.n) store_out(y, (size_t)a * ldy + n, s, ydt);
  }
}

template <int M>
__global__ __launch_bounds__(512) void gemv_exact_kernel(MatView w, const uint16_t *__restrict__ xw,
                                                         const int32_t *__restrict__ escale,
                                                         void *__restrict__ y, int64_t ldy, int ydt) {
  __shared__ u4 s_dtab[256];
  __shared__ _Float16 s_rtab[16];
  __shared__ float s_red[8][EXACT_MAX_M][16];
  gemv_exact_tile<M>(w, blockIdx.x, xw, escale, y, ldy, ydt, s_dtab, s_rtab, s_red);
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

// Exact per-slot preparation: slot q's activation row permuted by its
// expert's permutation.
__global__ __launch_bounds__(256) void moe_prep_exact_kernel(MoeShape sh, ExpertTable tab,
                                                              const uint16_t *__restrict__ x,
                                                              int64_t ldx, int x_per_slot, int topk,
                                                              const int32_t *__restrict__ ids,
                                                              uint16_t *__restrict__ xw,
                                                              int32_t *__restrict__ escale) {
  __shared__ float red4[4];
  const int q = blockIdx.x;
  const int e = ids[q];
  const int src = x_per_slot ? q : q / topk;
  const int Kp = sh.units * UNIT_SLOTS;
  prep_exact_row((const uint16_t *)(tab.base[e] + sh.off_perm), sh.k, Kp, x + (int64_t)src * ldx,
                 xw + (size_t)q * Kp, escale + q, red4);
}

// Exact per-slot GEMV: block (row tile, slot).
__global__ __launch_bounds__(512) void moe_gemv_exact_kernel(MoeShape sh, ExpertTable tab,
                                                             const int32_t *__restrict__ ids,
                                                             const uint16_t *__restrict__ xw,
                                                             const int32_t *__restrict__ escale,
                                                             void *__restrict__ y, int64_t ldy,
                                                             int ydt) {
  __shared__ u4 s_dtab[256];
  __shared__ _Float16 s_rtab[16];
  __shared__ float s_red[8][EXACT_MAX_M][16];
  const int q = blockIdx.y;
  const MatView w = expert_view(sh, tab, ids[q]);
  const int Kp = sh.units * UNIT_SLOTS;
  char *yq = (char *)y + (size_t)q * ldy * (ydt == 0 ? 2 : 4);
  gemv_exact_tile<1>(w, blockIdx.x, xw + (size_t)q * Kp, escale + q, yq, ldy, ydt, s_dtab, s_rtab,
                     s_red);
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

hipError_t launch_prep_exact(const MatView &w, const uint16_t *x, int64_t ldx, int m, uint16_t *xw,
                             int32_t *escale, hipStream_t s) {
  hipLaunchKernelGGL(prep_exact_kernel, dim3(m), dim3(256), 0, s, w, x, ldx, xw, escale);
  return hipGetLastError();
}

hipError_t launch_gemv_exact(const MatView &w, const uint16_t *xw, const int32_t *escale, int m,
                             void *y, int64_t ldy, int ydt, hipStream_t s) {
  const int waves = w.units < 8 ? w.units : 8;
  dim3 grid(w.n_tiles), block(64 * waves);
  switch (m) {
    case 1: hipLaunchKernelGGL(gemv_exact_kernel<1>, grid, block, 0, s, w, xw, escale, y, ldy, ydt); break;
    case 2: hipLaunchKernelGGL(gemv_exact_kernel<2>, grid, block, 0, s, w, xw, escale, y, ldy, ydt); break;
    case 3: hipLaunchKernelGGL(gemv_exact_kernel<3>, grid, block, 0, s, w, xw, escale, y, ldy, ydt); break;
    default: hipLaunchKernelGGL(gemv_exact_kernel<4>, grid, block, 0, s, w, xw, escale, y, ldy, ydt); break;
  }
  return hipGetLastError();
}

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
    const size_t o_esc = align256((size_t)S * Kp * 2);
    *need = o_esc + align256((size_t)S * 4);
    if (!ws) return hipSuccess;
    if (ws_bytes < *need) return hipErrorInvalidValue;
    uint16_t *xw = (uint16_t *)ws;
    int32_t *esc = (int32_t *)((uint8_t *)ws + o_esc);
    hipLaunchKernelGGL(moe_prep_exact_kernel, dim3(S), dim3(256), 0, s, sh, tab, xp, ldx,
                       x_per_slot, topk, ids, xw, esc);
    const int waves = sh.units < 8 ? sh.units : 8;
    hipLaunchKernelGGL(moe_gemv_exact_kernel, dim3(sh.n_tiles, S), dim3(64 * waves), 0, s, sh, tab,
                       ids, (const uint16_t *)xw, (const int32_t *)esc, y, ldy, ydt);
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
