// Calibration kernels of libsvq, for gfx950: the channel energies and the
// tiered permutation of Energy-Stratified Grouping (ESG), and the ordered
// error sums of Adaptive Bit Split (ABS).
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability", abstract and Fig. 2 caption: ESG groups, inside every
// 8-channel subvector, channels of different energy tiers measured on
// calibration activations; ABS keeps, per matrix, the direction/radius bit
// split with the lowest activation-weighted reconstruction error.  The
// readings (energy = mean square in token order, tiers of k/8 ranks, slot
// 8c + l <- rank l*k/8 + c, errors summed in code and row order) are stated
// in include/svq.h.
//
// The energies decide an integer result (the permutation), so their
// arithmetic is fixed: one float64 chain per channel in token order.  The
// chain, not the memory, bounds the energy kernel; a block stages a tile of
// 256 tokens x 32 channels in LDS (all 256 threads load, 16 bytes each)
// while 32 threads run the chains over the previous tile.  Ranks are counts
// of strictly larger energies (ties: lower index first), accumulated with
// integer atomics (order independent), so the permutation is exact.
#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

#pragma clang fp contract(off)

constexpr int ESG_CH = 32;       // channels per block
constexpr int ESG_TOK = 256;     // tokens per staged tile
constexpr int ESG_SPAN = 1024;   // energies compared per rank block

__global__ __launch_bounds__(256) void esg_energy_kernel(EsgArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[ESG_TOK][ESG_CH];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * ESG_CH;
  const int g = tid & 3, tr = tid >> 2;  // 8-channel group, token row 0..63
  const bool gok = c0 + 8 * g < a.k;     // k % 8 == 0: a group is all in or all out
  const int64_t T = a.t;
  u4 nx[4];
  auto load = [&](int64_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = t0 + tr + 64 * q;
      u4 v = {0u, 0u, 0u, 0u};
      if (gok && t < T) v = *(const u4 *)(a.x + t * a.ldx + c0 + 8 * g);
      nx[q] = v;
    }
  };
  load(0);
  double acc = 0.0;
  for (int64_t t0 = 0; t0 < T; t0 += ESG_TOK) {
    __syncthreads();  // the chains over the previous tile are done
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u4 *)&tile[tr + 64 * q][8 * g] = nx[q];
    __syncthreads();
    if (t0 + ESG_TOK < T) load(t0 + ESG_TOK);
    if (tid < ESG_CH) {
      const int nt = (int)min((int64_t)ESG_TOK, T - t0);
      for (int i = 0; i < nt; ++i) {
        const double v = (double)bf16_bits_to_f32(tile[i][tid]);
        acc = acc + v * v;
      }
    }
  }
  if (tid < ESG_CH && c0 + tid < a.k) {
    a.energy[c0 + tid] = acc / (double)T;
    a.rank[c0 + tid] = 0;
  }
}

// rank[j] += #{i in this block's span: e_i > e_j, or e_i == e_j and i < j}
__global__ __launch_bounds__(256) void esg_count_kernel(EsgArgs a) {
  __shared__ double s_e[ESG_SPAN];
  const int i0 = blockIdx.y * ESG_SPAN;
  for (int e = threadIdx.x; e < ESG_SPAN; e += 256) s_e[e] = i0 + e < a.k ? a.energy[i0 + e] : 0.0;
  __syncthreads();
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  if (j >= a.k) return;
  const double ej = a.energy[j];
  const int lo = (threadIdx.x >> 6) * (ESG_SPAN / 4);
  const int hi = min(lo + ESG_SPAN / 4, a.k - i0);
  int cnt = 0;
  for (int e = lo; e < hi; ++e) {
    const double ei = s_e[e];
    cnt += (ei > ej || (ei == ej && i0 + e < j)) ? 1 : 0;
  }
  if (cnt) atomicAdd(a.rank + j, cnt);
}

// slot 8 (r % C) + r / C <- channel of rank r (r < k, so the slot is too)
__global__ __launch_bounds__(256) void esg_scatter_kernel(EsgArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.k) return;
  const int C = a.k / 8, r = a.rank[j];
  a.perm[8 * (r % C) + r / C] = j;
}

hipError_t launch_esg(const EsgArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(esg_energy_kernel, dim3((unsigned)((a.k + ESG_CH - 1) / ESG_CH)), dim3(256), 0,
                     s, a);
  hipLaunchKernelGGL(esg_count_kernel,
                     dim3((unsigned)((a.k + 63) / 64), (unsigned)((a.k + ESG_SPAN - 1) / ESG_SPAN)),
                     dim3(256), 0, s, a);
  hipLaunchKernelGGL(esg_scatter_kernel, dim3((unsigned)((a.k + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// rows[i] = err[i][0] + err[i][1] + ... (code order)
__global__ __launch_bounds__(256) void abs_rows_kernel(const double *err, int32_t n, int32_t C,
                                                       double *rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const double *e = err + (int64_t)i * C;
  double r = e[0];
  for (int c = 1; c < C; ++c) r = r + e[c];
  rows[i] = r;
}

// totals[c] = 0 + rows[c][0] + rows[c][1] + ... (row order), one block per
// candidate; the rows are staged in LDS and summed by one thread
constexpr int ABS_STAGE = 4096;
__global__ __launch_bounds__(256) void abs_totals_kernel(const double *rows, int32_t n,
                                                         double *totals) {
  __shared__ double s_r[ABS_STAGE];
  const double *r = rows + (int64_t)blockIdx.x * n;
  double tot = 0.0;
  for (int i0 = 0; i0 < n; i0 += ABS_STAGE) {
    const int cnt = min(ABS_STAGE, n - i0);
    __syncthreads();
    for (int e = threadIdx.x; e < cnt; e += 256) s_r[e] = r[i0 + e];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int e = 0; e < cnt; ++e) tot = tot + s_r[e];
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = tot;
}

hipError_t launch_abs_rows(const double *err, int32_t n, int32_t C, double *rows, hipStream_t s) {
  hipLaunchKernelGGL(abs_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, err, n, C,
                     rows);
  return hipGetLastError();
}

hipError_t launch_abs_totals(const double *rows, int32_t n, int32_t n_cand, double *totals,
                             hipStream_t s) {
  hipLaunchKernelGGL(abs_totals_kernel, dim3((unsigned)n_cand), dim3(256), 0, s, rows, n, totals);
  return hipGetLastError();
}

}  // namespace svq
