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
// chain, not the memory, bounds the energy kernel; all 256 threads of a
// block load a tile of 256 tokens x 32 channels (16 bytes at a time, the
// next tile in flight) and store its squares in LDS as doubles, and 32
// threads run the chains of additions over them.  Ranks are counts
// of strictly larger energies (ties: lower index first), accumulated with
// integer atomics (order independent), so the permutation is exact.  The
// error sums of ABS are chains too (lanes, codes of a row, rows), each
// staged through LDS so that only the additions wait on one another.
#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

#pragma clang fp contract(off)

constexpr int ESG_CH = 32;       // channels per block
constexpr int ESG_TOK = 256;     // tokens per staged tile (64 KB of squares)
constexpr int ESG_LD = ESG_TOK / 64;  // 16-byte loads per thread and tile
constexpr int ESG_SPAN = 256;    // energies compared per rank block

__global__ __launch_bounds__(256) void esg_energy_kernel(EsgArgs a) {
  __shared__ __attribute__((aligned(16))) double sq[ESG_TOK][ESG_CH];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * ESG_CH;
  const int g = tid & 3, tr = tid >> 2;  // 8-channel group, token row 0..63
  const bool gok = c0 + 8 * g < a.k;     // k % 8 == 0: a group is all in or all out
  const int64_t T = a.t;
  u4 nx[ESG_LD];
  auto load = [&](int64_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < ESG_LD; ++q) {
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
    // every thread squares its 8 x ESG_LD values (exact in double)
#pragma unroll
    for (int q = 0; q < ESG_LD; ++q) {
      double *dst = &sq[tr + 64 * q][8 * g];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const double lo = (double)bf16_bits_to_f32(nx[q][h] & 0xFFFFu);
        const double hi = (double)bf16_bits_to_f32(nx[q][h] >> 16);
        dst[2 * h] = lo * lo;
        dst[2 * h + 1] = hi * hi;
      }
    }
    __syncthreads();
    if (t0 + ESG_TOK < T) load(t0 + ESG_TOK);
    if (tid < ESG_CH) {
      const int nt = (int)min((int64_t)ESG_TOK, T - t0);
      int i = 0;
      // eight reads ahead of the additions, which alone form the chain
      for (; i + 8 <= nt; i += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = sq[i + u][tid];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = acc + v[u];
      }
      for (; i < nt; ++i) acc = acc + sq[i][tid];
    }
  }
  if (tid < ESG_CH && c0 + tid < a.k) {
    a.energy[c0 + tid] = acc / (double)T;
    a.rank[c0 + tid] = 0;
  }
}

// rank[j] += #{i in this block's span: e_i > e_j, or e_i == e_j and i < j}.
// Energies are sums of squares divided by t: non-negative, so (for finite
// values) their bit patterns order like the values and the tie rule becomes
// one integer comparison of (bits, -index) keys.
__global__ __launch_bounds__(256) void esg_count_kernel(EsgArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t s_e[ESG_SPAN];
  const int i0 = blockIdx.y * ESG_SPAN;
  const uint64_t *bits = (const uint64_t *)a.energy;
  // entries past the end are never read (hi stops at k - i0)
  for (int e = threadIdx.x; e < ESG_SPAN; e += 256) s_e[e] = i0 + e < a.k ? bits[i0 + e] : 0;
  __syncthreads();
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  if (j >= a.k) return;
  const uint64_t ej = bits[j];
  const int lo = (threadIdx.x >> 6) * (ESG_SPAN / 4);
  const int hi = min(lo + ESG_SPAN / 4, a.k - i0);
  int cnt = 0;
  int e = lo;
  for (; e + 8 <= hi; e += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t ei = s_e[e + u];
      cnt += (ei > ej || (ei == ej && i0 + e + u < j)) ? 1 : 0;
    }
  }
  for (; e < hi; ++e) {
    const uint64_t ei = s_e[e];
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

// rows[i] = err[i][0] + err[i][1] + ... (code order).  A block takes 32
// rows; their errors pass through LDS 64 codes at a time (all 256 threads
// load, the next chunk in flight while the current one is summed), and one
// thread per row runs the chain.
constexpr int ABS_ROWS = 32, ABS_CODES = 64, ABS_LD = ABS_ROWS * ABS_CODES / 256;
__global__ __launch_bounds__(256) void abs_rows_kernel(const double *err, int32_t n, int32_t C,
                                                       double *rows) {
  __shared__ double s_e[ABS_ROWS][ABS_CODES + 1];
  const int r0 = blockIdx.x * ABS_ROWS;
  const int i = r0 + (int)threadIdx.x;
  double nx[ABS_LD];
  auto load = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < ABS_LD; ++q) {
      const int e = (int)threadIdx.x + 256 * q, rr = e / ABS_CODES, cc = e % ABS_CODES;
      nx[q] = (r0 + rr < n && c0 + cc < C) ? err[(int64_t)(r0 + rr) * C + c0 + cc] : 0.0;
    }
  };
  load(0);
  double r = 0.0;
  for (int c0 = 0; c0 < C; c0 += ABS_CODES) {
    const int nc = min(ABS_CODES, C - c0);
    __syncthreads();  // the chains over the previous chunk are done
#pragma unroll
    for (int q = 0; q < ABS_LD; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      s_e[e / ABS_CODES][e % ABS_CODES] = nx[q];
    }
    __syncthreads();
    if (c0 + ABS_CODES < C) load(c0 + ABS_CODES);
    if (threadIdx.x < ABS_ROWS && i < n) {
      int c = 0;
      if (c0 == 0) {
        r = s_e[threadIdx.x][0];
        c = 1;
      }
      for (; c < nc; ++c) r = r + s_e[threadIdx.x][c];
    }
  }
  if (threadIdx.x < ABS_ROWS && i < n) rows[i] = r;
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
    if (threadIdx.x == 0) {
      int e = 0;
      for (; e + 8 <= cnt; e += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s_r[e + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) tot = tot + v[u];
      }
      for (; e < cnt; ++e) tot = tot + s_r[e];
    }
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = tot;
}

hipError_t launch_abs_rows(const double *err, int32_t n, int32_t C, double *rows, hipStream_t s) {
  hipLaunchKernelGGL(abs_rows_kernel, dim3((unsigned)((n + ABS_ROWS - 1) / ABS_ROWS)), dim3(256), 0, s,
                     err, n, C, rows);
  return hipGetLastError();
}

hipError_t launch_abs_totals(const double *rows, int32_t n, int32_t n_cand, double *totals,
                             hipStream_t s) {
  hipLaunchKernelGGL(abs_totals_kernel, dim3((unsigned)n_cand), dim3(256), 0, s, rows, n, totals);
  return hipGetLastError();
}

}  // namespace svq
