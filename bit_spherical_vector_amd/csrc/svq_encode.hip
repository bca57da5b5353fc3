// Encoder of libsvq: float weights -> the canonical 18-bit code stream, for
// gfx950.
//
// Method: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World
// Usability", Fig. 2 caption: spherical vector quantization codes each
// 8-weight subvector (taken along the channel permutation) by its signs, a
// direction index into a codebook of unit directions and a quantized
// radius.  The coding rule (largest inner product of |v| with a direction,
// nearest radius to the norm, first index on ties) and its arithmetic are
// stated in include/svq.h (svq_encode); the activation-weighted fit (the
// pair of direction and radius with the smallest weighted squared error,
// SAGE Abstract and Fig. 2 caption) in include/svq.h (svq_encode_weighted).
//
// Every choice is an integer decided by floating-point comparisons, so the
// arithmetic is fixed to the last bit: float64 products (exact: float32 x
// fp16 and float32 x float32 squares both fit the 53-bit significand), sums
// taken lane by lane in order 0..7, no fused multiply-adds.  That rules out
// the matrix cores here (their accumulation order is not specified); the
// scores run on the double-precision VALU, one thread per group of four
// codes, the codebook broadcast from LDS (every lane of a wave reads the
// same row).  Per code: 2^bd x 15 double operations (bd = 8: 3840); the
// weighted fit 2^bd x (31 + 5 x 2^br) (bd = 8: 13 000).
#include "svq_device.h"
#include "../../include/svq.h"

namespace svq {

#pragma clang fp contract(off)

constexpr int ENC_CODES = 4;  // codes per thread: 4 x 18 bits = 9 whole bytes

// FIT: activation-weighted fit (a.fit_h non-null); the plain rule otherwise.
// Two instantiations, so that the plain rule keeps its own register budget.
template <bool FIT>
__global__ __launch_bounds__(256) void svq_encode_kernel(EncArgs a) {
  extern __shared__ __attribute__((aligned(16))) double s_tab[];  // codebook rows x 8, midpoints
  const int rows = 1 << a.bd;
  for (int e = threadIdx.x; e < rows * 8; e += 256) s_tab[e] = a.cb[e];
  double *s_msq = s_tab + rows * 8;
  for (int e = threadIdx.x; e < a.n_mid; e += 256) s_msq[e] = a.msq[e];
  double *s_rad = s_msq + a.n_mid;  // radius values: the error, and the weighted fit
  if (a.err || FIT)
    for (int e = threadIdx.x; e <= a.n_mid; e += 256) s_rad[e] = a.rad[e];
  __syncthreads();

  const int64_t grp = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t c0 = grp * ENC_CODES;
  if (c0 >= a.count) return;
  const int C = a.k / 8;
  double av[ENC_CODES][8], nsq[ENC_CODES];
  uint32_t sg[ENC_CODES];
#pragma unroll
  for (int q = 0; q < ENC_CODES; ++q) {
    const int64_t cq = min(c0 + q, a.count - 1);  // the last group may be partial
    const int64_t i = cq / C;
    const int c = (int)(cq - i * C);
    const float *row = a.w + i * a.ldw;
    const int4 p0 = *(const int4 *)(a.perm + 8 * c), p1 = *(const int4 *)(a.perm + 8 * c + 4);
    const int ch[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    uint32_t s = 0;
    double n2 = 0.0;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const float v = row[ch[l]];
      s |= (__builtin_bit_cast(uint32_t, v) >> 31) << l;
      av[q][l] = fabs((double)v);
      const double sq = av[q][l] * av[q][l];
      n2 = l == 0 ? sq : n2 + sq;
    }
    sg[q] = s;
    nsq[q] = n2;
  }

  // direction (and, for the weighted fit, radius) of every code
  double best[ENC_CODES];
  int bi[ENC_CODES];
  uint32_t rw[ENC_CODES];
#pragma unroll
  for (int q = 0; q < ENC_CODES; ++q) {
    bi[q] = 0;
    rw[q] = 0;
  }
  if constexpr (FIT) {
    // Weighted fit: the (d, r) pair with the smallest reduced error
    // (R R) B_d - (R + R) A_d, A_d = sum_l (h_l |v_l|) D_dl,
    // B_d = sum_l (h_l D_dl) D_dl, lanes in order, pairs in (d, r) order,
    // the first minimum kept.  One code at a time.
    const int nR = a.n_mid + 1;
#pragma unroll
    for (int q = 0; q < ENC_CODES; ++q) {
      const int64_t cq = min(c0 + q, a.count - 1);
      const int c = (int)(cq % C);
      double hl[8], hw[8];
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        hl[l] = a.fit_h[a.perm[8 * c + l]];
        hw[l] = hl[l] * av[q][l];
      }
      double eb = 0.0;
      int db = 0;
      uint32_t rb = 0;
      for (int j = 0; j < rows; ++j) {
        const double *D = s_tab + j * 8;
        double A = hw[0] * D[0];
        double B = (hl[0] * D[0]) * D[0];
#pragma unroll
        for (int l = 1; l < 8; ++l) {
          A = A + hw[l] * D[l];
          B = B + (hl[l] * D[l]) * D[l];
        }
        for (int t = 0; t < nR; ++t) {
          const double R = s_rad[t];
          const double E = (R * R) * B - (R + R) * A;
          if ((j == 0 && t == 0) || E < eb) {
            eb = E;
            db = j;
            rb = (uint32_t)t;
          }
        }
      }
      bi[q] = db;
      rw[q] = rb;
    }
  } else {
  for (int j = 0; j < rows; ++j) {
    double D[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) D[l] = s_tab[j * 8 + l];
#pragma unroll
    for (int q = 0; q < ENC_CODES; ++q) {
      double sc = av[q][0] * D[0];
#pragma unroll
      for (int l = 1; l < 8; ++l) sc = sc + av[q][l] * D[l];
      if (j == 0 || sc > best[q]) {
        best[q] = sc;
        bi[q] = j;
      }
    }
  }
  }

  // radius: number of squared midpoints strictly below the squared norm.
  // A partial last group packs only its own codes (the stream's trailing
  // bits stay zero) and writes only the bytes they reach.
  const int nq = (int)min((int64_t)ENC_CODES, a.count - c0);
  uint64_t lo = 0;
  uint32_t hi = 0;
#pragma unroll
  for (int q = 0; q < ENC_CODES; ++q) {
    uint32_t r = rw[q];
    if constexpr (!FIT)
      for (int t = 0; t < a.n_mid; ++t) r += nsq[q] > s_msq[t] ? 1u : 0u;
    const uint64_t code = q < nq ? (uint64_t)(sg[q] | ((uint32_t)bi[q] << 8) | (r << (8 + a.bd))) : 0;
    if (a.err && q < nq) {
      // (v[l] - w_hat[l])^2 * h[channel], lanes in order; w_hat = +-R[r] D[d][l]
      // is exact in double, v[l] = +-|v[l]| from the sign bit
      const int64_t cq = c0 + q;
      const int c = (int)(cq % C);
      const double R = s_rad[r];
      double e = 0.0;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        const bool neg = (sg[q] >> l) & 1u;
        const double wh = R * s_tab[bi[q] * 8 + l];
        const double d = neg ? wh - av[q][l] : av[q][l] - wh;  // v - w_hat, sign folded
        const double t = (d * d) * a.h[a.perm[8 * c + l]];
        e = l == 0 ? t : e + t;
      }
      a.err[cq] = e;
    }
    lo |= code << (18 * q);                   // code 3 keeps its low 10 bits here
    if (q == 3) hi = (uint32_t)(code >> 10);  // and its high 8 bits here
  }
  const int nbytes = (18 * nq + 7) / 8;
  uint8_t *out = a.codes + 9 * grp;
#pragma unroll
  for (int b = 0; b < 9; ++b)
    if (b < nbytes) out[b] = b < 8 ? (uint8_t)(lo >> (8 * b)) : (uint8_t)hi;
}

hipError_t launch_encode(const EncArgs &a, hipStream_t s) {
  const int64_t groups = (a.count + ENC_CODES - 1) / ENC_CODES;
  const size_t lds = ((size_t)(8 << a.bd) + 2 * (size_t)a.n_mid + 1) * sizeof(double);
  if (a.fit_h)
    hipLaunchKernelGGL(svq_encode_kernel<true>, dim3((unsigned)((groups + 255) / 256)), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(svq_encode_kernel<false>, dim3((unsigned)((groups + 255) / 256)), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace svq
