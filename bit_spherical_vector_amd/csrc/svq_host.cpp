// Host side of libsvq: argument validation, the one-time repack of a
// canonical SVQ matrix into coded units (svq_internal.h), and dispatch of the
// decode-and-multiply kernels.  Method: "SAGE: Pushing 2-Bit Vector-Quantized
// LLMs toward Real-World Usability", Fig. 2 caption (what a code holds) and
// Fig. 6 caption (subvectors multiply reordered activations).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/svq.h"
#include "svq_internal.h"

namespace svq {
hipError_t launch_moe(const svq_handle *const *experts, int32_t count, int32_t num_experts,
                      const void *const *x, const int64_t *ldx, int32_t x_per_slot,
                      const int32_t *expert_ids, int64_t m, int32_t topk, void *const *y,
                      const int64_t *ldy, int ydt, void *ws, size_t ws_bytes, hipStream_t s,
                      size_t *need);
}

using namespace svq;

static_assert(SCRATCH_BYTES == SVQ_SCRATCH_BYTES, "scratch size of svq.h and the library differ");

namespace {

constexpr uint32_t FIELD_MASK = (1u << 18) - 1;

// IEEE binary16 -> float (exact).
float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const uint32_t exp = (h >> 10) & 0x1F, frac = h & 0x3FF;
  uint32_t u;
  if (exp == 0) {
    if (frac == 0) {
      u = sign;
    } else {  // subnormal: frac * 2^-24, normalise
      int e = -1;
      uint32_t f = frac;
      do {
        f <<= 1;
        ++e;
      } while ((f & 0x400) == 0);
      u = sign | ((uint32_t)(127 - 15 - e) << 23) | ((f & 0x3FF) << 13);
    }
  } else if (exp == 0x1F) {
    u = sign | 0x7F800000u | (frac << 13);
  } else {
    u = sign | ((exp + 112) << 23) | (frac << 13);
  }
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// double -> IEEE binary16 bits, round to nearest even; |v| below 65520.
uint16_t double_to_half(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e = 0;
  std::frexp(a, &e);                  // a = f * 2^e, f in [0.5, 1)
  const int qexp = e - 11 < -24 ? -24 : e - 11;  // quantum: 11 significant bits, or subnormal
  const double r = std::nearbyint(std::ldexp(a, -qexp)) * std::ldexp(1.0, qexp);  // ties to even
  if (r < std::ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)std::ldexp(r, 24));
  int re = 0;
  const double rf = std::frexp(r, &re);  // r = rf * 2^re, rf in [0.5, 1)
  const uint32_t mant = (uint32_t)std::ldexp(rf, 11) - 1024;
  return (uint16_t)(sign | (uint16_t)((re - 1 + 15) << 10) | (uint16_t)mant);
}

// The exact split of a matrix's weights for the small-batch path: for the
// 1024 index values (direction d, radius r) and lanes l, v = R[r]*D[d][l]
// times 2^s is the sum of two fp16 values hi = RNE_fp16(v) and lo = v - hi.
// s puts the largest |v| in [2^14, 2^15); the split exists when every lo is
// itself an fp16 value (the low bits of v stay above the fp16 quantum).
// Fills xtab (row idx: hi[8] then lo[8]) and returns s, or
// SVQ_NO_EXACT_SPLIT.
int32_t exact_split(const svq_matrix_desc *d, uint16_t *xtab) {
  const uint32_t dmask = (1u << d->bd) - 1;
  double vmax = 0.0;
  for (int idx = 0; idx < 1024; ++idx)
    for (int l = 0; l < 8; ++l) {
      const double v = (double)half_to_float(d->radius_table[idx >> d->bd]) *
                       (double)half_to_float(d->dir_codebook[(idx & dmask) * 8 + l]);
      vmax = std::fabs(v) > vmax ? std::fabs(v) : vmax;
    }
  if (!(vmax > 0.0) || !std::isfinite(vmax)) return SVQ_NO_EXACT_SPLIT;
  int e = 0;
  std::frexp(vmax, &e);  // vmax in [2^(e-1), 2^e)
  const int32_t sexp = 15 - e;
  for (int idx = 0; idx < 1024; ++idx)
    for (int l = 0; l < 8; ++l) {
      const double v = std::ldexp((double)half_to_float(d->radius_table[idx >> d->bd]) *
                                      (double)half_to_float(d->dir_codebook[(idx & dmask) * 8 + l]),
                                  sexp);
      const uint16_t hi = double_to_half(v);
      const double lo = v - (double)half_to_float(hi);  // exact: both share v's quantum
      const uint16_t lob = double_to_half(lo);
      if ((double)half_to_float(lob) != lo) return SVQ_NO_EXACT_SPLIT;
      xtab[idx * 16 + l] = hi;
      xtab[idx * 16 + 8 + l] = lob;
    }
  return sexp;
}

// float -> bfloat16 bits, round to nearest even.
uint16_t float_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Layout {
  int32_t n_tiles, units;
  size_t off_dtab, off_rtab, off_btab, off_xtab, off_perm, off_codes, padded_code_bytes, bytes;
};

Layout make_layout(int32_t n, int32_t k) {
  Layout L;
  L.n_tiles = (n + UNIT_ROWS - 1) / UNIT_ROWS;
  L.units = (k + UNIT_SLOTS - 1) / UNIT_SLOTS;
  size_t off = 0;
  L.off_dtab = off;
  off += align256(DTAB_BYTES);
  L.off_rtab = off;
  off += align256(RTAB_BYTES);
  L.off_btab = off;
  off += align256(BTAB_BYTES);
  L.off_xtab = off;
  off += align256(XTAB_BYTES);
  L.off_perm = off;
  off += align256((size_t)L.units * UNIT_SLOTS * 2);  // zero padded to the unit width
  L.off_codes = off;
  L.padded_code_bytes = (size_t)L.n_tiles * L.units * UNIT_BYTES;
  off += align256(L.padded_code_bytes);
  L.bytes = off;
  return L;
}

svq_status validate_desc(const svq_matrix_desc *d) {
  if (!d) return SVQ_ERR_INVALID_ARG;
  if (d->n <= 0 || d->k <= 0 || d->k % 8 != 0) return SVQ_ERR_INVALID_ARG;
  if (d->bd + d->br != 10) return SVQ_ERR_INVALID_ARG;
  if (d->bd < 6 || d->bd > 8) return SVQ_ERR_UNSUPPORTED;
  if (d->k > SVQ_MAX_K || d->n > SVQ_MAX_N) return SVQ_ERR_UNSUPPORTED;
  if (!d->codes || !d->dir_codebook || !d->radius_table || !d->perm) return SVQ_ERR_INVALID_ARG;
  std::vector<uint8_t> seen((size_t)d->k, 0);
  for (int32_t p = 0; p < d->k; ++p) {
    const int32_t c = d->perm[p];
    if (c < 0 || c >= d->k || seen[(size_t)c]) return SVQ_ERR_INVALID_ARG;
    seen[(size_t)c] = 1;
  }
  return SVQ_OK;
}

svq_status validate_handle(const svq_handle *w) {
  if (!w || !w->dev) return SVQ_ERR_INVALID_ARG;
  if (w->n <= 0 || w->k <= 0 || w->k % 8 != 0 || w->bd < 6 || w->bd > 8 || w->bd + w->br != 10)
    return SVQ_ERR_INVALID_ARG;
  const Layout L = make_layout(w->n, w->k);
  if (w->n_tiles != L.n_tiles || w->units != L.units || w->off_codes != L.off_codes ||
      w->off_dtab != L.off_dtab || w->off_rtab != L.off_rtab || w->off_btab != L.off_btab ||
      w->off_xtab != L.off_xtab ||
      w->off_perm != L.off_perm || w->bytes != L.bytes)
    return SVQ_ERR_INVALID_ARG;
  return SVQ_OK;
}

// Build the whole packed image on the host; returns the exact split's power
// of two (or SVQ_NO_EXACT_SPLIT).
int32_t build_image(const svq_matrix_desc *d, const Layout &L, std::vector<uint8_t> &img) {
  img.assign(L.bytes, 0);
  const uint32_t dmask = (1u << d->bd) - 1;
  // direction rows by low index byte
  uint16_t *dtab = (uint16_t *)(img.data() + L.off_dtab);
  for (int b = 0; b < 256; ++b)
    for (int l = 0; l < 8; ++l) dtab[b * 8 + l] = d->dir_codebook[(b & dmask) * 8 + l];
  uint16_t *rtab = (uint16_t *)(img.data() + L.off_rtab);
  for (int idx = 0; idx < 1024; ++idx) rtab[idx] = d->radius_table[idx >> d->bd];
  // bf16 products by full 10-bit index: R*D is exact in float (22 bits)
  uint16_t *btab = (uint16_t *)(img.data() + L.off_btab);
  for (int idx = 0; idx < 1024; ++idx) {
    const int dd = idx & (int)dmask, r = idx >> d->bd;
    const float R = half_to_float(d->radius_table[r]);
    for (int l = 0; l < 8; ++l)
      btab[idx * 8 + l] = float_to_bf16(R * half_to_float(d->dir_codebook[dd * 8 + l]));
  }
  const int32_t xscale = exact_split(d, (uint16_t *)(img.data() + L.off_xtab));
  uint16_t *perm = (uint16_t *)(img.data() + L.off_perm);
  for (int p = 0; p < d->k; ++p) perm[p] = (uint16_t)d->perm[p];

  // coded units
  const int64_t C = d->k / 8;
  const uint8_t *st = d->codes;
  const size_t nbytes = ((size_t)d->n * (size_t)C * 18 + 7) / 8;
  uint8_t *codes = img.data() + L.off_codes;
  for (int64_t i = 0; i < d->n; ++i) {
    const int64_t rt = i / UNIT_ROWS, rho = i % UNIT_ROWS;
    for (int64_t c = 0; c < C; ++c) {
      const uint64_t bit = (uint64_t)(i * C + c) * 18;
      const size_t byte = bit >> 3;
      uint32_t wv = st[byte];
      if (byte + 1 < nbytes) wv |= (uint32_t)st[byte + 1] << 8;
      if (byte + 2 < nbytes) wv |= (uint32_t)st[byte + 2] << 16;
      const uint32_t code = (wv >> (bit & 7)) & FIELD_MASK;
      const int64_t u = c / UNIT_CODES, cc = c % UNIT_CODES;
      // lane 4b + j, code kb = 4*ri + ci: row 4*ri + j, column 16*ci + b
      const int lane = 4 * (int)(cc & 15) + (int)(rho & 3);
      const int kb = 4 * (int)(rho >> 2) + (int)(cc >> 4);
      uint8_t *ub = codes + ((size_t)rt * L.units + (size_t)u) * UNIT_BYTES;
      uint32_t *S = (uint32_t *)(ub + PLANE_SIGN + 16 * lane);
      for (int j = 0; j < 4; ++j) {
        S[j] |= ((code >> (2 * j)) & 1u) << (15 - kb);
        S[j] |= ((code >> (2 * j + 1)) & 1u) << (31 - kb);
      }
      const uint32_t idx = code >> 8;
      ub[PLANE_LOW + 16 * lane + kb] = (uint8_t)(idx & 0xFF);
      uint32_t *H = (uint32_t *)(ub + PLANE_HIGH + 4 * lane);
      *H |= (idx >> 8) << (2 * kb);
    }
  }
  return xscale;
}

MatView view_of(const svq_handle *w) {
  MatView v;
  v.base = (const uint8_t *)w->dev;
  v.off_dtab = (uint32_t)w->off_dtab;
  v.off_rtab = (uint32_t)w->off_rtab;
  v.off_btab = (uint32_t)w->off_btab;
  v.off_xtab = (uint32_t)w->off_xtab;
  v.off_perm = (uint32_t)w->off_perm;
  v.off_codes = w->off_codes;
  v.n = w->n;
  v.k = w->k;
  v.bd = w->bd;
  v.n_tiles = w->n_tiles;
  v.units = w->units;
  return v;
}

}  // namespace

extern "C" {

const char *svq_status_string(svq_status s) {
  switch (s) {
    case SVQ_OK: return "ok";
    case SVQ_ERR_INVALID_ARG: return "invalid argument";
    case SVQ_ERR_UNSUPPORTED: return "unsupported";
    case SVQ_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case SVQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

svq_status svq_pack(const svq_matrix_desc *src, void *dst_dev, size_t *dst_bytes, svq_handle *out,
                    void *stream) {
  if (!dst_bytes) return SVQ_ERR_INVALID_ARG;
  const svq_status st = validate_desc(src);
  if (st != SVQ_OK) return st;
  const Layout L = make_layout(src->n, src->k);
  if (!dst_dev) {
    *dst_bytes = L.bytes;
    return SVQ_OK;
  }
  if (*dst_bytes < L.bytes) {
    *dst_bytes = L.bytes;
    return SVQ_ERR_BUFFER_TOO_SMALL;
  }
  if (!out) return SVQ_ERR_INVALID_ARG;
  std::vector<uint8_t> img;
  const int32_t xscale = build_image(src, L, img);
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(dst_dev, img.data(), L.bytes, hipMemcpyHostToDevice, s) != hipSuccess)
    return SVQ_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SVQ_ERR_HIP;
  std::memset(out, 0, sizeof(*out));
  out->dev = dst_dev;
  out->n = src->n;
  out->k = src->k;
  out->bd = src->bd;
  out->br = src->br;
  out->n_tiles = L.n_tiles;
  out->units = L.units;
  out->off_dtab = L.off_dtab;
  out->off_rtab = L.off_rtab;
  out->off_btab = L.off_btab;
  out->off_xtab = L.off_xtab;
  out->xscale_log2 = xscale;
  out->off_perm = L.off_perm;
  out->off_codes = L.off_codes;
  out->code_bytes = ((uint64_t)src->n * (uint64_t)(src->k / 8) * 18 + 7) / 8;
  out->padded_code_bytes = L.padded_code_bytes;
  out->bytes = L.bytes;
  *dst_bytes = L.bytes;
  return SVQ_OK;
}

// Exact path (m <= 4): plan the blocks of the gather and main launches over
// `count` matrices.  R (row tiles per main block) starts as the largest that
// keeps the block's units (R*U, split evenly between its 4 waves) near
// GV_UNITS_PER_WAVE per wave, at most GV_MAX_R.  Three main blocks share a
// compute unit (registers and LDS allow it at every m), so while the launch
// has more blocks than that, the smallest blocks grow: a block left for a
// second round would start only when a first-round block ends.  Jobs are
// ordered by units per block, largest first: the dispatcher gives blocks i,
// i + CUs and i + 2 CUs to one unit, so a large block runs beside smaller
// ones.  Returns the main launch's blocks.
static int device_cus();
static int plan_gemv(GemvBatch &b, int *gather_blocks) {
  int R[GV_MAX_JOBS];
  for (int j = 0; j < b.count; ++j) {
    const int U = b.job[j].w.units;
    const int r = 4 * GV_UNITS_PER_WAVE / U;
    R[j] = r < 1 ? 1 : (r > GV_MAX_R ? GV_MAX_R : r);
  }
  auto blocks_of = [&](int j) { return (b.job[j].w.n_tiles + R[j] - 1) / R[j]; };
  auto total_blocks = [&]() {
    int t = 0;
    for (int j = 0; j < b.count; ++j) t += blocks_of(j);
    return t;
  };
  const int slots = 3 * device_cus();
  while (total_blocks() > slots) {
    int best = -1;
    for (int j = 0; j < b.count; ++j)
      if (R[j] < GV_MAX_R && blocks_of(j) > 1 &&
          (best < 0 || R[j] * b.job[j].w.units < R[best] * b.job[best].w.units))
        best = j;
    if (best < 0) break;
    ++R[best];
  }
  // order by units per block, largest first (stable)
  int order[GV_MAX_JOBS];
  for (int j = 0; j < b.count; ++j) order[j] = j;
  for (int i = 1; i < b.count; ++i)
    for (int j = i; j > 0 && R[order[j]] * b.job[order[j]].w.units > R[order[j - 1]] * b.job[order[j - 1]].w.units; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  GemvJob sorted[GV_MAX_JOBS];
  int Rs[GV_MAX_JOBS];
  for (int j = 0; j < b.count; ++j) {
    sorted[j] = b.job[order[j]];
    Rs[j] = R[order[j]];
  }
  int begin = 0, gbegin = 0;
  for (int j = 0; j < b.count; ++j) {
    b.job[j] = sorted[j];
    const int U = b.job[j].w.units;
    b.job[j].R = Rs[j];
    b.job[j].block_begin = begin;
    b.starts.first[j] = begin;
    begin += (b.job[j].w.n_tiles + Rs[j] - 1) / Rs[j];
    b.gather_starts.first[j] = gbegin;
    gbegin += b.m * ((U + 3) / 4);
  }
  // table-touch blocks start on a multiple of 8 (block i runs on XCD i % 8)
  b.touch_begin = (gbegin + 7) / 8 * 8;
  *gather_blocks = b.touch_begin + 8 * b.count;
  return begin;
}

// Exact path, m = 1 (one fused launch): R (row tiles per block, 1, 2 or 4)
// is the largest that keeps every wave's work items (one 512-slot unit of one
// row tile each) within GF_ITEMS_PER_WAVE; R halves while the launch has
// fewer than 512 blocks.  Jobs with the largest k come first (their blocks
// run longest).  Returns the launch's blocks.
// Fused m = 1 launch: three 4-wave blocks share a compute unit (LDS and
// registers allow it for every matrix shape this path takes), and the
// dispatcher gives blocks i, i + CUs and i + 2 CUs to one unit when all of
// them fit at once.  So: about total / (3 CUs) items per block (R tiles of
// U units), at most 3 CUs blocks, and jobs ordered by items per block,
// largest first, which puts a large block beside two small ones.
static int plan_fused(GemvBatch &b) {
  int64_t total = 0;
  for (int j = 0; j < b.count; ++j) total += (int64_t)b.job[j].w.n_tiles * b.job[j].w.units;
  // Three blocks per compute unit hide the code latency best when the
  // launch is large; below 8192 items (8 per SIMD) the per-block prologue
  // weighs more and two larger blocks per compute unit are faster
  // (measured: the four calls of a decoder layer, 36 layers, 1.06 against
  // 1.10 ms; the seven-matrix call, 12,320 items, keeps three).
  const int slots = (total < 8192 ? 2 : 3) * device_cus();
  const int target = (int)((total + slots - 1) / slots);
  int R[GV_MAX_JOBS];
  // a block's LDS grows with its row tiles (partial sums): R stays where the
  // block still fits (R = 1 always does: the caller checked)
  auto fits = [&](int j, int r) {
    return gemv_fused_smem_bytes(b.job[j].w.k, b.job[j].w.units, b.job[j].w.bd, r) <= GV_LDS_LIMIT;
  };
  for (int j = 0; j < b.count; ++j) {
    const int U = b.job[j].w.units;
    int r = (target + U / 2) / U;
    R[j] = r < 1 ? 1 : (r > GF_MAX_R ? GF_MAX_R : r);
    while (R[j] > 1 && !fits(j, R[j])) --R[j];
  }
  auto blocks_of = [&](int j) { return (b.job[j].w.n_tiles + R[j] - 1) / R[j]; };
  auto total_blocks = [&]() {
    int t = 0;
    for (int j = 0; j < b.count; ++j) t += blocks_of(j);
    return t;
  };
  // too many blocks for one round: grow the smallest blocks
  while (total_blocks() > slots) {
    int best = -1;
    for (int j = 0; j < b.count; ++j)
      if (R[j] < GF_MAX_R && blocks_of(j) > 1 && fits(j, R[j] + 1) &&
          (best < 0 || R[j] * b.job[j].w.units < R[best] * b.job[best].w.units))
        best = j;
    if (best < 0) break;
    ++R[best];
  }
  int order[GV_MAX_JOBS];
  for (int j = 0; j < b.count; ++j) order[j] = j;
  for (int i = 1; i < b.count; ++i)
    for (int j = i; j > 0 && R[order[j]] * b.job[order[j]].w.units > R[order[j - 1]] * b.job[order[j - 1]].w.units; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  GemvJob sorted[GV_MAX_JOBS];
  int Rs[GV_MAX_JOBS];
  for (int j = 0; j < b.count; ++j) {
    sorted[j] = b.job[order[j]];
    Rs[j] = R[order[j]];
  }
  int begin = 0;
  for (int j = 0; j < b.count; ++j) {
    b.job[j] = sorted[j];
    b.job[j].R = Rs[j];
    b.job[j].block_begin = begin;
    b.starts.first[j] = begin;
    begin += (b.job[j].w.n_tiles + Rs[j] - 1) / Rs[j];
  }
  return begin;
}

// Compute units of the current device.
static int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// K splits of the dequant-GEMM jobs: when the output tiles alone give fewer
// than two blocks per compute unit (small m), each job's units are cut into
// splits of about the same number of units, so that about two blocks per
// compute unit result.  ups[j] = units per split; returns the partial-sum
// workspace bytes (0 without splits).
static size_t plan_splits(const svq_handle *w, int32_t count, int m_pad, int bm, int *splits,
                          int *ups) {
  const int tiles_m = m_pad / bm;
  int64_t blocks = 0, work = 0;
  for (int32_t j = 0; j < count; ++j) {
    const int64_t tn = prefill_tiles_n((w[j].n + UNIT_ROWS - 1) / UNIT_ROWS);
    blocks += tn * tiles_m;
    work += tn * tiles_m * w[j].units;
    splits[j] = 1;
    ups[j] = w[j].units;
  }
  const int64_t target = 2 * (int64_t)device_cus();
  if (blocks >= target) return 0;
  const int64_t per = (work + target - 1) / target;  // units per block
  size_t bytes = 0;
  for (int32_t j = 0; j < count; ++j) {
    const int U = w[j].units;
    int sp = (int)((U + per - 1) / per);
    sp = sp < 1 ? 1 : sp;
    ups[j] = (U + sp - 1) / sp;
    splits[j] = (U + ups[j] - 1) / ups[j];
    if (splits[j] > 1) {
      const size_t n_pad = (size_t)prefill_tiles_n((w[j].n + UNIT_ROWS - 1) / UNIT_ROWS) * 256;
      bytes += align256((size_t)splits[j] * m_pad * n_pad * 4);
    }
  }
  return bytes;
}

static svq_status linear_impl(const svq_handle *w, int32_t count, const void *const *xs,
                              const int64_t *ldx, int64_t m, void *const *ys, const int64_t *ldy,
                              svq_dtype ydt, void *workspace, size_t *workspace_bytes,
                              void *stream) {
  if (!workspace_bytes || !w) return SVQ_ERR_INVALID_ARG;
  if (count < 1 || count > GV_MAX_JOBS) return SVQ_ERR_INVALID_ARG;
  if (m < 1 || m > (1 << 24)) return SVQ_ERR_INVALID_ARG;
  if (ydt != SVQ_BF16 && ydt != SVQ_F32) return SVQ_ERR_INVALID_ARG;
  for (int32_t j = 0; j < count; ++j) {
    const svq_status st = validate_handle(&w[j]);
    if (st != SVQ_OK) return st;
  }
  int k_max = 0, bd_max = 0, u_max = 0;
  for (int32_t j = 0; j < count; ++j) {
    k_max = w[j].k > k_max ? w[j].k : k_max;
    bd_max = w[j].bd > bd_max ? w[j].bd : bd_max;
    u_max = w[j].units > u_max ? w[j].units : u_max;
  }
  const bool exact = m <= EXACT_MAX_M;
  bool split_ok = true;
  for (int32_t j = 0; j < count; ++j)
    if (w[j].xscale_log2 == SVQ_NO_EXACT_SPLIT || w[j].xscale_log2 < -120 || w[j].xscale_log2 > 120)
      split_ok = false;
  if (!exact && m <= SB_MAX_M && !split_ok) {
    // tables without an exact fp16 split: the m <= 4 kernels, four
    // activation rows at a time (each chunk's workspace is the same size)
    size_t need4 = 0;
    svq_status st = linear_impl(w, count, nullptr, ldx, EXACT_MAX_M, nullptr, ldy, ydt, nullptr, &need4,
                                stream);
    if (st != SVQ_OK) return st;
    if (!workspace) {
      *workspace_bytes = need4;
      return SVQ_OK;
    }
    if (!xs || !ys || !ldx || !ldy) return SVQ_ERR_INVALID_ARG;
    const size_t esz = ydt == SVQ_BF16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < m; r0 += EXACT_MAX_M) {
      const void *xc[GV_MAX_JOBS];
      void *yc[GV_MAX_JOBS];
      for (int32_t j = 0; j < count; ++j) {
        if (!xs[j] || !ys[j]) return SVQ_ERR_INVALID_ARG;
        xc[j] = (const uint16_t *)xs[j] + r0 * ldx[j];
        yc[j] = (uint8_t *)ys[j] + (size_t)(r0 * ldy[j]) * esz;
      }
      size_t cap = *workspace_bytes;
      const int64_t mc = m - r0 < EXACT_MAX_M ? m - r0 : EXACT_MAX_M;
      st = linear_impl(w, count, xc, ldx, mc, yc, ldy, ydt, workspace, &cap, stream);
      if (st != SVQ_OK) return st;
    }
    return SVQ_OK;
  }
  const bool small = !exact && m <= SB_MAX_M;
  int sb_items = 0;
  if (small) {
    int64_t total = 0;
    for (int32_t j = 0; j < count; ++j) total += (int64_t)w[j].n_tiles * w[j].units;
    sb_items = sb_block_items(total, device_cus());
  }
  // m = 1: the fused launch, when the activation row and its permuted copy
  // fit in LDS beside the tables
  size_t fused_smem = 0;
  for (int32_t j = 0; j < count; ++j) {
    const size_t b = gemv_fused_smem_bytes(w[j].k, w[j].units, w[j].bd, 1);
    fused_smem = b > fused_smem ? b : fused_smem;
  }
  const bool fused = m == 1 && fused_smem <= GV_LDS_LIMIT;
  size_t need = 0;
  int m_pad = 0;
  int splits[GV_MAX_JOBS], ups[GV_MAX_JOBS];
  if (fused) {
    need = 256;  // unused: the fused launch gathers in LDS
  } else if (exact) {
    for (int32_t j = 0; j < count; ++j) need += gemv_ws_bytes((int)m, w[j].units);
  } else if (small) {
    for (int32_t j = 0; j < count; ++j) need += sb_ws_bytes(w[j].n_tiles, w[j].units, sb_items);
  } else {
    m_pad = prefill_m_pad((int)m);
    need = plan_splits(w, count, m_pad, prefill_bm((int)m), splits, ups);
    for (int32_t j = 0; j < count; ++j)
      need += align256((size_t)m_pad * w[j].units * UNIT_SLOTS * 2);
  }
  if (!workspace) {
    if (ldx && ldy)
      for (int32_t j = 0; j < count; ++j)
        if (ldx[j] < w[j].k || ldy[j] < w[j].n) return SVQ_ERR_INVALID_ARG;
    *workspace_bytes = need;
    return SVQ_OK;
  }
  if (!xs || !ys || !ldx || !ldy) return SVQ_ERR_INVALID_ARG;
  for (int32_t j = 0; j < count; ++j) {
    if (!xs[j] || !ys[j]) return SVQ_ERR_INVALID_ARG;
    if (ldx[j] < w[j].k || ldy[j] < w[j].n) return SVQ_ERR_INVALID_ARG;
  }
  if (*workspace_bytes < need) return SVQ_ERR_BUFFER_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (exact) {
    GemvBatch b;
    std::memset(&b, 0, sizeof(b));
    b.count = count;
    b.m = (int)m;
    b.ydt = (int)ydt;
    uint8_t *ws = (uint8_t *)workspace;
    for (int32_t j = 0; j < count; ++j) {
      b.job[j].w = view_of(&w[j]);
      b.job[j].x = (const uint16_t *)xs[j];
      b.job[j].ldx = ldx[j];
      if (!fused) {
        b.job[j].xg = ws;
        b.job[j].xs = (float *)(ws + align256((size_t)m * w[j].units * GV_XG_UNIT_BYTES));
        ws += gemv_ws_bytes((int)m, w[j].units);
      }
      b.job[j].y = ys[j];
      b.job[j].ldy = ldy[j];
    }
    b.xvec = 1;
    for (int32_t j = 0; j < count; ++j)
      if ((((uintptr_t)xs[j]) | ((uintptr_t)ldx[j] * 2)) & 15) b.xvec = 0;
    if (fused) {
      const int blocks = plan_fused(b);
      // LDS of the launch: the largest block of the plan (the partial sums
      // grow with the row tiles per block)
      size_t smem = 0;
      for (int32_t j = 0; j < count; ++j) {
        const size_t bj = gemv_fused_smem_bytes(b.job[j].w.k, b.job[j].w.units, b.job[j].w.bd, b.job[j].R);
        smem = bj > smem ? bj : smem;
      }
      if (smem > GV_LDS_LIMIT) return SVQ_ERR_UNSUPPORTED;
      e = launch_gemv_fused(b, blocks, smem, s);
      return e == hipSuccess ? SVQ_OK : SVQ_ERR_HIP;
    }
    int gather_blocks = 0;
    const int blocks = plan_gemv(b, &gather_blocks);
    int r_max = 1;
    for (int32_t j = 0; j < count; ++j) r_max = b.job[j].R > r_max ? b.job[j].R : r_max;
    const size_t smem = gemv_smem_bytes((int)m, bd_max, r_max);
    b.red_off = (int32_t)gemv_smem_bytes((int)m, bd_max, 0);
    e = launch_gemv_batched(b, gather_blocks, k_max, blocks, smem, s);
  } else if (small) {
    // fragment-ordered activations (one prep launch), then one launch over
    // every (tile group, K range) of every matrix
    SbBatch b;
    std::memset(&b, 0, sizeof(b));
    b.count = count;
    b.m = (int)m;
    b.ydt = (int)ydt;
    uint8_t *ws = (uint8_t *)workspace;
    int blocks = 0, prep_blocks = 0;
    for (int32_t j = 0; j < count; ++j) {
      SbJob &J = b.job[j];
      J.w = view_of(&w[j]);
      J.x = (const uint16_t *)xs[j];
      J.ldx = ldx[j];
      J.y = ys[j];
      J.ldy = ldy[j];
      const SbPlan pl = sb_plan(J.w.n_tiles, J.w.units, sb_items);
      J.tiles = pl.tiles;
      J.upr = pl.upr;
      J.groups = pl.groups;
      J.splits = pl.splits;
      J.xa = ws;
      J.xs = (float *)(ws + align256((size_t)J.w.units * SB_XA_UNIT_BYTES));
      J.xinv = std::ldexp(1.0f, -w[j].xscale_log2);
      uint8_t *p = (uint8_t *)J.xs + align256((size_t)J.w.units * 16 * 4);
      if (J.splits > 1) {
        J.part = (float *)p;
        p += align256((size_t)J.groups * J.tiles * J.splits * 1024);
        J.cnt = (int32_t *)p;
      }
      ws += sb_ws_bytes(J.w.n_tiles, J.w.units, sb_items);
    }
    // matrices cut into K ranges first: the tail of their blocks (partial
    // tiles, arrival counts) then overlaps the other matrices' blocks
    for (int i = 1; i < b.count; ++i)
      for (int j = i; j > 0 && b.job[j].splits > b.job[j - 1].splits; --j) {
        const SbJob t = b.job[j];
        b.job[j] = b.job[j - 1];
        b.job[j - 1] = t;
      }
    for (int32_t j = 0; j < count; ++j) {
      SbJob &J = b.job[j];
      J.block_begin = blocks;
      blocks += J.groups * J.splits;
      J.prep_begin = prep_blocks;
      prep_blocks += J.w.units;
      b.starts.first[j] = J.block_begin;
      b.prep_starts.first[j] = J.prep_begin;
    }
    e = launch_sb(b, prep_blocks, blocks, s);
  } else {
    // permuted activations of every matrix in fragment order (one prep
    // launch), then one GEMM launch over all of them, longest k first
    PrefillBatch b;
    std::memset(&b, 0, sizeof(b));
    b.count = count;
    b.ydt = (int)ydt;
    uint8_t *ws = (uint8_t *)workspace;
    bool xvec = true;
    for (int32_t j = 0; j < count; ++j) {
      const MatView v = view_of(&w[j]);
      b.job[j].w = v;
      b.job[j].x = (const uint16_t *)xs[j];
      b.job[j].ldx = ldx[j];
      b.job[j].xb = (uint16_t *)ws;
      ws += align256((size_t)m_pad * w[j].units * UNIT_SLOTS * 2);
      b.job[j].m = (int32_t)m;
      b.job[j].y = ys[j];
      b.job[j].ldy = ldy[j];
      b.job[j].tiles_n = prefill_tiles_n(v.n_tiles);
      b.job[j].splits = splits[j];
      b.job[j].units_per_split = ups[j];
      b.job[j].m_pad = m_pad;
      b.job[j].n_pad = b.job[j].tiles_n * 256;
      if ((((uintptr_t)xs[j]) | ((uintptr_t)ldx[j] * 2)) & 15) xvec = false;
    }
    bool any_split = false;
    for (int32_t j = 0; j < count; ++j) {
      if (splits[j] > 1) {
        b.job[j].part = (float *)ws;
        ws += align256((size_t)splits[j] * m_pad * b.job[j].n_pad * 4);
        any_split = true;
      }
    }
    const size_t esz = ydt == SVQ_BF16 ? 2 : 4;
    b.yvec = 1;
    for (int32_t j = 0; j < count; ++j)
      if ((((uintptr_t)ys[j]) | ((uintptr_t)ldy[j] * esz)) & 15) b.yvec = 0;
    for (int i = 1; i < b.count; ++i)
      for (int j = i; j > 0 && b.job[j].w.k > b.job[j - 1].w.k; --j) {
        const PrefillJob t = b.job[j];
        b.job[j] = b.job[j - 1];
        b.job[j - 1] = t;
      }
    // jobs start on multiples of 8 GEMM blocks (the XCD count) so that a
    // job's blocks with one m-tile share an XCD; the padding blocks exit at
    // once
    int blocks = 0, prep_blocks = 0, red_blocks = 0;
    // prep: row groups of prep_rpb rows (fewer rows for long k); with few
    // groups, each job's chunks are also cut into ranges (at least 64 chunks
    // each) for about 512 blocks
    size_t prep_lds = 0;
    int row_groups = 0;
    for (int j = 0; j < b.count; ++j) {
      const int rpb = prefill_prep_rows(b.job[j].w.k);
      b.job[j].prep_rpb = rpb;
      row_groups += m_pad / rpb;
      const size_t l = prefill_prep_lds(rpb, b.job[j].w.k);
      prep_lds = l > prep_lds ? l : prep_lds;
    }
    const int want = (512 + row_groups - 1) / row_groups;
    for (int j = 0; j < b.count; ++j) {
      const int nch = b.job[j].w.units * UNIT_SLOTS / 8;
      int cs = want < nch / 64 ? want : nch / 64;
      b.job[j].prep_csplit = cs < 1 ? 1 : cs;
    }
    for (int j = 0; j < b.count; ++j) {
      b.job[j].tiles_m = m_pad / prefill_bm((int)m);
      b.job[j].block_begin = blocks;
      blocks += (b.job[j].tiles_n * b.job[j].tiles_m * b.job[j].splits + 7) / 8 * 8;
      b.job[j].prep_begin = prep_blocks;
      prep_blocks += (m_pad / b.job[j].prep_rpb) * b.job[j].prep_csplit;
      b.job[j].red_begin = red_blocks;
      if (b.job[j].splits > 1) red_blocks += (int)m * ((b.job[j].w.n + 1023) / 1024);
      b.gemm_starts.first[j] = b.job[j].block_begin;
      b.prep_starts.first[j] = b.job[j].prep_begin;
      b.red_starts.first[j] = b.job[j].red_begin;
    }
    e = launch_prefill_prep(b, prep_blocks, prep_lds, xvec, s);
    if (e == hipSuccess) e = launch_prefill_batched(b, prefill_bm((int)m), blocks, s);
    if (e == hipSuccess && any_split) e = launch_prefill_reduce(b, red_blocks, s);
  }
  return e == hipSuccess ? SVQ_OK : SVQ_ERR_HIP;
}

svq_status svq_linear(const svq_handle *w, const void *x, int64_t m, int64_t ldx, void *y,
                      int64_t ldy, svq_dtype ydt, void *workspace, size_t *workspace_bytes,
                      void *stream) {
  void *yy = y;
  return linear_impl(w, 1, &x, &ldx, m, &yy, &ldy, ydt, workspace, workspace_bytes, stream);
}

svq_status svq_linear_batched(const svq_handle *w, int32_t count, const void *const *x,
                              const int64_t *ldx, int64_t m, void *const *y, const int64_t *ldy,
                              svq_dtype ydt, void *workspace, size_t *workspace_bytes,
                              void *stream) {
  return linear_impl(w, count, x, ldx, m, y, ldy, ydt, workspace, workspace_bytes, stream);
}

svq_status svq_linear_noalloc(const svq_handle *w, const void *x, int64_t m, int64_t ldx, void *y,
                              int64_t ldy, svq_dtype ydt, void *stream) {
  // the same plan as svq_linear; its workspace comes from the library's
  // scratch, so the size is checked before anything touches the device
  size_t need = 0;
  svq_status st = svq_linear(w, nullptr, m, ldx, nullptr, ldy, ydt, nullptr, &need, stream);
  if (st != SVQ_OK) return st;
  if (need > SCRATCH_BYTES) return SVQ_ERR_UNSUPPORTED;
  void *ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return SVQ_ERR_HIP;
  size_t cap = SCRATCH_BYTES;
  return svq_linear(w, x, m, ldx, y, ldy, ydt, ws, &cap, stream);
}

// Checks shared by the MoE calls: the routing arguments, then every
// projection's experts (one n and k per projection).
static svq_status moe_check(const svq_handle *const *experts, int32_t count, int32_t num_experts,
                            int32_t x_per_slot, int64_t m, int32_t topk, svq_dtype ydt) {
  if (num_experts < 1 || num_experts > MAX_EXPERTS) return SVQ_ERR_UNSUPPORTED;
  if (count < 1 || count > MOE_BATCH_MAX) return SVQ_ERR_INVALID_ARG;
  if (count * num_experts > MAX_EXPERTS) return SVQ_ERR_UNSUPPORTED;
  if (topk < 1 || topk > num_experts || m < 1 || m > (1 << 20)) return SVQ_ERR_INVALID_ARG;
  if (x_per_slot != 0 && x_per_slot != 1) return SVQ_ERR_INVALID_ARG;
  if (ydt != SVQ_BF16 && ydt != SVQ_F32) return SVQ_ERR_INVALID_ARG;
  for (int32_t c = 0; c < count; ++c) {
    if (!experts[c]) return SVQ_ERR_INVALID_ARG;
    for (int32_t e = 0; e < num_experts; ++e) {
      const svq_status st = validate_handle(&experts[c][e]);
      if (st != SVQ_OK) return st;
      if (experts[c][e].n != experts[c][0].n || experts[c][e].k != experts[c][0].k)
        return SVQ_ERR_INVALID_ARG;
    }
  }
  return SVQ_OK;
}

static svq_status moe_impl(const svq_handle *const *experts, int32_t count, int32_t num_experts,
                           const void *const *x, const int64_t *ldx, int32_t x_per_slot,
                           const int32_t *expert_ids, int64_t m, int32_t topk, void *const *y,
                           const int64_t *ldy, svq_dtype ydt, void *workspace,
                           size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes || !experts) return SVQ_ERR_INVALID_ARG;
  svq_status st = moe_check(experts, count, num_experts, x_per_slot, m, topk, ydt);
  if (st != SVQ_OK) return st;
  // strides are checked whenever they are given (the query may omit them)
  for (int32_t c = 0; c < count; ++c) {
    if (ldx && ldx[c] < experts[c][0].k) return SVQ_ERR_INVALID_ARG;
    if (ldy && ldy[c] < experts[c][0].n) return SVQ_ERR_INVALID_ARG;
  }
  size_t need = 0;
  hipError_t e = launch_moe(experts, count, num_experts, nullptr, nullptr, x_per_slot, expert_ids, m,
                            topk, nullptr, nullptr, (int)ydt, nullptr, 0, (hipStream_t)stream, &need);
  if (e != hipSuccess) return SVQ_ERR_INVALID_ARG;
  if (!workspace) {
    *workspace_bytes = need;
    return SVQ_OK;
  }
  if (*workspace_bytes < need) return SVQ_ERR_BUFFER_TOO_SMALL;
  if (!x || !ldx || !y || !ldy || !expert_ids) return SVQ_ERR_INVALID_ARG;
  for (int32_t c = 0; c < count; ++c)
    if (!x[c] || !y[c]) return SVQ_ERR_INVALID_ARG;
  e = launch_moe(experts, count, num_experts, x, ldx, x_per_slot, expert_ids, m, topk, y, ldy, (int)ydt,
                 workspace, *workspace_bytes, (hipStream_t)stream, &need);
  return e == hipSuccess ? SVQ_OK : SVQ_ERR_HIP;
}

svq_status svq_moe_linear(const svq_handle *experts, int32_t num_experts, const void *x,
                          int64_t ldx, int32_t x_per_slot, const int32_t *expert_ids, int64_t m,
                          int32_t topk, void *y, int64_t ldy, svq_dtype ydt, void *workspace,
                          size_t *workspace_bytes, void *stream) {
  const svq_handle *const sets[1] = {experts};
  const void *const xs[1] = {x};
  void *const ys[1] = {y};
  return moe_impl(sets, 1, num_experts, xs, &ldx, x_per_slot, expert_ids, m, topk, ys, &ldy, ydt,
                  workspace, workspace_bytes, stream);
}

svq_status svq_moe_linear_batched(const svq_handle *const *experts, int32_t count,
                                  int32_t num_experts, const void *const *x, const int64_t *ldx,
                                  int32_t x_per_slot, const int32_t *expert_ids, int64_t m,
                                  int32_t topk, void *const *y, const int64_t *ldy, svq_dtype ydt,
                                  void *workspace, size_t *workspace_bytes, void *stream) {
  return moe_impl(experts, count, num_experts, x, ldx, x_per_slot, expert_ids, m, topk, y, ldy, ydt,
                  workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Encoder tables in double precision: the codebook (rows x 8), the squared
// midpoints of consecutive radii and the radii.  Rejects a non-finite
// codebook and radii that are not finite, >= 0 and strictly increasing.
struct EncTables {
  std::vector<double> cb, msq, rad;
};

svq_status enc_tables(int32_t bd, const uint16_t *codebook, const uint16_t *radius, EncTables &t) {
  if (!codebook || !radius) return SVQ_ERR_INVALID_ARG;
  if (bd < 6 || bd > 8) return SVQ_ERR_UNSUPPORTED;
  const int rows = 1 << bd, nrad = 1 << (10 - bd);
  t.cb.assign((size_t)rows * 8, 0.0);
  t.msq.assign((size_t)nrad - 1, 0.0);
  t.rad.assign((size_t)nrad, 0.0);
  for (int e = 0; e < rows * 8; ++e) {
    if (((codebook[e] >> 10) & 0x1F) == 0x1F) return SVQ_ERR_INVALID_ARG;
    t.cb[(size_t)e] = (double)half_to_float(codebook[e]);
  }
  for (int r = 0; r < nrad; ++r) {
    if (((radius[r] >> 10) & 0x1F) == 0x1F) return SVQ_ERR_INVALID_ARG;
    t.rad[(size_t)r] = (double)half_to_float(radius[r]);
    if (t.rad[(size_t)r] < 0.0 || (r > 0 && !(t.rad[(size_t)r] > t.rad[(size_t)r - 1])))
      return SVQ_ERR_INVALID_ARG;
  }
  for (int r = 0; r + 1 < nrad; ++r) {
    const double mid = (t.rad[(size_t)r] + t.rad[(size_t)r + 1]) / 2.0;  // exact (12 significant bits)
    t.msq[(size_t)r] = mid * mid;                                         // exact (24 significant bits)
  }
  return SVQ_OK;
}

bool valid_perm(const int32_t *perm, int32_t k) {
  std::vector<uint8_t> seen((size_t)k, 0);
  for (int32_t p = 0; p < k; ++p) {
    const int32_t c = perm[p];
    if (c < 0 || c >= k || seen[(size_t)c]) return false;
    seen[(size_t)c] = 1;
  }
  return true;
}

// device copies of one candidate's tables: codebook, squared midpoints, radii
constexpr size_t ENC_TAB_BYTES = 256 * 8 * sizeof(double) + 2 * 16 * sizeof(double);

hipError_t stage_tables(const EncTables &t, uint8_t *dst, EncArgs &a, hipStream_t s) {
  const size_t cb = t.cb.size() * sizeof(double), ms = t.msq.size() * sizeof(double);
  a.cb = (const double *)dst;
  a.msq = (const double *)(dst + cb);
  a.rad = (const double *)(dst + cb + ms);
  a.n_mid = (int32_t)t.msq.size();
  hipError_t e = hipMemcpyAsync(dst, t.cb.data(), cb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(dst + cb, t.msq.data(), ms, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dst + cb + ms, t.rad.data(), t.rad.size() * sizeof(double),
                       hipMemcpyHostToDevice, s);
  return e;
}

}  // namespace

namespace {

// svq_encode and svq_encode_weighted: fit_h null selects the plain rule.
svq_status encode_impl(const float *w, int64_t ldw, int32_t n, int32_t k, int32_t bd,
                       const uint16_t *codebook, const uint16_t *radius, const int32_t *perm,
                       const double *fit_h, bool weighted, void *codes, void *workspace,
                       size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes || !codebook || !radius || !perm) return SVQ_ERR_INVALID_ARG;
  if (n <= 0 || k <= 0 || k % 8 != 0) return SVQ_ERR_INVALID_ARG;
  if (bd < 6 || bd > 8) return SVQ_ERR_UNSUPPORTED;
  if (k > SVQ_MAX_K || n > SVQ_MAX_N) return SVQ_ERR_UNSUPPORTED;
  if (ldw < k) return SVQ_ERR_INVALID_ARG;
  EncTables tab;
  const svq_status st = enc_tables(bd, codebook, radius, tab);
  if (st != SVQ_OK) return st;
  if (!valid_perm(perm, k)) return SVQ_ERR_INVALID_ARG;
  const size_t tab_bytes = align256(ENC_TAB_BYTES);
  const size_t need = tab_bytes + align256((size_t)k * sizeof(int32_t));
  if (!workspace) {
    *workspace_bytes = need;
    return SVQ_OK;
  }
  if (!w || !codes || (weighted && !fit_h)) return SVQ_ERR_INVALID_ARG;
  if (*workspace_bytes < need) return SVQ_ERR_BUFFER_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  EncArgs a{};
  a.w = w;
  a.ldw = ldw;
  a.n = n;
  a.k = k;
  a.bd = bd;
  a.perm = (const int32_t *)(ws + tab_bytes);
  a.codes = (uint8_t *)codes;
  a.count = (int64_t)n * (k / 8);
  a.fit_h = weighted ? fit_h : nullptr;
  hipError_t e = stage_tables(tab, ws, a, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(ws + tab_bytes, perm, (size_t)k * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = launch_encode(a, s);
  // the staged host arrays must outlive the copies
  const hipError_t e2 = hipStreamSynchronize(s);
  if (e == hipSuccess) e = e2;
  return e == hipSuccess ? SVQ_OK : SVQ_ERR_HIP;
}

}  // namespace

svq_status svq_encode(const float *w, int64_t ldw, int32_t n, int32_t k, int32_t bd,
                      const uint16_t *codebook, const uint16_t *radius, const int32_t *perm,
                      void *codes, void *workspace, size_t *workspace_bytes, void *stream) {
  return encode_impl(w, ldw, n, k, bd, codebook, radius, perm, nullptr, false, codes, workspace,
                     workspace_bytes, stream);
}

svq_status svq_encode_weighted(const float *w, int64_t ldw, int32_t n, int32_t k, int32_t bd,
                               const uint16_t *codebook, const uint16_t *radius, const int32_t *perm,
                               const double *h, void *codes, void *workspace, size_t *workspace_bytes,
                               void *stream) {
  return encode_impl(w, ldw, n, k, bd, codebook, radius, perm, h, true, codes, workspace,
                     workspace_bytes, stream);
}

svq_status svq_esg_perm(const void *x, int64_t t, int64_t ldx, int32_t k, double *energy,
                        int32_t *perm, void *workspace, size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes) return SVQ_ERR_INVALID_ARG;
  if (k <= 0 || k % 8 != 0 || t < 1 || ldx < k || ldx % 8 != 0) return SVQ_ERR_INVALID_ARG;
  if (k > SVQ_MAX_K) return SVQ_ERR_UNSUPPORTED;
  const size_t need = align256((size_t)k * sizeof(int32_t));
  if (!workspace) {
    *workspace_bytes = need;
    return SVQ_OK;
  }
  if (!x || !energy || !perm || ((uintptr_t)x & 15) != 0) return SVQ_ERR_INVALID_ARG;
  if (*workspace_bytes < need) return SVQ_ERR_BUFFER_TOO_SMALL;
  EsgArgs a;
  a.x = (const uint16_t *)x;
  a.t = t;
  a.ldx = ldx;
  a.k = k;
  a.energy = energy;
  a.rank = (int32_t *)workspace;
  a.perm = perm;
  return launch_esg(a, (hipStream_t)stream) == hipSuccess ? SVQ_OK : SVQ_ERR_HIP;
}

svq_status svq_abs_select(const float *w, int64_t ldw, int32_t n, int32_t k, const double *h,
                          const int32_t *perm, int32_t n_cand, const int32_t *bd,
                          const uint16_t *const *codebooks, const uint16_t *const *radii,
                          int32_t weighted_fit, void *codes, int32_t *chosen, double *errors,
                          void *workspace, size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes || !perm || !bd || !codebooks || !radii) return SVQ_ERR_INVALID_ARG;
  if (weighted_fit != 0 && weighted_fit != 1) return SVQ_ERR_INVALID_ARG;
  if (n <= 0 || k <= 0 || k % 8 != 0 || ldw < k) return SVQ_ERR_INVALID_ARG;
  if (n_cand < 1 || n_cand > 8) return SVQ_ERR_INVALID_ARG;
  if (k > SVQ_MAX_K || n > SVQ_MAX_N) return SVQ_ERR_UNSUPPORTED;
  std::vector<EncTables> tabs((size_t)n_cand);
  for (int c = 0; c < n_cand; ++c) {
    const svq_status st = enc_tables(bd[c], codebooks[c], radii[c], tabs[(size_t)c]);
    if (st != SVQ_OK) return st;
  }
  if (!valid_perm(perm, k)) return SVQ_ERR_INVALID_ARG;
  const int64_t count = (int64_t)n * (k / 8);
  const size_t stream_bytes = (size_t)((count * 18 + 7) / 8);
  const size_t tab_bytes = align256(ENC_TAB_BYTES), perm_bytes = align256((size_t)k * sizeof(int32_t));
  const size_t codes_slot = align256(stream_bytes), err_bytes = align256((size_t)count * sizeof(double));
  const size_t rows_bytes = align256((size_t)n_cand * (size_t)n * sizeof(double));
  const size_t off_perm = (size_t)n_cand * tab_bytes, off_codes = off_perm + perm_bytes;
  const size_t off_err = off_codes + (size_t)n_cand * codes_slot, off_rows = off_err + err_bytes;
  const size_t off_tot = off_rows + rows_bytes, need = off_tot + align256(8 * sizeof(double));
  if (!workspace) {
    *workspace_bytes = need;
    return SVQ_OK;
  }
  if (!w || !h || !codes || !chosen || !errors) return SVQ_ERR_INVALID_ARG;
  if (*workspace_bytes < need) return SVQ_ERR_BUFFER_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  hipError_t e = hipMemcpyAsync(ws + off_perm, perm, (size_t)k * sizeof(int32_t), hipMemcpyHostToDevice, s);
  for (int c = 0; c < n_cand && e == hipSuccess; ++c) {
    EncArgs a{};
    a.w = w;
    a.ldw = ldw;
    a.n = n;
    a.k = k;
    a.bd = bd[c];
    a.perm = (const int32_t *)(ws + off_perm);
    a.codes = ws + off_codes + (size_t)c * codes_slot;
    a.count = count;
    a.h = h;
    a.fit_h = weighted_fit ? h : nullptr;
    a.err = (double *)(ws + off_err);  // reused: the row sums of c run before c + 1 is coded
    e = stage_tables(tabs[(size_t)c], ws + (size_t)c * tab_bytes, a, s);
    if (e == hipSuccess) e = launch_encode(a, s);
    if (e == hipSuccess)
      e = launch_abs_rows(a.err, n, k / 8, (double *)(ws + off_rows) + (size_t)c * n, s);
  }
  if (e == hipSuccess) e = launch_abs_totals((const double *)(ws + off_rows), n, n_cand,
                                             (double *)(ws + off_tot), s);
  double tot[8] = {0};
  if (e == hipSuccess)
    e = hipMemcpyAsync(tot, ws + off_tot, (size_t)n_cand * sizeof(double), hipMemcpyDeviceToHost, s);
  // the staged host tables must outlive the copies; the totals decide
  const hipError_t e2 = hipStreamSynchronize(s);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) return SVQ_ERR_HIP;
  int best = 0;
  for (int c = 1; c < n_cand; ++c)
    if (tot[c] < tot[best]) best = c;
  e = hipMemcpyAsync(codes, ws + off_codes + (size_t)best * codes_slot, stream_bytes,
                     hipMemcpyDeviceToDevice, s);
  const hipError_t e3 = hipStreamSynchronize(s);
  if (e == hipSuccess) e = e3;
  if (e != hipSuccess) return SVQ_ERR_HIP;
  *chosen = best;
  for (int c = 0; c < n_cand; ++c) errors[c] = tot[c];
  return SVQ_OK;
}
