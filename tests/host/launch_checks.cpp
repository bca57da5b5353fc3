// Host-side stand-ins for libsvq's kernel launchers and for the few HIP
// runtime calls svq_host.cpp makes, so that the library's host code (argument
// checks, repack, planners, workspace layout) runs on a machine without a GPU
// under AddressSanitizer / UndefinedBehaviorSanitizer.  Each launcher checks
// the launch it is handed instead of running it: every block's tiles and
// units lie inside its matrix, every code load of every wave (from the
// schedule helpers the kernels use) lies inside the packed buffer's code
// region, LDS fits a compute unit and workspace regions fit the workspace.
// A failed check prints the launch and aborts.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../bit_spherical_vector_amd/csrc/svq_internal.h"
#include "../../include/svq.h"

#define CHECK(cond, ...)                                                   \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "launch check failed (%s:%d): %s: ", __FILE__, \
                   __LINE__, #cond);                                       \
      std::fprintf(stderr, __VA_ARGS__);                                   \
      std::fprintf(stderr, "\n");                                          \
      std::abort();                                                        \
    }                                                                      \
  } while (0)

// ---- workspace and buffer registry (filled by the harness) -------------
namespace check {
const uint8_t *ws_base = nullptr;
size_t ws_bytes = 0;
long launches = 0, loads_checked = 0;

// Codes of a matrix: [base + off_codes, base + off_codes + n_tiles*units*UNIT_BYTES)
void check_code_load(const svq::MatView &w, size_t off, const char *what) {
  const size_t lo = w.off_codes, hi = w.off_codes + (size_t)w.n_tiles * w.units * svq::UNIT_BYTES;
  CHECK(off >= lo && off + svq::UNIT_BYTES <= hi, "%s: unit at +%zu outside codes [%zu, %zu)", what,
        off, lo, hi);
  ++loads_checked;
}
void check_ws(const void *p, size_t bytes, const char *what) {
  const uint8_t *q = (const uint8_t *)p;
  CHECK(ws_base && q >= ws_base && q + bytes <= ws_base + ws_bytes,
        "%s: %zu bytes at ws+%td outside the %zu-byte workspace", what, bytes, q - ws_base, ws_bytes);
}
}  // namespace check

// ---- HIP runtime calls of svq_host.cpp -----------------------------------
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t a, int) {
  *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

namespace svq {

// ---- exact path ----------------------------------------------------------
hipError_t launch_gemv_fused(GemvBatch &b, int blocks, size_t smem, hipStream_t) {
  ++check::launches;
  CHECK(smem <= GV_LDS_LIMIT, "fused LDS %zu", smem);
  CHECK(b.count >= 1 && b.count <= GV_MAX_JOBS, "count %d", b.count);
  int next = 0;
  for (int j = 0; j < b.count; ++j) {
    const GemvJob &J = b.job[j];
    const MatView &w = J.w;
    CHECK(b.starts.first[j] == next && J.block_begin == next, "job %d starts at %d", j, next);
    CHECK(J.R >= 1 && J.R <= GF_MAX_R, "R %d", J.R);
    CHECK(gemv_fused_smem_bytes(w.k, w.units, w.bd, J.R) <= smem, "job %d LDS", j);
    const int nb = (w.n_tiles + J.R - 1) / J.R;
    for (int blk = 0; blk < nb; ++blk) {
      const int rt0 = blk * J.R, Reff = w.n_tiles - rt0 < J.R ? w.n_tiles - rt0 : J.R;
      CHECK(Reff >= 1, "empty block %d of job %d", blk, j);
      const int n_items = Reff * w.units;
      const size_t codes0 = w.off_codes + (size_t)rt0 * w.units * UNIT_BYTES;
      for (int wv = 0; wv < 4; ++wv) {
        const int b0 = gf_wave_begin(n_items, 4, wv), e0 = gf_wave_begin(n_items, 4, wv + 1);
        CHECK(b0 <= e0 && e0 <= n_items, "wave range");
        // the kernel loads units begin .. end + GV_PIPE - 1 (2 in flight)
        for (int u = b0; u < e0 + 2; ++u) {
          const int lu = gf_load_unit(u, e0);
          if (lu >= 0) check::check_code_load(w, codes0 + (size_t)lu * UNIT_BYTES, "fused");
        }
      }
    }
    next += nb;
  }
  CHECK(next == blocks, "blocks %d planned %d", blocks, next);
  return hipSuccess;
}

hipError_t launch_gemv_batched(GemvBatch &b, int gather_blocks, int k_max, int blocks, size_t smem,
                               hipStream_t) {
  ++check::launches;
  CHECK(smem <= GV_LDS_LIMIT, "main LDS %zu", smem);
  CHECK((size_t)k_max * 2 <= GV_LDS_LIMIT, "gather LDS");
  CHECK(b.m >= 1 && b.m <= EXACT_MAX_M, "m %d", b.m);  // m = 1 when the fused LDS does not fit
  CHECK(gather_blocks >= b.touch_begin + 8 * b.count, "gather blocks");
  int next = 0, gnext = 0;
  for (int j = 0; j < b.count; ++j) {
    const GemvJob &J = b.job[j];
    const MatView &w = J.w;
    check::check_ws(J.xg, (size_t)b.m * w.units * GV_XG_UNIT_BYTES, "gathered activations");
    check::check_ws(J.xs, (size_t)w.units * 16, "unit scales");
    CHECK(b.gather_starts.first[j] == gnext, "gather start");
    gnext += b.m * ((w.units + 3) / 4);
    CHECK(b.starts.first[j] == next, "main start");
    const int nb = (w.n_tiles + J.R - 1) / J.R;
    for (int blk = 0; blk < nb; ++blk) {
      const int t0 = blk * J.R, Reff = w.n_tiles - t0 < J.R ? w.n_tiles - t0 : J.R;
      CHECK(Reff >= 1 && Reff <= GV_MAX_R, "Reff %d", Reff);
      const int F = Reff * w.units;
      const size_t codes = w.off_codes + (size_t)t0 * w.units * UNIT_BYTES;
      for (int wv = 0; wv < 4; ++wv) {
        const int n_items = gv_wave_items(F, wv);
        // prologue loads items 0, 1; the main loop refills item k + 2 after
        // item k, for every k it processes before its last two
        for (int k = 0; k < n_items + 2; ++k)
          check::check_code_load(w, codes + (size_t)gv_load_flat(wv + 4 * k, F) * UNIT_BYTES, "m2-4");
      }
    }
    next += nb;
  }
  CHECK(next == blocks && gnext <= b.touch_begin, "blocks");
  return hipSuccess;
}

// ---- small batch (m = 5..16) ----------------------------------------------
hipError_t launch_sb(SbBatch &b, int prep_blocks, int blocks, hipStream_t) {
  ++check::launches;
  CHECK(b.m > EXACT_MAX_M && b.m <= SB_MAX_M, "m %d", b.m);
  int next = 0, pnext = 0;
  for (int j = 0; j < b.count; ++j) {
    const SbJob &J = b.job[j];
    const MatView &w = J.w;
    CHECK(J.tiles >= 1 && J.tiles <= SB_TMAX, "tiles %d", J.tiles);
    CHECK(J.groups * J.tiles >= w.n_tiles && (J.groups - 1) * J.tiles < w.n_tiles, "groups");
    CHECK(J.splits * J.upr >= w.units && (J.splits - 1) * J.upr < w.units, "splits");
    CHECK(b.starts.first[j] == next && J.block_begin == next, "start");
    CHECK(b.prep_starts.first[j] == pnext && J.prep_begin == pnext, "prep start");
    check::check_ws(J.xa, (size_t)w.units * SB_XA_UNIT_BYTES, "fragments");
    check::check_ws(J.xs, (size_t)w.units * 16 * 4, "activation scales");
    CHECK(J.xinv > 0.f, "split scale %g", (double)J.xinv);
    if (J.splits > 1) {
      check::check_ws(J.part, (size_t)J.groups * J.tiles * J.splits * 1024, "partial tiles");
      check::check_ws(J.cnt, (size_t)J.groups * 4, "arrival counters");
    }
    for (int g = 0; g < J.groups; ++g)
      for (int r = 0; r < J.splits; ++r) {
        const int t0 = g * J.tiles, tn = w.n_tiles - t0 < J.tiles ? w.n_tiles - t0 : J.tiles;
        const int u0 = r * J.upr, ul = w.units - u0 < J.upr ? w.units - u0 : J.upr;
        CHECK(tn >= 1 && ul >= 1, "empty block");
        const int N = ul * tn;
        for (int wv = 0; wv < SB_WAVES; ++wv) {
          const int i0 = wv * N / SB_WAVES, nk = (wv + 1) * N / SB_WAVES - i0;
          CHECK(nk <= SB_NMAX, "wave of %d items (at most %d)", nk, SB_NMAX);
          for (int k = 0; k < (nk > 2 ? nk : 2); ++k) {
            const int i = i0 + k < N - 1 ? i0 + k : N - 1, u = i / tn, t = i - u * tn;
            check::check_code_load(w, w.off_codes + ((size_t)(t0 + t) * w.units + u0 + u) * UNIT_BYTES, "sb");
          }
        }
      }
    next += J.groups * J.splits;
    pnext += w.units;
  }
  CHECK(next == blocks && pnext == prep_blocks, "blocks");
  return hipSuccess;
}

// ---- dequant-GEMM (m > 16) -------------------------------------------------
static PrefillBatch last_prefill;
hipError_t launch_prefill_prep(PrefillBatch &b, int blocks, size_t lds, bool, hipStream_t) {
  ++check::launches;
  CHECK(lds <= GV_LDS_LIMIT, "prep LDS %zu", lds);
  int pnext = 0;
  for (int j = 0; j < b.count; ++j) {
    const PrefillJob &J = b.job[j];
    CHECK(J.prep_begin == pnext && b.prep_starts.first[j] == pnext, "prep start");
    CHECK(J.m_pad % J.prep_rpb == 0 && J.m_pad >= J.m, "prep rows");
    CHECK(prefill_prep_lds(J.prep_rpb, J.w.k) <= lds, "prep LDS of job %d", j);
    check::check_ws(J.xb, (size_t)J.m_pad * J.w.units * UNIT_SLOTS * 2, "fragment copy");
    pnext += (J.m_pad / J.prep_rpb) * J.prep_csplit;
  }
  CHECK(pnext == blocks, "prep blocks");
  last_prefill = b;
  return hipSuccess;
}
hipError_t launch_prefill_batched(PrefillBatch &b, int bm, int blocks, hipStream_t) {
  ++check::launches;
  int next = 0;
  for (int j = 0; j < b.count; ++j) {
    const PrefillJob &J = b.job[j];
    const MatView &w = J.w;
    CHECK(J.block_begin == next && b.gemm_starts.first[j] == next, "gemm start");
    CHECK(J.tiles_m * bm == J.m_pad && J.tiles_n * 16 * 16 >= w.n_tiles * 16, "tiles");
    CHECK(J.splits >= 1 && J.splits * J.units_per_split >= w.units &&
          (J.splits - 1) * J.units_per_split < w.units, "splits");
    if (J.splits > 1) check::check_ws(J.part, (size_t)J.splits * J.m_pad * J.n_pad * 4, "partials");
    for (int nt = 0; nt < J.tiles_n; ++nt)
      for (int sp = 0; sp < J.splits; ++sp) {
        const int u0 = sp * J.units_per_split;
        const int u1 = u0 + J.units_per_split < w.units ? u0 + J.units_per_split : w.units;
        const int rt_lo = nt * 16, rt_hi = (nt + 1) * 16 < w.n_tiles ? (nt + 1) * 16 : w.n_tiles;
        if (rt_lo >= w.n_tiles) continue;  // a tile of padding rows only
        for (int rt = rt_lo; rt < rt_hi; ++rt)
          for (int u = u0; u < u1; ++u)
            check::check_code_load(w, w.off_codes + ((size_t)rt * w.units + u) * UNIT_BYTES, "gemm");
      }
    next += (J.tiles_n * J.tiles_m * J.splits + 7) / 8 * 8;
  }
  CHECK(next == blocks, "gemm blocks");
  return hipSuccess;
}
hipError_t launch_prefill_reduce(PrefillBatch &b, int blocks, hipStream_t) {
  ++check::launches;
  int next = 0;
  for (int j = 0; j < b.count; ++j) {
    CHECK(b.job[j].red_begin == next, "reduce start");
    if (b.job[j].splits > 1) next += b.job[j].m * ((b.job[j].w.n + 1023) / 1024);
  }
  CHECK(next == blocks, "reduce blocks");
  return hipSuccess;
}

// ---- calls the harness does not drive ---------------------------------------
hipError_t launch_moe(const svq_handle *const *, int32_t, int32_t, const void *const *,
                      const int64_t *, int32_t, const int32_t *, int64_t, int32_t, void *const *,
                      const int64_t *, int, void *, size_t, hipStream_t, size_t *need) {
  *need = 256;
  return hipSuccess;
}
hipError_t launch_encode(const EncArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_esg(const EsgArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_abs_rows(const double *, int32_t, int32_t, double *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_abs_totals(const double *, int32_t, int32_t, double *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t scratch_ptr(void **p) {
  *p = nullptr;
  return hipErrorNotSupported;
}

}  // namespace svq
