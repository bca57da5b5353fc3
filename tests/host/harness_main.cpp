// Drives libsvq's host code on the CPU (see launch_checks.cpp): packs random
// canonical matrices into buffers of exactly the reported size, then plans
// svq_linear / svq_linear_batched for many row counts, each call's workspace
// allocated at exactly the size its query returned.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_harness.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <vector>

#include "../../include/svq.h"

namespace check {
extern const uint8_t *ws_base;
extern size_t ws_bytes;
extern long launches, loads_checked;
}

struct Canon {
  int n, k, bd;
  std::vector<uint8_t> codes;
  std::vector<uint16_t> cb, rad;
  std::vector<int32_t> perm;
};

static Canon make(int n, int k, int bd, unsigned seed) {
  std::mt19937 g(seed);
  Canon c{n, k, bd, {}, {}, {}, {}};
  c.codes.resize(((size_t)n * (k / 8) * 18 + 7) / 8);
  for (auto &b : c.codes) b = (uint8_t)g();
  c.cb.resize((size_t)8 << bd);
  for (auto &v : c.cb) v = (uint16_t)(g() & 0x3BFF);  // finite, non-negative
  c.rad.resize((size_t)1 << (10 - bd));
  for (size_t r = 0; r < c.rad.size(); ++r) c.rad[r] = (uint16_t)(0x2000 + 0x100 * r);
  c.perm.resize(k);
  for (int p = 0; p < k; ++p) c.perm[p] = p;
  std::shuffle(c.perm.begin(), c.perm.end(), g);
  return c;
}

static svq_matrix_desc desc_of(const Canon &c) {
  return svq_matrix_desc{c.n, c.k, c.bd, 10 - c.bd, c.codes.data(), c.cb.data(), c.rad.data(), c.perm.data()};
}

static int fails = 0;
#define EXPECT(cond, ...)                                    \
  do {                                                       \
    if (!(cond)) {                                           \
      std::fprintf(stderr, "harness: %s: ", #cond);          \
      std::fprintf(stderr, __VA_ARGS__);                     \
      std::fprintf(stderr, "\n");                            \
      ++fails;                                               \
    }                                                        \
  } while (0)

struct Packed {
  std::vector<uint8_t> owner;  // unused: the buffer is malloc'd at its exact size
  uint8_t *buf = nullptr;
  svq_handle h{};
};

static Packed pack(const Canon &c) {
  Packed p;
  const svq_matrix_desc d = desc_of(c);
  size_t bytes = 0;
  EXPECT(svq_pack(&d, nullptr, &bytes, nullptr, nullptr) == SVQ_OK, "size query %dx%d", c.n, c.k);
  p.buf = (uint8_t *)std::malloc(bytes);
  size_t cap = bytes;
  EXPECT(svq_pack(&d, p.buf, &cap, &p.h, nullptr) == SVQ_OK, "pack %dx%d", c.n, c.k);
  EXPECT(p.h.bytes == bytes && p.h.off_codes + p.h.padded_code_bytes <= bytes, "layout");
  return p;
}

// One svq_linear_batched call over `mats` at m rows; the workspace is
// allocated at exactly the queried size.
static void plan(std::vector<Packed> &mats, int m) {
  const int cnt = (int)mats.size();
  std::vector<svq_handle> hs;
  std::vector<int64_t> ldx, ldy;
  std::vector<const void *> xs;
  std::vector<void *> ys;
  for (auto &p : mats) {
    hs.push_back(p.h);
    ldx.push_back(p.h.k + (m % 3) * 8);
    ldy.push_back(p.h.n);
    xs.push_back((const void *)0x1000);  // never dereferenced on the host
    ys.push_back((void *)0x2000);
  }
  size_t need = 0;
  svq_status st = svq_linear_batched(hs.data(), cnt, nullptr, ldx.data(), m, nullptr, ldy.data(),
                                     SVQ_BF16, nullptr, &need, nullptr);
  EXPECT(st == SVQ_OK, "query m=%d status %d", m, (int)st);
  uint8_t *ws = (uint8_t *)std::malloc(need ? need : 1);
  check::ws_base = ws;
  check::ws_bytes = need;
  size_t cap = need;
  st = svq_linear_batched(hs.data(), cnt, xs.data(), ldx.data(), m, ys.data(), ldy.data(), SVQ_F32, ws,
                          &cap, nullptr);
  EXPECT(st == SVQ_OK, "call m=%d count=%d status %d", m, cnt, (int)st);
  if (cnt == 1) {
    // the single-matrix entry point plans the same launches
    cap = need;
    st = svq_linear(&hs[0], xs[0], m, ldx[0], ys[0], ldy[0], SVQ_BF16, ws, &cap, nullptr);
    EXPECT(st == SVQ_OK, "svq_linear m=%d status %d", m, (int)st);
    // without a device array the allocation-free call reports the HIP
    // error, or UNSUPPORTED when the scratch would be too small
    st = svq_linear_noalloc(&hs[0], xs[0], m, ldx[0], ys[0], ldy[0], SVQ_BF16, nullptr);
    EXPECT(st == (need > SVQ_SCRATCH_BYTES ? SVQ_ERR_UNSUPPORTED : SVQ_ERR_HIP), "noalloc m=%d %d", m, (int)st);
  }
  // one byte short: rejected before any launch
  if (need > 256) {
    const long before = check::launches;
    cap = need - 1;
    st = svq_linear_batched(hs.data(), cnt, xs.data(), ldx.data(), m, ys.data(), ldy.data(), SVQ_F32, ws,
                            &cap, nullptr);
    EXPECT(st == SVQ_ERR_BUFFER_TOO_SMALL && check::launches == before, "short workspace m=%d", m);
  }
  std::free(ws);
  check::ws_base = nullptr;
}

int main() {
  const int ms[] = {1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 40, 64, 65, 129, 200, 255, 256, 257, 300, 511, 2048};
  // single matrices: the configurations' shapes and ragged edges
  const int shapes[][3] = {
      {512, 1024, 8}, {4096, 2560, 7}, {1024, 2560, 6}, {2560, 4096, 8}, {9728, 2560, 7},
      {2560, 9728, 8}, {768, 2048, 6}, {2048, 768, 7}, {1, 8, 8}, {37, 104, 6}, {16, 512, 7},
      {33, 1032, 8}, {100, 104, 7}, {17, 520, 6}, {15, 2048, 8}, {64, 4096, 6}, {20, 53248, 8},
      {40, 1000, 6}, {70, 1536, 7}, {260, 3000, 6}, {130, 4600, 7}, {50, 5600, 6}, {70, 9728, 8},
      {200, 1032, 8}, {129, 520, 6}, {300, 2560, 7}, {1000, 65536, 7}};
  unsigned seed = 1;
  for (auto &s : shapes) {
    std::vector<Packed> one{pack(make(s[0], s[1], s[2], seed++))};
    for (int m : ms) {
      if ((size_t)m * s[1] > ((size_t)1 << 26) && m > 16) continue;  // keep the host run short
      plan(one, m);
    }
    std::free(one[0].buf);
  }
  // the decoder layer in one call (and the first two, three ... matrices)
  const int layer[][3] = {{4096, 2560, 7}, {1024, 2560, 7}, {1024, 2560, 7}, {2560, 4096, 7},
                          {9728, 2560, 7}, {9728, 2560, 8}, {2560, 9728, 8}};
  std::vector<Packed> mats;
  for (auto &s : layer) mats.push_back(pack(make(s[0], s[1], s[2], seed++)));
  for (int cnt = 2; cnt <= 7; ++cnt) {
    std::vector<Packed> sub(mats.begin(), mats.begin() + cnt);
    for (int m : {1, 3, 4, 5, 16, 64, 2048}) plan(sub, m);
  }
  for (auto &p : mats) std::free(p.buf);
  // tables without an exact fp16 split: a radius of 60000 next to a
  // direction entry of 2^-24 spans more than the split can hold
  {
    Canon c2 = make(70, 1536, 7, 77);
    c2.rad[0] = 0x3C01;  // 1 + 2^-10
    c2.rad[1] = 0x7B53;  // 60000
    for (int l = 0; l < 8; ++l) c2.cb[l] = 0x0001;  // 2^-24
    std::vector<Packed> one{pack(c2)};
    EXPECT(one[0].h.xscale_log2 == SVQ_NO_EXACT_SPLIT, "expected no exact split");
    for (int m : {5, 8, 13, 16}) plan(one, m);
    std::free(one[0].buf);
  }
  // malformed canonical inputs are rejected before any copy
  Canon c = make(32, 64, 7, 99);
  c.perm[3] = c.perm[4];
  svq_matrix_desc d = desc_of(c);
  size_t bytes = 0;
  EXPECT(svq_pack(&d, nullptr, &bytes, nullptr, nullptr) == SVQ_ERR_INVALID_ARG, "duplicate perm");
  std::printf("host harness: %ld launches checked, %ld code loads, %d failures\n", check::launches,
              check::loads_checked, fails);
  return fails ? 1 : 0;
}
