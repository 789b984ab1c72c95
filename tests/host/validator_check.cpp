// Host-only exercise of the C ABI's argument checks and workspace planning,
// built with AddressSanitizer and UndefinedBehaviorSanitizer around the
// library's host code (api.cpp).  Every call made here is either a size
// query or a call with a defect that the host side must refuse before any
// HIP call, so no GPU is needed.  Exit status 0: every refusal carried the
// expected status and a message; the sanitizers abort the run on the first
// error they find.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "wq.h"

namespace {

int failures = 0;

void expect(bool ok, const char *what, long long a, long long b) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (%lld, %lld): %s\n", what, a, b, wq_last_error());
    ++failures;
  }
}

// pointers that are never dereferenced on the host (device addresses in a
// real call); 16-byte aligned, or deliberately not
void *const P16 = reinterpret_cast<void *>(uintptr_t(1) << 20);
void *const P8 = reinterpret_cast<void *>((uintptr_t(1) << 20) + 8);

wq_weight weight(int bits, int64_t n, int64_t k) {
  wq_weight w;
  std::memset(&w, 0, sizeof w);
  w.bits = bits;
  w.group = 128;
  w.n = n;
  w.k = k;
  w.codes = static_cast<const uint32_t *>(P16);
  w.scales = static_cast<const uint16_t *>(P16);
  w.zeros = static_cast<const uint16_t *>(P16);
  return w;
}

}  // namespace

int main() {
  const int bits_list[] = {3, 4, 6, 8, 0, 5, -1, 1 << 30};
  const int64_t ns[] = {-1, 0, 1, 63, 64, 4096, 151936, (int64_t)1 << 20, INT32_MAX, (int64_t)INT32_MAX + 1,
                        INT64_MAX};
  const int64_t ks[] = {-128, 0, 100, 128, 1152, 9728, 65536, (int64_t)1 << 30, (int64_t)INT32_MAX - 127,
                        (int64_t)1 << 40, INT64_MAX - 127};
  const int64_t ms[] = {INT64_MIN, -1, 0, 1, 2, 5, 13, 16, 17, 33, 64, 65, 512, 4096, (int64_t)1 << 20,
                        (int64_t)INT32_MAX + 1, INT64_MAX};

  // 1. workspace queries over every combination, with and without rotation,
  //    alone and as groups of up to WQ_MAX_BATCH: any answer, no UB
  size_t sink = 0;
  for (int bits : bits_list)
    for (int64_t n : ns)
      for (int64_t k : ks)
        for (int rht = 0; rht < 2; ++rht) {
          wq_weight w = weight(bits, n, k);
          if (bits == 0) {
            w.block_bits = static_cast<const uint8_t *>(P16);
            w.block_off = static_cast<const uint64_t *>(P16);
          }
          if (rht) {
            w.rht_signs = static_cast<const uint32_t *>(P16);
            w.rht_block = 128;
          }
          std::vector<wq_weight> g(WQ_MAX_BATCH, w);
          for (int64_t m : ms) {
            sink += wq_linear_workspace(&w, m);
            for (int c : {1, 2, WQ_MAX_BATCH}) sink += wq_linear_batch_workspace(c, g.data(), m);
          }
          expect(wq_linear_batch_workspace(0, g.data(), 4) == (size_t)-1, "batch workspace count 0", n, k);
          expect(wq_linear_batch_workspace(WQ_MAX_BATCH + 1, g.data(), 4) == (size_t)-1,
                 "batch workspace count > max", n, k);
        }
  expect(wq_linear_workspace(nullptr, 4) == (size_t)-1, "workspace of NULL weight", 0, 0);

  // 2. packed word counts, host block widths included
  for (int bits : bits_list)
    for (int64_t n : ns)
      for (int64_t k : ks) sink += wq_packed_words(bits, n, k, nullptr);
  {
    std::vector<uint8_t> sel(1 << 12);
    for (size_t i = 0; i < sel.size(); ++i) sel[i] = (i % 3) ? 6 : 8;
    for (int64_t k : ks) sink += wq_packed_words(0, 64 * (int64_t)sel.size(), k, sel.data());
    sel[7] = 7;
    expect(wq_packed_words(0, 64 * 8, 128, sel.data()) == 0, "packed words, bad block width", 7, 0);
    expect(wq_packed_words(0, 64 * 8, 128, nullptr) == 0, "packed words, no block widths", 0, 0);
  }

  // 3. calls with one defect each: refused with their status, and a message
  const uint16_t *x = static_cast<const uint16_t *>(P16);
  struct Case {
    const char *what;
    wq_weight w;
    int64_t m, ldx, ldy;
    const void *xp;
    wq_dtype dt;
    uint32_t flags;
    wq_status want;
  };
  std::vector<Case> cases;
  for (int bits : {3, 4, 6, 8}) {
    for (int64_t k : {128, 9728}) {
      const int64_t n = 256;
      auto base = [&] { return Case{"", weight(bits, n, k), 4, k, n, x, WQ_F16, 0, WQ_OK}; };
      Case c = base(); c.what = "bits 5"; c.w.bits = 5; c.want = WQ_E_UNSUPPORTED; cases.push_back(c);
      c = base(); c.what = "group 64"; c.w.group = 64; c.want = WQ_E_UNSUPPORTED; cases.push_back(c);
      c = base(); c.what = "k % 128"; c.w.k = k + 64; c.ldx = k + 64; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "n 0"; c.w.n = 0; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "n > 2^31"; c.w.n = (int64_t)INT32_MAX + 1; c.ldy = c.w.n; c.want = WQ_E_UNSUPPORTED;
      cases.push_back(c);
      c = base(); c.what = "codes NULL"; c.w.codes = nullptr; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "zeros misaligned"; c.w.zeros = static_cast<const uint16_t *>(P8);
      c.want = WQ_E_ALIGN; cases.push_back(c);
      c = base(); c.what = "mixed n"; c.w.bits = 0; c.w.n = 96; c.ldy = 96; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "mixed tables"; c.w.bits = 0; c.want = WQ_E_ARG; cases.push_back(c);
      // the optional host copy of the widths (n / 64 = 4 bytes, read on the host)
      static const uint8_t bad_widths[4] = {6, 8, 6, 5};
      c = base(); c.what = "mixed host widths"; c.w.bits = 0; c.w.block_bits = static_cast<const uint8_t *>(P16);
      c.w.block_off = static_cast<const uint64_t *>(P16); c.w.block_bits_host = bad_widths; c.want = WQ_E_ARG;
      cases.push_back(c);
      c = base(); c.what = "rht block"; c.w.rht_signs = static_cast<const uint32_t *>(P16); c.w.rht_block = 64;
      c.want = WQ_E_UNSUPPORTED; cases.push_back(c);
      for (int64_t m : {INT64_MIN, (int64_t)-1, (int64_t)0}) {
        c = base(); c.what = "m <= 0"; c.m = m; c.want = WQ_E_ARG; cases.push_back(c);
      }
      c = base(); c.what = "x NULL"; c.xp = nullptr; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "x misaligned"; c.xp = P8; c.want = WQ_E_ALIGN; cases.push_back(c);
      c = base(); c.what = "ldx short"; c.ldx = k - 8; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "ldx not a multiple of 8"; c.ldx = k + 4; c.want = WQ_E_ALIGN; cases.push_back(c);
      c = base(); c.what = "ldy short"; c.ldy = n - 1; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "y dtype"; c.dt = (wq_dtype)9; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "flags"; c.flags = 6; c.want = WQ_E_ARG; cases.push_back(c);
      c = base(); c.what = "workspace too small"; c.m = 64; c.w.rht_signs = static_cast<const uint32_t *>(P16);
      c.w.rht_block = 128; c.flags = WQ_FUSE_RHT; c.want = WQ_E_WORKSPACE; cases.push_back(c);
    }
  }
  for (const Case &c : cases) {
    const size_t ws = std::strcmp(c.what, "workspace too small") == 0 ? 256 : ((size_t)1 << 40);
    wq_status st = wq_linear(&c.w, static_cast<const uint16_t *>(c.xp), c.m, c.ldx, P16, c.dt, c.ldy, c.flags,
                             P16, ws, nullptr);
    expect(st == c.want, c.what, st, c.want);
    expect(wq_last_error()[0] != 0, "message", st, 0);
    // the same defect in a group of two (the second member carries it)
    wq_weight pair[2] = {weight(c.w.bits == 0 ? 4 : c.w.bits, c.w.n > 0 ? c.w.n : 64, c.w.k), c.w};
    pair[0].group = 128;
    const uint16_t *xs[2] = {static_cast<const uint16_t *>(c.xp), static_cast<const uint16_t *>(c.xp)};
    const int64_t ldxs[2] = {c.ldx, c.ldx}, ldys[2] = {c.ldy, c.ldy};
    void *ys[2] = {P16, P16};
    const wq_dtype dts[2] = {c.dt, c.dt};
    st = wq_linear_batch(2, pair, xs, ldxs, c.m, ys, dts, ldys, c.flags, P16, ws, nullptr);
    expect(st != WQ_OK, c.what, st, 0);
    st = wq_linear_batch_noalloc(2, pair, xs, ldxs, c.m, ys, dts, ldys, c.flags, nullptr);
    expect(st != WQ_OK, c.what, st, 0);
  }

  // 4. the other entry points' refusals
  expect(rht_apply(x, (uint16_t *)P16, (const uint32_t *)P16, 1, 256, 256, 256, 64, nullptr) == WQ_E_UNSUPPORTED,
         "rht block", 0, 0);
  expect(rht_apply(x, (uint16_t *)P16, (const uint32_t *)P16, 1, 100, 256, 256, 128, nullptr) == WQ_E_ARG,
         "rht k", 0, 0);
  expect(rht_apply(nullptr, (uint16_t *)P16, (const uint32_t *)P16, 1, 256, 256, 256, 128, nullptr) == WQ_E_ARG,
         "rht NULL", 0, 0);
  expect(wq_pack(7, 4, 128, (const uint8_t *)P16, nullptr, (uint32_t *)P16, nullptr, nullptr) ==
             WQ_E_UNSUPPORTED, "pack bits", 0, 0);
  expect(wq_pack(0, 64, 128, (const uint8_t *)P16, nullptr, (uint32_t *)P16, nullptr, nullptr) == WQ_E_ARG,
         "pack mixed without tables", 0, 0);
  expect(wq_unpack(4, 4, 128, nullptr, nullptr, nullptr, (uint8_t *)P16, nullptr) == WQ_E_ARG, "unpack NULL", 0, 0);
  expect(wq_quantize(4, 4, 100, (const float *)P16, nullptr, nullptr, (uint8_t *)P16, (uint16_t *)P16,
                     (uint16_t *)P16, nullptr) == WQ_E_ARG, "quantize k", 0, 0);
  {
    wq_weight t = weight(8, 1000, 256);
    expect(wq_embed(&t, nullptr, 4, P16, WQ_F16, 256, nullptr) == WQ_E_ARG, "embed ids NULL", 0, 0);
    expect(wq_embed(&t, (const int32_t *)P16, -1, P16, WQ_F16, 256, nullptr) == WQ_E_ARG, "embed count", 0, 0);
    expect(wq_embed(&t, (const int32_t *)P16, 4, P16, WQ_F16, 100, nullptr) == WQ_E_ARG, "embed ldo", 0, 0);
    t.bits = 0;
    expect(wq_embed(&t, (const int32_t *)P16, 4, P16, WQ_F16, 256, nullptr) != WQ_OK, "embed mixed", 0, 0);
  }
  std::printf("checked %zu defect cases; size sink %zu\n", cases.size(), sink);
  return failures ? 1 : 0;
}
