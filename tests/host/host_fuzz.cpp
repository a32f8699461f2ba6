// Randomised driver for the library's host C++ (the KV pool manager and the
// decode planner), built with AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py.  Every call takes arguments drawn at random,
// valid and not: documents reused with other lengths, rows too short,
// corrupted table words, sequence lengths outside the table, plan buffers
// too small.  The sanitizers report any access outside an object; the
// driver checks the documented promises on top (no table word past
// max_blocks, untouched outputs on failure, plans within plan_ints).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "lazyattn.h"
#include "lazyattn_cache.h"

namespace {

constexpr uint32_t kPoison = 0xdeadbeefu;

int fail(const char *what, int it) {
  std::printf("FAIL at iteration %d: %s\n", it, what);
  return 1;
}

}  // namespace

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200;
  const unsigned seed = argc > 2 ? (unsigned)std::atoi(argv[2]) : 12345u;
  std::mt19937 rng(seed);
  auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long long calls = 0;
  for (int it = 0; it < iters; ++it) {
    // ---- pool manager: random acquire / release on a random pool
    lazyattn_cache *c = lazyattn_cache_create(U(1, 3000), U(0, 2));
    if (!c) return fail("create", it);
    std::vector<int32_t> live;
    for (int op = 0; op < 400; ++op, ++calls) {
      if (!live.empty() && U(0, 2) == 0) {
        const int k = U(0, (int)live.size() - 1);
        if (lazyattn_cache_release(c, live[(size_t)k]) != LAZYATTN_CACHE_OK) return fail("release", it);
        live.erase(live.begin() + k);
        continue;
      }
      const int nd = U(0, 6);
      std::vector<int32_t> ids((size_t)nd + 1), lens((size_t)nd + 1);
      for (int i = 0; i < nd; ++i) {
        ids[(size_t)i] = U(0, 40);
        lens[(size_t)i] = 16 * U(1, 60);  // a document id comes back with other lengths
      }
      if (nd && U(0, 20) == 0) lens[0] = U(-5, 15);  // not a positive multiple of 16
      const int prompt = U(0, 500), maxb = U(0, 300);
      std::vector<uint32_t> row((size_t)maxb + 1, kPoison);
      std::vector<uint8_t> miss((size_t)nd + 1, 7);
      int32_t rid = -1;
      const int r = lazyattn_cache_acquire(c, ids.data(), lens.data(), nd, prompt, row.data(), maxb, miss.data(),
                                           &rid);
      if (row[(size_t)maxb] != kPoison) return fail("table word written past max_blocks", it);
      if (r >= 0) {
        if (r > maxb) return fail("more words than max_blocks", it);
        live.push_back(rid);
      } else {
        for (int i = 0; i <= maxb; ++i)
          if (row[(size_t)i] != kPoison) return fail("row written by a failed request", it);
        for (int i = 0; i <= nd; ++i)
          if (miss[(size_t)i] != 7) return fail("miss flags written by a failed request", it);
      }
      int64_t st[10];
      lazyattn_cache_stats(c, st, 10);
    }
    if (lazyattn_cache_release(c, 1 << 30) != LAZYATTN_CACHE_ERR_ARG) return fail("unknown request", it);
    lazyattn_cache_destroy(c);

    // ---- decode planner: tables of shared documents, some words corrupted
    const int batch = U(1, 12), maxb = U(1, 200), hkv = U(1, 8), g = 1 << U(0, 4);
    std::vector<uint32_t> table((size_t)batch * maxb);
    std::vector<int32_t> lens((size_t)batch);
    const int ndocs = U(1, 10);
    std::vector<int> dstart((size_t)ndocs), dlen((size_t)ndocs), doff((size_t)ndocs);
    for (int d = 0; d < ndocs; ++d) {
      dstart[(size_t)d] = U(0, 60000);
      dlen[(size_t)d] = U(1, 40);
      doff[(size_t)d] = U(0, 60000);
    }
    for (int b = 0; b < batch; ++b) {
      for (int j = 0; j < maxb;) {
        const size_t d = (size_t)U(0, ndocs - 1);
        for (int k = 0; k < dlen[d] && j < maxb; ++k, ++j)
          table[(size_t)b * maxb + j] = (uint32_t)((dstart[d] + k) & 0xffff) | ((uint32_t)(doff[d] & 0xffff) << 16);
      }
      lens[(size_t)b] = U(-3, maxb * 16 + 20);  // outside [0, 16 max_blocks] now and then
      if (U(0, 10) == 0) table[(size_t)b * maxb + U(0, maxb - 1)] = (uint32_t)rng();
    }
    size_t nints = lazyattn_decode_plan_ints(batch, maxb, hkv);
    if (U(0, 5) == 0) nints = (size_t)U(0, (int)nints);  // too small
    std::vector<int32_t> plan(nints + 1, (int32_t)kPoison);
    int items = -1, mx = -1;
    lazyattn_decode_plan(table.data(), lens.data(), batch, maxb, hkv * g, hkv, U(0, 3) ? 0 : U(1, 300), plan.data(),
                         nints, &items, &mx);
    if (plan[nints] != (int32_t)kPoison) return fail("plan written past plan_ints", it);
    ++calls;
  }
  std::printf("ok: %lld calls\n", calls);
  return 0;
}
