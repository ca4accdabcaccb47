// Host-only exercise of mf_plan and the prefix cache's index under
// AddressSanitizer and UndefinedBehaviorSanitizer (no device calls): random
// and malformed batches through mf_plan; inserts of entries without kept
// blocks (which copy nothing), lookups, pins, releases and LRU evictions
// through the cache, checked against a plain model of the same rules.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <random>
#include <vector>

#include "mapflow.h"

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void plan_cases(std::mt19937& rng) {
  mf_plan_info info;
  // malformed inputs are rejected
  CHECK(mf_plan(nullptr, nullptr, nullptr, 1, 64, nullptr, 0, &info) == MF_ERR_INVALID);
  const int32_t cq[3] = {0, 100, 50}, ck[3] = {0, 100, 300};
  CHECK(mf_plan(cq, ck, nullptr, 2, 64, nullptr, 0, &info) == MF_ERR_INVALID);     // decreasing q
  const int32_t cq2[2] = {0, 100}, ck2[2] = {0, 90};
  CHECK(mf_plan(cq2, ck2, nullptr, 1, 64, nullptr, 0, &info) == MF_ERR_INVALID);   // keys short of queries
  const int32_t p0[1] = {32};
  const int32_t ck3[2] = {0, 200};
  CHECK(mf_plan(cq2, ck3, p0, 1, 64, nullptr, 0, &info) == MF_ERR_UNSUPPORTED);    // chunk off the grid
  CHECK(mf_plan(cq2, ck3, nullptr, 1, 48, nullptr, 0, &info) == MF_ERR_UNSUPPORTED);
  CHECK(mf_plan(cq2, ck3, nullptr, -1, 64, nullptr, 0, &info) == MF_ERR_INVALID);
  // random valid batches: sizing call, then the plan itself, against a model
  for (int it = 0; it < 2000; ++it) {
    const int B = 32 << (rng() % 3);
    const int S = rng() % 9;
    std::vector<int32_t> cu_q(S + 1, 0), cu_k(S + 1, 0), pos0(S, 0);
    std::vector<int64_t> nrb(S);
    for (int s = 0; s < S; ++s) {
      const int q = rng() % 700;
      const int p = (rng() % 4) * B;
      const int k = p + q + rng() % 50;
      pos0[s] = p;
      cu_q[s + 1] = cu_q[s] + q;
      cu_k[s + 1] = cu_k[s] + k;
      nrb[s] = (q + B - 1) / B;
    }
    const bool with_pos = rng() % 2;
    if (!with_pos)
      for (int s = 0; s < S; ++s) {   // without q_pos0 every chunk starts at 0
        const int q = cu_q[s + 1] - cu_q[s], k = cu_k[s + 1] - cu_k[s];
        if (k < q) { CHECK(false); }
      }
    const int32_t* pp = with_pos ? pos0.data() : nullptr;
    const mf_status sz = mf_plan(cu_q.data(), cu_k.data(), pp, S, B, nullptr, 0, &info);
    CHECK(sz == MF_ERR_CAPACITY || (sz == MF_OK && info.plan_len == 0));
    std::vector<int32_t> plan(info.plan_len > 0 ? info.plan_len : 1, -1);
    CHECK(mf_plan(cu_q.data(), cu_k.data(), pp, S, B, plan.data(), info.plan_len, &info) == MF_OK);
    int64_t tot = 0;
    for (int s = 0; s < S; ++s) tot += nrb[s];
    CHECK(info.total_rowblocks == tot);
    CHECK(info.plan_len == S + 1 + tot);
    int64_t at = 0;
    for (int s = 0; s < S; ++s) {
      CHECK(plan[s] == at);
      for (int64_t i = 0; i < nrb[s]; ++i) CHECK(plan[S + 1 + at + i] == s);
      at += nrb[s];
    }
    if (S > 0) CHECK(plan[S] == at);
  }
}

static void cache_cases(std::mt19937& rng) {
  // a host buffer stands in for the device pool: entries without kept
  // blocks copy nothing, so the pool is never read or written
  const size_t pool_bytes = 64 << 10;
  void* pool = aligned_alloc(256, pool_bytes);
  mf_map_cache_desc d = {MF_BF16, 2, 3, 64};
  mf_map_cache* c = nullptr;
  CHECK(mf_map_cache_create(&d, pool, pool_bytes, &c) == MF_OK);
  mf_map_cache_stats st;
  CHECK(mf_map_cache_get_stats(c, &st) == MF_OK);
  const int64_t cap = st.bytes_capacity;
  CHECK(mf_map_cache_create(&d, (char*)pool + 8, pool_bytes, &c) != MF_OK || c != nullptr);
  // chains of hashes: sequence t's block i hashes to a value unique to (t, i)
  const int maxb = 16;
  auto hashes = [&](int t) {
    std::vector<uint64_t> h(maxb);
    for (int i = 0; i < maxb; ++i) h[i] = 0x9e3779b97f4a7c15ull * (uint64_t)(t + 1) + (uint64_t)i;
    return h;
  };
  std::map<int, int> held;      // model: sequence -> blocks held
  std::map<int, int> pins;
  for (int it = 0; it < 3000; ++it) {
    const int t = rng() % 24;
    const std::vector<uint64_t> h = hashes(t);
    const int op = rng() % 4;
    if (op == 0) {
      const int n = 1 + rng() % maxb;
      const int L = d.num_layers, H = d.H_s, total_rb = maxb;
      std::vector<int32_t> rp((size_t)L * H * total_rb + 1, 0);   // no kept blocks
      const mf_status s = mf_map_cache_insert(c, h.data(), n, rp.data(), total_rb, 0, nullptr, nullptr, nullptr);
      CHECK(s == MF_OK || s == MF_ERR_CAPACITY);
      if (s == MF_OK && held[t] < n) held[t] = n;
    } else if (op == 1) {
      const int n = 1 + rng() % maxb;
      const int m = mf_map_cache_lookup(c, h.data(), n);
      CHECK(m >= 0 && m <= n);
      if (m > 0) pins[t * 100 + m] += 1;
    } else if (op == 2) {
      // release one pin taken earlier
      for (auto& kv : pins)
        if (kv.first / 100 == t && kv.second > 0) {
          mf_map_cache_release(c, h.data(), kv.first % 100);
          kv.second -= 1;
          break;
        }
    } else {
      CHECK(mf_map_cache_get_stats(c, &st) == MF_OK);
      CHECK(st.bytes_used >= 0 && st.bytes_used <= cap);
      CHECK(st.pinned_entries >= 0 && st.pinned_entries <= st.entries);
    }
  }
  // a lookup never claims more than was inserted for that chain
  for (auto& kv : held) {
    const std::vector<uint64_t> h = hashes(kv.first);
    const int m = mf_map_cache_lookup(c, h.data(), maxb);
    CHECK(m <= kv.second);
    if (m > 0) mf_map_cache_release(c, h.data(), m);
  }
  // bad arguments
  std::vector<int32_t> rp(2 * 3 * 4 + 1, 0);
  const std::vector<uint64_t> h = hashes(0);
  CHECK(mf_map_cache_insert(c, h.data(), 5, rp.data(), 4, 0, nullptr, nullptr, nullptr) == MF_ERR_INVALID);
  CHECK(mf_map_cache_insert(c, nullptr, 1, rp.data(), 4, 0, nullptr, nullptr, nullptr) == MF_ERR_INVALID);
  CHECK(mf_map_cache_lookup(c, h.data(), 0) == 0);
  mf_map_cache_destroy(c);
  free(pool);
}

int main() {
  std::mt19937 rng(12345);
  plan_cases(rng);
  cache_cases(rng);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host sanitizer driver: all checks passed\n");
  return 0;
}
