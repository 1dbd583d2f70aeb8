// Randomised stress of the host prefix cache's C ABI (control plane only),
// built by tests/test_host_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer. Checks the contract stated in mqa_int8.h:
// matches are whole blocks of a prefix, slots lie in the pool and are
// distinct along a chain, a chain just inserted matches in full, usage never
// exceeds capacity, and invalid arguments return error codes.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "../include/mqa_int8.h"

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                          \
    }                                                                        \
  } while (0)

static void run(int32_t bs, int64_t cap, int vocab, int events, uint32_t seed) {
  mqa_prefix_cache* c = nullptr;
  CHECK(mqa_prefix_cache_create(bs, cap, &c) == MQA_OK && c != nullptr);
  std::mt19937 g(seed);
  const int n_conv = 8;
  std::vector<std::vector<int32_t>> hist(n_conv);
  for (int e = 0; e < events; ++e) {
    auto& h = hist[g() % n_conv];
    if (g() % 5 == 0 && h.size() > 4) h.resize(g() % h.size());  // regenerate: keep part of it
    const int add = 1 + (int)(g() % (3 * bs + 5));
    for (int i = 0; i < add; ++i) h.push_back((int32_t)(g() % vocab));
    const int64_t n = (int64_t)h.size();
    const int64_t nb = n / bs;

    int64_t matched = -1;
    std::vector<int64_t> ms(nb + 1, -7);
    const bool with_slots = g() % 4 != 0;
    CHECK(mqa_prefix_cache_match(c, h.data(), n, &matched, with_slots ? ms.data() : nullptr) == MQA_OK);
    CHECK(matched >= 0 && matched <= n && matched % bs == 0);
    if (with_slots) {
      std::set<int64_t> seen;
      for (int64_t i = 0; i < matched / bs; ++i) {
        CHECK(ms[i] >= 0 && ms[i] < cap);
        CHECK(seen.insert(ms[i]).second);
      }
      CHECK(ms[nb] == -7);  // nothing written past n_tokens / block_size entries
    }

    std::vector<int64_t> is(nb + 1, -7);
    int64_t first = -1, nblk = -1;
    CHECK(mqa_prefix_cache_insert(c, h.data(), n, is.data(), &first, &nblk) == MQA_OK);
    CHECK(nblk >= 0 && nblk <= nb && first >= 0 && first <= nblk);
    CHECK(is[nb] == -7);
    {
      std::set<int64_t> seen;
      for (int64_t i = 0; i < nblk; ++i) {
        CHECK(is[i] >= 0 && is[i] < cap);
        CHECK(seen.insert(is[i]).second);
      }
    }
    // the chain just inserted is the most recently used: it matches in full
    int64_t again = -1;
    std::vector<int64_t> as(nb + 1, -7);
    CHECK(mqa_prefix_cache_match(c, h.data(), n, &again, as.data()) == MQA_OK);
    CHECK(again == nblk * bs);
    for (int64_t i = 0; i < nblk; ++i) CHECK(as[i] == is[i]);

    mqa_prefix_cache_stats st;
    CHECK(mqa_prefix_cache_get_stats(c, &st) == MQA_OK);
    CHECK(st.capacity_blocks == cap && st.used_blocks >= 0 && st.used_blocks <= cap);
    CHECK(st.matched_tokens <= st.lookup_tokens);
  }
  // empty and short inputs
  int64_t matched = -1, first = -1, nblk = -1;
  int64_t slot = -7;
  CHECK(mqa_prefix_cache_match(c, hist[0].data(), 0, &matched, &slot) == MQA_OK && matched == 0 && slot == -7);
  if (bs > 1) {
    CHECK(mqa_prefix_cache_insert(c, hist[0].data(), bs - 1, &slot, &first, &nblk) == MQA_OK);
    CHECK(nblk == 0 && first == 0 && slot == -7);
  }
  // invalid arguments
  CHECK(mqa_prefix_cache_match(nullptr, hist[0].data(), 1, &matched, nullptr) != MQA_OK);
  CHECK(mqa_prefix_cache_match(c, hist[0].data(), 1, nullptr, nullptr) != MQA_OK);
  CHECK(mqa_prefix_cache_insert(c, hist[0].data(), 1, nullptr, &first, &nblk) != MQA_OK);
  CHECK(mqa_prefix_cache_get_stats(c, nullptr) != MQA_OK);
  mqa_prefix_cache_destroy(c);
}

int main() {
  mqa_prefix_cache* c = nullptr;
  CHECK(mqa_prefix_cache_create(0, 4, &c) != MQA_OK);
  CHECK(mqa_prefix_cache_create(4, 0, &c) != MQA_OK);
  CHECK(mqa_prefix_cache_create(4, 4, nullptr) != MQA_OK);
  mqa_prefix_cache_destroy(nullptr);
  const struct { int32_t bs; int64_t cap; int vocab; } cases[] = {
      {1, 1, 3}, {1, 64, 4}, {4, 3, 2}, {4, 40, 50}, {8, 25, 5}, {16, 200, 50}, {16, 2, 2}, {32, 1000, 7}};
  uint32_t seed = 1;
  for (const auto& k : cases) run(k.bs, k.cap, k.vocab, 3000, seed++);
  std::printf("prefix cache stress ok\n");
  return 0;
}
