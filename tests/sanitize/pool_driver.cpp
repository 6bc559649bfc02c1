// Host driver for the block pool with the prefix-cache index (pkv_pool_* in
// include/pkv.h), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_sanitizers.py.  It runs seeded random requests (admit, cache,
// fork, free) against the pool, checks the pool's counters after every step
// against a shadow count kept here, exercises the argument errors, and
// destroys the pool: any out-of-bounds access, leak or undefined behaviour
// ends the run with a sanitizer report.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

namespace {

struct Request {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
};

}  // namespace

int main() {
  const int32_t kBlocks = 96, kB = 16;
  pkv_block_pool* p = pkv_pool_create(kBlocks, kB);
  CHECK(p != nullptr);
  CHECK(pkv_pool_create(0, 16) == nullptr && pkv_pool_create(4, 0) == nullptr);
  std::mt19937 rng(7);
  std::vector<int32_t> refs(kBlocks, 0);   // shadow reference counts
  std::vector<Request> live;
  const std::vector<int32_t> prompts[3] = {std::vector<int32_t>(37 * kB / 2, 5), std::vector<int32_t>(5 * kB, 9),
                                           std::vector<int32_t>(3 * kB + 3, 2)};
  for (int step = 0; step < 4000; ++step) {
    const int op = (int)(rng() % 4);
    if (op <= 1 || live.empty()) {   // admit a request: a shared prompt plus its own tokens
      Request r;
      r.tokens = prompts[rng() % 3];
      const int extra = 1 + (int)(rng() % (3 * kB));
      for (int i = 0; i < extra; ++i) r.tokens.push_back((int32_t)(rng() % 50));
      const int32_t n = (int32_t)r.tokens.size();
      std::vector<int32_t> hit(n / kB + 1);
      const int32_t h = pkv_pool_match_prefix(p, r.tokens.data(), n, 3, hit.data(), (int32_t)hit.size());
      CHECK(h >= 0 && h <= (n - 1) / kB);
      const int32_t need = (n + kB - 1) / kB - h;
      std::vector<int32_t> fresh(need > 0 ? need : 1);
      const int32_t got = pkv_pool_allocate(p, need, fresh.data());
      if (got == PKV_ENOSPACE) {   // no room: give the hits back
        CHECK(pkv_pool_free(p, hit.data(), h) == PKV_OK);
        continue;
      }
      CHECK(got == need);
      for (int32_t j = 0; j < h; ++j) r.blocks.push_back(hit[j]);
      for (int32_t j = 0; j < need; ++j) r.blocks.push_back(fresh[j]);
      for (int32_t b : r.blocks) ++refs[b];
      CHECK(pkv_pool_cache_blocks(p, r.tokens.data(), n, 3, r.blocks.data(), (int32_t)r.blocks.size()) >= 0);
      live.push_back(r);
    } else if (op == 2) {          // fork a live request
      Request r = live[rng() % live.size()];
      CHECK(pkv_pool_ref(p, r.blocks.data(), (int32_t)r.blocks.size()) == PKV_OK);
      for (int32_t b : r.blocks) ++refs[b];
      live.push_back(r);
    } else {                       // a request finishes
      const size_t i = rng() % live.size();
      CHECK(pkv_pool_free(p, live[i].blocks.data(), (int32_t)live[i].blocks.size()) == PKV_OK);
      for (int32_t b : live[i].blocks) --refs[b];
      live.erase(live.begin() + (long)i);
    }
    int32_t referenced = 0;
    for (int32_t b = 0; b < kBlocks; ++b) {
      CHECK(pkv_pool_ref_count(p, b) == refs[b]);
      referenced += refs[b] > 0;
    }
    CHECK(pkv_pool_num_free(p) + referenced == kBlocks);
    CHECK(pkv_pool_num_cached(p) >= 0 && pkv_pool_num_cached(p) <= kBlocks);
  }
  // argument errors change nothing
  int32_t out[4];
  uint8_t hashes[64];
  const int32_t bad_block = kBlocks;
  CHECK(pkv_pool_match_prefix(nullptr, prompts[0].data(), 4, 0, out, 4) == PKV_EINVAL);
  CHECK(pkv_pool_match_prefix(p, nullptr, 4, 0, out, 4) == PKV_EINVAL);
  CHECK(pkv_pool_allocate(p, -1, out) == PKV_EINVAL);
  CHECK(pkv_pool_allocate(p, kBlocks + 1, out) == PKV_ENOSPACE);
  CHECK(pkv_pool_free(p, &bad_block, 1) == PKV_EINVAL);
  CHECK(pkv_pool_ref(p, &bad_block, 1) == PKV_EINVAL);
  CHECK(pkv_pool_cache_blocks(p, prompts[1].data(), 16, 0, &bad_block, 1) == PKV_EINVAL);
  CHECK(pkv_pool_block_hash(p, prompts[1].data(), 32, 0, hashes, 2) == 2);
  CHECK(pkv_pool_block_hash(p, prompts[1].data(), 32, 0, nullptr, 2) == PKV_EINVAL);
  CHECK(pkv_pool_ref_count(p, -1) == PKV_EINVAL);
  for (const Request& r : live) CHECK(pkv_pool_free(p, r.blocks.data(), (int32_t)r.blocks.size()) == PKV_OK);
  CHECK(pkv_pool_num_free(p) == kBlocks);
  pkv_pool_destroy(p);
  std::printf("pool driver: ok\n");
  return 0;
}
