// Host-side block pool with a prefix-cache index.
//
// What it implements (all host logic; no GPU work):
//  - Habr KV-Cache article (habr.com/ru/articles/1021832), section 7 "That
//    same Cache Read": each full block is identified by a hash that covers
//    every token from the start of the sequence; a flat table maps block
//    hash -> physical block; a request walks its blocks from block 0 and the
//    first miss ends the hit; hit blocks gain a reference; blocks nobody
//    references stay cached until memory runs short, then the least recently
//    used of them is evicted; cached blocks are never modified.  The worked
//    example: a 2000-token system prompt is 125 blocks; a second request with
//    the same prompt reuses all 125 and computes only its own 13.
//  - "Why one character breaks the cache", section on the git-style hash
//    chain: a block's hash is the hash of (parent block's hash, the block's
//    token ids, extra keys); the first block's parent is a fixed seed; the
//    hit is capped at num_tokens - 1 tokens so that the last token is always
//    computed; freed blocks join an LRU queue and a hit on a free block takes
//    it out of the queue.
//  - "Shared KV-cache across replicas without self-deception", section on
//    counting blocks: only whole matched blocks are useful,
//    floor(T / B) * B tokens of a T-token match.
//
// The hash is SHA-256 (FIPS 180-4), the default the gotacat page names.  A
// block's hashed message is: parent hash (32 bytes; all zeros for block 0),
// the extra key (8 bytes little-endian, e.g. a tenant salt), then the
// block's token ids as 4-byte little-endian integers.

#include "pkv.h"

#include <stdint.h>
#include <string.h>

#include <array>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// SHA-256, written from FIPS 180-4 sections 4.1.2, 4.2.2, 5.1.1, 6.2.
// ---------------------------------------------------------------------------
using Digest = std::array<uint8_t, 32>;

constexpr uint32_t kRoundK[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4, 0xab1c5ed5,
    0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174,
    0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
    0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967,
    0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85,
    0xa2bfe8a1, 0xa81a664b, 0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
    0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

class Sha256 {
 public:
  Sha256() : h_{0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a, 0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19} {}

  void update(const uint8_t* p, size_t n) {
    total_ += n;
    while (n > 0) {
      const size_t take = n < 64 - fill_ ? n : 64 - fill_;
      memcpy(buf_ + fill_, p, take);
      fill_ += take;
      p += take;
      n -= take;
      if (fill_ == 64) {
        block(buf_);
        fill_ = 0;
      }
    }
  }

  Digest finish() {
    const uint64_t bits = total_ * 8;
    // padding (FIPS 180-4 5.1.1): 0x80, zeros up to 56 mod 64, 64-bit length
    uint8_t pad[72] = {0x80};
    const size_t zeros = (fill_ < 56 ? 56 - fill_ : 120 - fill_) - 1;
    for (int i = 0; i < 8; ++i) pad[1 + zeros + i] = (uint8_t)(bits >> (56 - 8 * i));
    update(pad, 1 + zeros + 8);
    Digest d;
    for (int i = 0; i < 8; ++i)
      for (int b = 0; b < 4; ++b) d[4 * i + b] = (uint8_t)(h_[i] >> (24 - 8 * b));
    return d;
  }

 private:
  void block(const uint8_t* m) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t)m[4 * t] << 24 | (uint32_t)m[4 * t + 1] << 16 | (uint32_t)m[4 * t + 2] << 8 | m[4 * t + 3];
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6], h = h_[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = h + S1 + ch + kRoundK[t] + w[t];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + maj;
      h = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h_[0] += a;
    h_[1] += b;
    h_[2] += c;
    h_[3] += d;
    h_[4] += e;
    h_[5] += f;
    h_[6] += g;
    h_[7] += h;
  }

  uint32_t h_[8];
  uint8_t buf_[64] = {};
  size_t fill_ = 0;
  uint64_t total_ = 0;
};

// Hash of one full block: SHA-256(parent || extra key || token ids).
Digest block_hash(const Digest& parent, uint64_t extra_key, const int32_t* tokens, int block_size) {
  uint8_t stack_msg[40 + 4 * 64];
  std::vector<uint8_t> heap_msg;
  const size_t len = 40 + 4 * (size_t)block_size;
  uint8_t* msg = stack_msg;
  if (len > sizeof(stack_msg)) {
    heap_msg.resize(len);
    msg = heap_msg.data();
  }
  memcpy(msg, parent.data(), 32);
  for (int i = 0; i < 8; ++i) msg[32 + i] = (uint8_t)(extra_key >> (8 * i));
  for (int t = 0; t < block_size; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    uint8_t* o = msg + 40 + 4 * t;
    o[0] = (uint8_t)v;
    o[1] = (uint8_t)(v >> 8);
    o[2] = (uint8_t)(v >> 16);
    o[3] = (uint8_t)(v >> 24);
  }
  Sha256 s;
  s.update(msg, len);
  return s.finish();
}

struct DigestHash {
  size_t operator()(const Digest& d) const {
    size_t h;
    memcpy(&h, d.data(), sizeof(h));   // SHA-256 output bits are already uniform
    return h;
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// The pool: refcounts, an LRU queue of unreferenced blocks, and the index.
// ---------------------------------------------------------------------------
struct pkv_block_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;                       // references per block
  std::vector<uint8_t> cached;                    // block carries a hash in the index
  std::vector<Digest> hash;                       // its hash when cached
  std::list<int32_t> free_queue;                  // unreferenced blocks, least recently used first
  std::vector<std::list<int32_t>::iterator> pos;  // position in free_queue (valid when ref == 0)
  std::unordered_map<Digest, int32_t, DigestHash> index;
  int64_t evictions = 0;
};

namespace {

void take_from_free(pkv_block_pool* p, int32_t b) {
  p->free_queue.erase(p->pos[b]);
}

void evict(pkv_block_pool* p, int32_t b) {
  if (!p->cached[b]) return;
  auto it = p->index.find(p->hash[b]);
  if (it != p->index.end() && it->second == b) p->index.erase(it);
  p->cached[b] = 0;
  ++p->evictions;
}

bool valid_block(const pkv_block_pool* p, int32_t b) { return b >= 0 && b < p->num_blocks; }

// Chained hashes of the first `nblocks` full blocks of `tokens`.
void chain(const pkv_block_pool* p, const int32_t* tokens, int32_t nblocks, uint64_t extra_key,
           std::vector<Digest>* out) {
  out->resize(nblocks);
  Digest parent{};   // block 0's parent: the all-zero seed
  for (int32_t j = 0; j < nblocks; ++j) {
    (*out)[j] = block_hash(parent, extra_key, tokens + (size_t)j * p->block_size, p->block_size);
    parent = (*out)[j];
  }
}

}  // namespace

extern "C" {

pkv_block_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool();
  if (!p) return nullptr;
  try {
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->ref.assign(num_blocks, 0);
    p->cached.assign(num_blocks, 0);
    p->hash.assign(num_blocks, Digest{});
    p->pos.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) p->pos[b] = p->free_queue.insert(p->free_queue.end(), b);
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

int32_t pkv_pool_num_free(const pkv_block_pool* pool) {
  return pool ? (int32_t)pool->free_queue.size() : PKV_EINVAL;
}

int32_t pkv_pool_num_cached(const pkv_block_pool* pool) {
  return pool ? (int32_t)pool->index.size() : PKV_EINVAL;
}

int32_t pkv_pool_ref_count(const pkv_block_pool* pool, int32_t block) {
  if (!pool || !valid_block(pool, block)) return PKV_EINVAL;
  return pool->ref[block];
}

int64_t pkv_pool_evictions(const pkv_block_pool* pool) { return pool ? pool->evictions : PKV_EINVAL; }

int pkv_pool_block_hash(const pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens, uint64_t extra_key,
                        uint8_t* hashes_out, int32_t cap) {
  if (!pool || num_tokens < 0 || (num_tokens > 0 && !tokens) || cap < 0 || (cap > 0 && !hashes_out))
    return PKV_EINVAL;
  const int32_t full = num_tokens / pool->block_size;
  const int32_t n = full < cap ? full : cap;
  try {
    std::vector<Digest> h;
    chain(pool, tokens, n, extra_key, &h);
    for (int32_t j = 0; j < n; ++j) memcpy(hashes_out + 32 * (size_t)j, h[j].data(), 32);
  } catch (...) {
    return PKV_ELAUNCH;
  }
  return n;
}

int32_t pkv_pool_match_prefix(pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens, uint64_t extra_key,
                              int32_t* blocks_out, int32_t cap) {
  if (!pool || num_tokens < 0 || (num_tokens > 0 && !tokens) || cap < 0 || (cap > 0 && !blocks_out))
    return PKV_EINVAL;
  if (num_tokens == 0) return 0;
  // at most floor((n - 1) / B) blocks: the last token is always computed
  int32_t limit = (num_tokens - 1) / pool->block_size;
  if (limit > cap) limit = cap;
  std::vector<int32_t> hit;
  try {
    Digest parent{};
    for (int32_t j = 0; j < limit; ++j) {
      const Digest h = block_hash(parent, extra_key, tokens + (size_t)j * pool->block_size, pool->block_size);
      auto it = pool->index.find(h);
      if (it == pool->index.end()) break;   // first miss: nothing after it can be cached
      hit.push_back(it->second);
      parent = h;
    }
  } catch (...) {
    return PKV_ELAUNCH;
  }
  for (size_t j = 0; j < hit.size(); ++j) {
    const int32_t b = hit[j];
    if (pool->ref[b] == 0) take_from_free(pool, b);   // "touch": a hit leaves the free queue
    ++pool->ref[b];
    blocks_out[j] = b;
  }
  return (int32_t)hit.size();
}

int32_t pkv_pool_allocate(pkv_block_pool* pool, int32_t count, int32_t* blocks_out) {
  if (!pool || count < 0 || (count > 0 && !blocks_out)) return PKV_EINVAL;
  if ((size_t)count > pool->free_queue.size()) return PKV_ENOSPACE;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t b = pool->free_queue.front();   // least recently used
    pool->free_queue.pop_front();
    evict(pool, b);                               // a cached block loses its hash before reuse
    pool->ref[b] = 1;
    blocks_out[i] = b;
  }
  return count;
}

int32_t pkv_pool_cache_blocks(pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens, uint64_t extra_key,
                              const int32_t* blocks, int32_t num_blocks) {
  if (!pool || num_tokens < 0 || num_blocks < 0 || (num_tokens > 0 && !tokens) || (num_blocks > 0 && !blocks))
    return PKV_EINVAL;
  int32_t full = num_tokens / pool->block_size;
  if (full > num_blocks) full = num_blocks;
  for (int32_t j = 0; j < full; ++j)
    if (!valid_block(pool, blocks[j]) || pool->ref[blocks[j]] == 0) return PKV_EINVAL;
  int32_t added = 0;
  try {
    std::vector<Digest> h;
    chain(pool, tokens, full, extra_key, &h);
    for (int32_t j = 0; j < full; ++j) {
      const int32_t b = blocks[j];
      if (pool->cached[b]) continue;                 // already indexed (a hit, or cached earlier)
      if (pool->index.count(h[j])) continue;         // same content held by another block: keep that one
      pool->index.emplace(h[j], b);
      pool->hash[b] = h[j];
      pool->cached[b] = 1;
      ++added;
    }
  } catch (...) {
    return PKV_ELAUNCH;
  }
  return added;
}

int pkv_pool_ref(pkv_block_pool* pool, const int32_t* blocks, int32_t num_blocks) {
  if (!pool || num_blocks < 0 || (num_blocks > 0 && !blocks)) return PKV_EINVAL;
  for (int32_t j = 0; j < num_blocks; ++j)
    if (!valid_block(pool, blocks[j]) || pool->ref[blocks[j]] == 0) return PKV_EINVAL;
  for (int32_t j = 0; j < num_blocks; ++j) ++pool->ref[blocks[j]];
  return PKV_OK;
}

int pkv_pool_free(pkv_block_pool* pool, const int32_t* blocks, int32_t num_blocks) {
  if (!pool || num_blocks < 0 || (num_blocks > 0 && !blocks)) return PKV_EINVAL;
  try {   // every id valid and referenced at least as often as it is listed
    std::unordered_map<int32_t, int32_t> times;
    for (int32_t j = 0; j < num_blocks; ++j) {
      const int32_t b = blocks[j];
      if (!valid_block(pool, b) || ++times[b] > pool->ref[b]) return PKV_EINVAL;
    }
  } catch (...) {
    return PKV_ELAUNCH;
  }
  // The last block first: a chain's tail then becomes least recently used
  // before its head, so eviction never strands reachable blocks behind a
  // missing prefix block.
  for (int32_t j = num_blocks - 1; j >= 0; --j) {
    const int32_t b = blocks[j];
    if (--pool->ref[b] == 0) pool->pos[b] = pool->free_queue.insert(pool->free_queue.end(), b);
  }
  return PKV_OK;
}

}  // extern "C"
