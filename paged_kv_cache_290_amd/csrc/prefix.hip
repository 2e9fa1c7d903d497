// Prefix caching (host): content keys of full blocks and the bookkeeping that lets a
// new request point its table at blocks already holding its prefix.
//
// Method (pages cited by title and section):
//  * Serving-engine KV page (ttlab), section 4 "prefix cache": each full block gets a
//    key hashed from the previous block's key, the block's token ids and extra inputs
//    (adapter, multimodal hashes, a cache salt), so a key stands for the whole prefix;
//    SHA-256 is the hash; freed blocks keep their contents in a queue, entered tail
//    first and evicted least recently used first when space is needed.
//  * "How inference engines actually work" page (xiaohu-jiedu), prefix caching in the
//    agent-traffic section: a request whose prefix matches reuses the blocks through
//    its block table, so only the new tail is prefilled.
//
// Hash input of a block (a layout choice; the pages name only the three parts): the
// previous key (32 bytes, all zero before the first block), the 16 token ids as
// little-endian int32, the extras length as little-endian uint32, the extras bytes.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "pkv_internal.h"

namespace pkv {
// SHA-256 compression with the x86 SHA extensions (sha256_x86.cpp, host compiler).
bool sha256_x86_available();
void sha256_x86_chunks(uint32_t h[8], const uint8_t *data, size_t nchunks);
}  // namespace pkv

namespace {

// ---------------------------------------------------------------------------
// SHA-256 (FIPS 180-4): 64 rounds over 512-bit chunks, big-endian words.
// ---------------------------------------------------------------------------

constexpr uint32_t kSha256K[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
    0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
    0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
    0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
    0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
    0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
    0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
    0xc67178f2};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha256_chunk(uint32_t h[8], const uint8_t *p) {
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t)p[4 * i] << 24 | (uint32_t)p[4 * i + 1] << 16 |
           (uint32_t)p[4 * i + 2] << 8 | (uint32_t)p[4 * i + 3];
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + kSha256K[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

void sha256(const uint8_t *msg, size_t len, uint8_t out[32]) {
  uint32_t h[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                   0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
  // The SHA extensions are used when the host CPU has them.  A build with
  // PKV_SHA256_PORTABLE_ONLY defined always takes the portable rounds (the tests build
  // such a copy to check that path as well).
#ifdef PKV_SHA256_PORTABLE_ONLY
  static const bool x86 = false;
#else
  static const bool x86 = pkv::sha256_x86_available();
#endif
  auto chunks = [&](const uint8_t *p, size_t n) {
    if (x86) {
      pkv::sha256_x86_chunks(h, p, n);
    } else {
      for (size_t i = 0; i < n; ++i) sha256_chunk(h, p + 64 * i);
    }
  };
  size_t off = len / 64 * 64;
  chunks(msg, len / 64);
  // Final chunk(s): the rest, 0x80, zeros, the bit length as a big-endian uint64.
  uint8_t tail[128] = {0};
  const size_t rest = len - off;
  memcpy(tail, msg + off, rest);
  tail[rest] = 0x80;
  const size_t tl = rest + 9 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8;
  for (int i = 0; i < 8; ++i) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  chunks(tail, tl / 64);
  for (int i = 0; i < 8; ++i) {
    out[4 * i] = (uint8_t)(h[i] >> 24);
    out[4 * i + 1] = (uint8_t)(h[i] >> 16);
    out[4 * i + 2] = (uint8_t)(h[i] >> 8);
    out[4 * i + 3] = (uint8_t)h[i];
  }
}

pkv_block_key key_from(const uint8_t *p) {
  pkv_block_key k;
  memcpy(k.w, p, sizeof(k.w));
  return k;
}

}  // namespace

namespace pkv {

void lru_unlink(pkv_block_allocator *a, int32_t b) {
  const int32_t p = a->lru_prev[b], n = a->lru_next[b];
  if (p >= 0) a->lru_next[p] = n; else a->lru_head = n;
  if (n >= 0) a->lru_prev[n] = p; else a->lru_tail = p;
  a->lru_prev[b] = a->lru_next[b] = -1;
  a->in_lru[b] = 0;
  --a->lru_count;
}

void lru_push_back(pkv_block_allocator *a, int32_t b) {
  a->lru_prev[b] = a->lru_tail;
  a->lru_next[b] = -1;
  if (a->lru_tail >= 0) a->lru_next[a->lru_tail] = b; else a->lru_head = b;
  a->lru_tail = b;
  a->in_lru[b] = 1;
  ++a->lru_count;
}

void forget_key(pkv_block_allocator *a, int32_t b) {
  if (!a->prefix || !a->has_key[b]) return;
  a->block_of.erase(a->key[b]);
  a->has_key[b] = 0;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

pkv_status pkv_block_keys(const int32_t *tokens, int32_t num_tokens, const void *extras,
                          int32_t extras_len, const uint8_t *parent_key, uint8_t *keys,
                          int32_t max_keys, int32_t *num_keys) {
  if (num_keys) *num_keys = 0;
  if (num_tokens < 0 || extras_len < 0 || max_keys < 0 || !num_keys ||
      (num_tokens > 0 && !tokens) || (extras_len > 0 && !extras))
    return PKV_ERR_INVALID_ARG;
  const int32_t n = num_tokens / kBlock;
  if (n > max_keys || (n > 0 && !keys)) return PKV_ERR_INVALID_ARG;
  std::vector<uint8_t> msg;
  try {
    msg.resize(32 + 4 * kBlock + 4 + (size_t)extras_len);
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  if (parent_key) memcpy(msg.data(), parent_key, 32); else memset(msg.data(), 0, 32);
  uint8_t *tok = msg.data() + 32;
  uint8_t *len = tok + 4 * kBlock;
  for (int i = 0; i < 4; ++i) len[i] = (uint8_t)((uint32_t)extras_len >> (8 * i));
  if (extras_len > 0) memcpy(len + 4, extras, (size_t)extras_len);
  for (int32_t b = 0; b < n; ++b) {
    for (int i = 0; i < kBlock; ++i) {
      const uint32_t t = (uint32_t)tokens[b * kBlock + i];
      for (int j = 0; j < 4; ++j) tok[4 * i + j] = (uint8_t)(t >> (8 * j));
    }
    sha256(msg.data(), msg.size(), keys + 32 * (size_t)b);
    memcpy(msg.data(), keys + 32 * (size_t)b, 32);  // the next block chains this key
  }
  *num_keys = n;
  return PKV_OK;
}

pkv_status pkv_allocator_enable_prefix_cache(pkv_block_allocator *alloc) {
  if (!alloc) return PKV_ERR_INVALID_ARG;
  if (alloc->prefix) return PKV_OK;
  const size_t n = alloc->ref.size();
  try {
    alloc->has_key.assign(n, 0);
    alloc->key.assign(n, pkv_block_key{});
    alloc->lru_prev.assign(n, -1);
    alloc->lru_next.assign(n, -1);
    alloc->in_lru.assign(n, 0);
    alloc->block_of.reserve(n);
  } catch (...) {
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  alloc->prefix = true;
  return PKV_OK;
}

pkv_status pkv_prefix_match(pkv_block_allocator *alloc, const uint8_t *keys, int32_t num_keys,
                            int32_t *table, int32_t *num_hit) {
  if (num_hit) *num_hit = 0;
  if (!alloc || !alloc->prefix || num_keys < 0 || !num_hit || (num_keys > 0 && (!keys || !table)))
    return PKV_ERR_INVALID_ARG;
  int32_t h = 0;
  for (; h < num_keys; ++h) {
    const auto it = alloc->block_of.find(key_from(keys + 32 * (size_t)h));
    if (it == alloc->block_of.end()) break;
    table[h] = it->second;
  }
  for (int32_t i = 0; i < h; ++i) {
    const int32_t b = table[i];
    if (alloc->ref[b] == 0) lru_unlink(alloc, b);
    ++alloc->ref[b];
  }
  *num_hit = h;
  return PKV_OK;
}

pkv_status pkv_prefix_register(pkv_block_allocator *alloc, const int32_t *table,
                               const uint8_t *keys, int32_t num_keys) {
  if (!alloc || !alloc->prefix || num_keys < 0 || (num_keys > 0 && (!keys || !table)))
    return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_keys; ++i)
    if (!held(alloc, table[i])) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_keys; ++i) {
    const int32_t b = table[i];
    const pkv_block_key k = key_from(keys + 32 * (size_t)i);
    if (alloc->has_key[b] || alloc->block_of.count(k)) continue;  // first mapping stays
    alloc->key[b] = k;
    alloc->has_key[b] = 1;
    alloc->block_of.emplace(k, b);
  }
  return PKV_OK;
}

int32_t pkv_prefix_num_cached(const pkv_block_allocator *alloc) {
  return alloc ? (int32_t)alloc->block_of.size() : -1;
}

int32_t pkv_prefix_num_evictable(const pkv_block_allocator *alloc) {
  return alloc ? alloc->lru_count : -1;
}

}  // extern "C"
