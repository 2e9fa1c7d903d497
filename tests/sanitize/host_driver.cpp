// Host-only exercise of libpagedkv's C ABI for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code: the block allocator (append, fork,
// release, copy-on-write, out-of-blocks), prefix caching (keys, match, register,
// eviction), the chunked-prefill step planner, the metadata validator, and the
// argument checks of the GPU entry points (calls that return before any launch).
// No GPU is touched.  A random serving loop runs for a fixed number of steps from a
// fixed seed; every status is checked against what the header promises, and the
// program exits non-zero on the first mismatch.  Memory errors abort through the
// sanitizers.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "pagedkv.h"

static int g_fail = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                         \
    }                                                                     \
  } while (0)

namespace {

constexpr int kBlocks = 96;
constexpr int kMaxBlocks = 40;  // per request
constexpr int kRequests = 12;

struct Request {
  std::vector<int32_t> table = std::vector<int32_t>(kMaxBlocks, -1);
  std::vector<int32_t> tokens;
  int32_t prompt = 0, computed = 0;
  bool live = false;
};

void allocator_loop(std::mt19937 &rng) {
  pkv_block_allocator *al = nullptr;
  EXPECT(pkv_allocator_create(kBlocks, &al) == PKV_OK && al);
  EXPECT(pkv_allocator_enable_prefix_cache(al) == PKV_OK);
  std::vector<Request> req(kRequests);
  std::vector<int32_t> slots(kMaxBlocks * 16), copies(2), keys;
  for (int it = 0; it < 4000; ++it) {
    Request &r = req[rng() % kRequests];
    const int op = (int)(rng() % 5);
    if (!r.live) {  // start a request, possibly hitting the prefix cache
      r = Request();
      r.prompt = 1 + (int)(rng() % 200);
      for (int t = 0; t < r.prompt; ++t) r.tokens.push_back((int32_t)(rng() % 7));
      std::vector<uint8_t> k((size_t)(r.prompt / 16 + 1) * PKV_KEY_BYTES);
      int32_t nk = -1, hit = -1;
      EXPECT(pkv_block_keys(r.tokens.data(), r.prompt, nullptr, 0, nullptr, k.data(),
                            r.prompt / 16 + 1, &nk) == PKV_OK);
      EXPECT(nk == r.prompt / 16);
      // keep at least one token to compute
      const int32_t usable = (r.prompt - 1) / 16;
      EXPECT(pkv_prefix_match(al, k.data(), usable, r.table.data(), &hit) == PKV_OK);
      EXPECT(hit >= 0 && hit <= usable);
      r.computed = hit * 16;
      r.live = true;
      continue;
    }
    const int32_t used = (r.computed + 15) / 16;
    if (op == 0) {  // finish: register full blocks, release
      std::vector<uint8_t> k((size_t)(r.computed / 16 + 1) * PKV_KEY_BYTES);
      int32_t nk = 0;
      EXPECT(pkv_block_keys(r.tokens.data(), r.computed, nullptr, 0, nullptr, k.data(),
                            r.computed / 16 + 1, &nk) == PKV_OK);
      EXPECT(pkv_prefix_register(al, r.table.data(), k.data(), nk) == PKV_OK);
      EXPECT(pkv_allocator_release(al, r.table.data(), used) == PKV_OK);
      r.live = false;
    } else if (op == 1 && used > 0) {  // fork into another free request slot
      for (Request &o : req) {
        if (o.live) continue;
        EXPECT(pkv_allocator_fork(al, r.table.data(), used) == PKV_OK);
        o = r;
        break;
      }
    } else {  // append tokens
      const int32_t n = 1 + (int32_t)(rng() % 40);
      if ((r.computed + n + 15) / 16 > kMaxBlocks) {
        int32_t nc = -1;
        EXPECT(pkv_allocator_append(al, r.table.data(), kMaxBlocks, r.computed, n,
                                    slots.data(), copies.data(), 1, &nc) ==
               PKV_ERR_INVALID_ARG);
        continue;
      }
      int32_t nc = -1;
      const pkv_status st = pkv_allocator_append(al, r.table.data(), kMaxBlocks,
                                                 r.computed, n, slots.data(),
                                                 copies.data(), 1, &nc);
      EXPECT(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
      if (st == PKV_OK) {
        for (int t = 0; t < n; ++t) r.tokens.push_back((int32_t)(rng() % 7));
        r.computed += n;
        EXPECT(nc == 0 || nc == 1);
      }
    }
    EXPECT(pkv_allocator_num_free(al) >= 0 && pkv_allocator_num_free(al) <= kBlocks);
    EXPECT(pkv_prefix_num_evictable(al) <= pkv_prefix_num_cached(al));
  }
  for (Request &r : req)
    if (r.live) EXPECT(pkv_allocator_release(al, r.table.data(), (r.computed + 15) / 16) == PKV_OK);
  EXPECT(pkv_allocator_refcount(al, -1) == -1 && pkv_allocator_refcount(al, kBlocks) == -1);
  pkv_allocator_destroy(al);
  EXPECT(pkv_allocator_num_free(nullptr) == -1);
}

void planner_loop(std::mt19937 &rng) {
  pkv_block_allocator *al = nullptr;
  EXPECT(pkv_allocator_create(kBlocks, &al) == PKV_OK);
  const int n = 8;
  std::vector<int32_t> prompt(n), computed(n, 0), qlen(n), tables(n * kMaxBlocks, -1);
  for (int i = 0; i < n; ++i) prompt[i] = 1 + (int32_t)(rng() % 300);
  std::vector<int32_t> seq_req(n), bt(n * kMaxBlocks), qsl(n + 1), ctx(n), slots(512),
      cps(2 * n);
  for (int step = 0; step < 200; ++step) {
    const int32_t budget = 1 + (int32_t)(rng() % 256);
    EXPECT(pkv_plan_step(n, prompt.data(), computed.data(), budget, qlen.data()) == PKV_OK);
    int32_t tot = 0;
    for (int i = 0; i < n; ++i) tot += qlen[i];
    EXPECT(tot <= budget);
    int32_t ns = -1, nc = -1;
    const pkv_status st = pkv_build_step(al, n, tables.data(), kMaxBlocks, computed.data(),
                                         qlen.data(), seq_req.data(), bt.data(), qsl.data(),
                                         ctx.data(), slots.data(), (int32_t)slots.size(),
                                         cps.data(), &ns, &nc);
    EXPECT(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_INVALID_ARG);
    if (st != PKV_OK) {
      EXPECT(ns == 0 && nc == 0);
      // drop the longest request to make room
      int big = 0;
      for (int i = 1; i < n; ++i)
        if (computed[i] > computed[big]) big = i;
      EXPECT(pkv_allocator_release(al, &tables[big * kMaxBlocks], (computed[big] + 15) / 16) ==
             PKV_OK);
      for (int b = 0; b < kMaxBlocks; ++b) tables[big * kMaxBlocks + b] = -1;
      computed[big] = 0;
      prompt[big] = 1 + (int32_t)(rng() % 300);
      continue;
    }
    int32_t bad = -1;
    EXPECT(pkv_validate_metadata(bt.data(), ctx.data(), qsl.data(), slots.data(), ns,
                                 qsl[ns], kBlocks, kMaxBlocks, &bad) == PKV_OK);
    for (int i = 0; i < n; ++i) {
      computed[i] += qlen[i];
      if (computed[i] >= prompt[i] + 20) {  // finished: start a new prompt
        EXPECT(pkv_allocator_release(al, &tables[i * kMaxBlocks], (computed[i] + 15) / 16) ==
               PKV_OK);
        for (int b = 0; b < kMaxBlocks; ++b) tables[i * kMaxBlocks + b] = -1;
        computed[i] = 0;
        prompt[i] = 1 + (int32_t)(rng() % 300);
      } else if (computed[i] >= prompt[i] && computed[i] + 1 > kMaxBlocks * 16) {
        computed[i] = kMaxBlocks * 16;  // never reached with these sizes
      }
    }
  }
  pkv_allocator_destroy(al);
}

void validator_and_arguments() {
  // A broken table entry, duplicate slots, q_len > context: all rejected.
  int32_t bt[2 * 4] = {0, 1, -1, -1, 2, 99, -1, -1};
  int32_t ctx[2] = {20, 30};
  int32_t qsl[3] = {0, 1, 2};
  int32_t slots[2] = {19, 19};
  int32_t bad = -1;
  EXPECT(pkv_validate_metadata(bt, ctx, qsl, nullptr, 2, 2, 8, 4, &bad) ==
             PKV_ERR_INVALID_ARG &&
         bad == 1);
  bt[5] = 3;
  EXPECT(pkv_validate_metadata(bt, ctx, qsl, nullptr, 2, 2, 8, 4, &bad) == PKV_OK);
  EXPECT(pkv_validate_metadata(bt, ctx, qsl, slots, 2, 2, 8, 4, &bad) == PKV_ERR_INVALID_ARG);
  int32_t qsl2[3] = {0, 25, 26};
  EXPECT(pkv_validate_metadata(bt, ctx, qsl2, nullptr, 2, 26, 8, 4, &bad) ==
         PKV_ERR_INVALID_ARG);
  // GPU entry points: scalar checks return before any launch.
  char dummy[64];
  void *p = dummy;
  EXPECT(paged_attention_varlen(p, p, p, p, bt, ctx, qsl, 2, 2, 8, 4, 30, 1, 6, 4, 64, 16,
                                0.125f, PKV_BF16, p, 64, nullptr) == PKV_ERR_INVALID_ARG);
  EXPECT(paged_attention_varlen(p, p, p, p, bt, ctx, qsl, 2, 2, 8, 4, 30, 1, 8, 4, 64, 32,
                                0.125f, PKV_BF16, p, 64, nullptr) == PKV_ERR_UNSUPPORTED);
  EXPECT(paged_attention_varlen(p, p, p, p, bt, ctx, qsl, 0, 0, 8, 4, 30, 1, 8, 4, 64, 16,
                                0.125f, PKV_BF16, p, 64, nullptr) == PKV_OK);
  EXPECT(paged_kv_write(p, p, p, p, slots, 2, 8, 4, 96, 16, PKV_BF16, nullptr) ==
         PKV_ERR_UNSUPPORTED);
  EXPECT(paged_attention_workspace_size(32, 32, 32, 8, 64, 2048, PKV_BF16) == 0);
  EXPECT(paged_attention_workspace_size(32, 32, 32, 8, 64, 9000, PKV_BF16) > 0);
  EXPECT(paged_attention_workspace_size(32, 32, 30, 8, 64, 2048, PKV_BF16) == 0);
  for (int s = -1; s < 8; ++s) EXPECT(pkv_status_string((pkv_status)s) != nullptr);
  // The fused call's positional slots: row 0 is position 19 (table block 1 = physical
  // 1, offset 3), row 1 position 29 (table block 1 = physical 3, offset 13).
  int32_t pos_slots[2] = {1 * 16 + 3, 3 * 16 + 13};
  EXPECT(pkv_validate_fused_metadata(bt, ctx, qsl, pos_slots, 2, 2, 8, 4, &bad) == PKV_OK);
  pos_slots[0] = 0 * 16 + 3;
  EXPECT(pkv_validate_fused_metadata(bt, ctx, qsl, pos_slots, 2, 2, 8, 4, &bad) ==
         PKV_ERR_INVALID_ARG && bad == 0);
  pos_slots[0] = 1 * 16 + 3;
  pos_slots[1] = 2 * 16 + 13;
  EXPECT(pkv_validate_fused_metadata(bt, ctx, qsl, pos_slots, 2, 2, 8, 4, &bad) ==
         PKV_ERR_INVALID_ARG && bad == 1);
  // Shared prefixes: the first table entry differs between the rows.
  EXPECT(pkv_validate_shared_prefix(bt, ctx, qsl, 2, 4, 1, &bad) == PKV_ERR_INVALID_ARG &&
         bad == 1);
  EXPECT(pkv_validate_shared_prefix(bt, ctx, qsl, 2, 4, 0, &bad) == PKV_OK);
  EXPECT(pkv_validate_shared_prefix(bt, ctx, qsl, 2, 4, 5, &bad) == PKV_ERR_INVALID_ARG);
  EXPECT(paged_attention_varlen_shared_prefix(p, p, nullptr, nullptr, p, p, nullptr, bt, ctx,
                                              qsl, 2, 2, 8, 4, 30, 1, 1, 8, 4, 64, 16,
                                              0.125f, PKV_F32, p, 64, nullptr) ==
         PKV_ERR_UNSUPPORTED);
  EXPECT(paged_attention_varlen_shared_prefix(p, p, nullptr, nullptr, p, p, nullptr, bt, ctx,
                                              qsl, 2, 2, 8, 4, 30, 1, 1, 8, 4, 64, 16,
                                              0.125f, PKV_BF16, p, 64, nullptr) ==
         PKV_ERR_WORKSPACE);
  EXPECT(paged_attention_shared_prefix_workspace_size(2, 8, 4, 64, 30, 1, PKV_BF16) > 64);
  // The no-alloc call: a batch beyond its scratch is refused before any device call.
  EXPECT(paged_attention_varlen_with_write_noalloc(p, p, p, p, p, p, slots, bt, ctx, qsl, 256,
                                                   256, 8, 4, 32768, 1, 16, 8, 128, 16,
                                                   0.125f, PKV_BF16, nullptr) ==
         PKV_ERR_WORKSPACE);
}

}  // namespace

int main() {
  std::mt19937 rng(20261202u);
  allocator_loop(rng);
  planner_loop(rng);
  validator_and_arguments();
  if (g_fail) return 1;
  printf("host driver ok\n");
  return 0;
}
