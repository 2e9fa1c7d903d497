// Internal declarations shared by the HIP translation units of libpagedkv.
// Not part of the public ABI (that is include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <functional>
#include <queue>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

// Host block allocator state (blocks.hip, prefix.hip), also read by the step planner.
// A block with no references is either free (no content kept; in free_ids) or, with
// the prefix cache enabled, evictable (its cached content kept; in the LRU list).
struct pkv_block_key {
  uint64_t w[4];  // the 32 key bytes
  bool operator==(const pkv_block_key &o) const {
    return w[0] == o.w[0] && w[1] == o.w[1] && w[2] == o.w[2] && w[3] == o.w[3];
  }
};
struct pkv_block_key_hash {
  size_t operator()(const pkv_block_key &k) const { return (size_t)k.w[0]; }
};
struct pkv_block_allocator {
  std::vector<int32_t> ref;  // reference count per physical block
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_ids;
  // Prefix cache (off until enabled): key per cached block, the key -> block map, and
  // the evictable blocks as a doubly linked list in least-recently-used order.
  bool prefix = false;
  std::vector<uint8_t> has_key;
  std::vector<pkv_block_key> key;
  std::unordered_map<pkv_block_key, int32_t, pkv_block_key_hash> block_of;
  std::vector<int32_t> lru_prev, lru_next;  // -1 = none; membership: in_lru
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1, lru_count = 0;
};

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;  // tokens per physical block
constexpr int kWaves = 4;               // waves per workgroup in every kernel
constexpr int kThreads = 64 * kWaves;

// Whether block b is held (reference count > 0) by the allocator.
inline bool held(const pkv_block_allocator *a, int32_t b) {
  return b >= 0 && b < (int32_t)a->ref.size() && a->ref[b] > 0;
}

// Blocks that can be handed out: free ones plus evictable cached ones.
inline int64_t available(const pkv_block_allocator *a) {
  return (int64_t)a->free_ids.size() + a->lru_count;
}

// Eviction-list and key bookkeeping of the prefix cache (prefix.hip).
void lru_unlink(pkv_block_allocator *a, int32_t b);
void lru_push_back(pkv_block_allocator *a, int32_t b);
void forget_key(pkv_block_allocator *a, int32_t b);

// The append of pkv_allocator_append after its checks: the caller has verified the
// table's used entries and that enough blocks are free.  Returns the copies made (0
// or 1, the pair written to copies[0..1]).
int32_t append_unchecked(pkv_block_allocator *a, int32_t *table, int32_t context_len,
                         int32_t num_new, int32_t *slots, int32_t *copies);

// Decode (single-query rows) plan.
//
// Work items ("rows") are sequences with one query (bf16) or every query row (fp32,
// where prefill rows also take this path).  A segment is (row, kv-head group).  Its
// blocks are cut into `splits` contiguous key ranges, one workgroup each, whose waves
// take the range's blocks in turn and merge their states in LDS.  With one range per
// segment the workgroup writes the output; otherwise each range leaves a normalised
// partial (o, log2-sum-exp) and a merge kernel combines them.
// ---------------------------------------------------------------------------
constexpr int kDecodeWavesMax = 16;  // waves per decode workgroup: 16 when the
constexpr int kDecodeWavesMin = 8;   // segments fit the compute units one each, else 8
constexpr int kBlocksPerWave = 16;   // blocks a wave may take before segments split
// The same bound for the decode rows of a mixed launch: those run longest first after
// the chunk tiles, so longer pieces start early, and rows up to 4,096 keys then need
// no key ranges (no merge launch).
constexpr int kMixedBlocksPerWave = 32;

struct DecodePlan {
  int items;            // work rows: num_seqs (bf16) or total_q (fp32)
  int group;            // G = num_q_heads / num_kv_heads
  int head_group;       // q heads handled together by one wave (divides G)
  int num_head_groups;  // G / head_group
  int waves;            // waves per workgroup (kDecodeWavesMax or kDecodeWavesMin)
  int splits;           // key ranges (workgroups) per segment
  int skip_blocks;      // leading blocks of every row left out (a shared prefix), or 0
  int max_context_len;  // the call's bound on context_lens
  bool cascade;         // partials even with one range, no merge launch (the shared-
                        // prefix merge combines them with the shared run's partials)
  size_t ws_o_offset, ws_lse_offset, ws_bytes;
  void *workspace;      // set by the caller before launching
};

// mixed: the decode rows run in the workgroups of the chunk launch that follow its
// tiles (kDecodeWavesMin waves each).
DecodePlan plan_decode(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len, pkv_dtype dtype,
                       int skip_blocks = 0, bool cascade = false, bool mixed = false);

struct AttnArgs {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;
  int num_seqs, total_q, num_blocks, max_blocks_per_seq;
  int num_q_heads, num_kv_heads, head_dim;
  int max_query_len;
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
  // Fused slot write (all null otherwise): this step's new rows [total_q][Hkv][D] and
  // their slots.  The decode kernel stores them into the pools and takes each decode
  // row's newest key and value from k_new / v_new instead of the pool.
  const void *k_new;
  const void *v_new;
  const int32_t *slot_mapping;
};

// Per-launch arguments of the decode and merge kernels.
struct SegArgs {
  int items;             // work rows
  int num_head_groups;   // G / head_group
  int groups;            // num_kv_heads * num_head_groups
  int splits;            // key ranges per segment
  int skip_blocks;       // leading logical blocks of every row this launch leaves out
  int partials;          // nonzero: every range writes its partial instead of `out`
  float *ws_o;           // [segment][range][head_group][D] normalised partial outputs
  float *ws_lse;         // [segment][range][head_group] log2-sum-exp (-inf: no key)
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_kv_write(const void *k_new, const void *v_new, void *k_pool,
                           void *v_pool, const int32_t *slot_mapping, int num_tokens,
                           int num_blocks, int num_kv_heads, int head_dim, pkv_dtype dtype,
                           hipStream_t stream);

hipError_t launch_decode(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                         hipStream_t stream);
// Kernel arguments of a decode plan, and the merge of its key ranges alone (for plans
// whose decode workgroups ran inside another launch).
SegArgs decode_seg_args(const DecodePlan &p, int num_kv_heads);
hipError_t launch_decode_merge(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                               hipStream_t stream);

// Prefill (chunk) plan.  A workgroup owns kPrefillCols (query row, q head) columns of
// one KV head; with fewer tiles than compute units the key range of each tile is split
// over `splits` workgroups whose partial results a merge kernel combines.
constexpr int kPrefillCols = 128;
constexpr int kPrefillStepKeys = 128;  // keys per step of the chunk kernel
struct PrefillPlan {
  int head_group;       // q heads per tile (4, 2 or 1)
  int num_head_groups;  // G / head_group
  int tile_slots;       // tile slots per (kv head, head group)
  int tiles;            // tile_slots * num_kv_heads * num_head_groups
  int splits;           // key-range splits per tile (1 = none)
  size_t ws_o_offset, ws_lse_offset, ws_col_offset, ws_end;  // ws_end: bytes used
  void *workspace;      // set by the caller before launching
};
// Partial-result buffers of a split launch (unused when splits == 1).
struct PrefillSplit {
  int splits;
  float *o;    // [tile][split][column][D] normalised partial outputs
  float *lse;  // [tile][split][column] log2-sum-exp (-inf: no key seen)
  int *col;    // [tile][column] output row index (row * Hq + head), -1 = unused
  // Shared-run mode (> 0): every query row of the batch is a column of one chunk over
  // the first shared_keys keys of table row 0, without a causal limit (each row sees
  // them all); tile slot t holds rows [t*BM, (t+1)*BM).  Partials are always written.
  int shared_keys;
};

PrefillPlan plan_prefill(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                         int head_dim, int max_context_len, pkv_dtype dtype,
                         size_t ws_offset);
// Plan of the shared-run pass (bf16): tiles of every query row over shared_keys keys,
// split over enough workgroups to fill the GPU (one or more key steps each).
PrefillPlan plan_shared_run(int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                            int shared_keys, size_t ws_offset);
hipError_t launch_prefill(const AttnArgs &a, const PrefillPlan &p, pkv_dtype dtype,
                          hipStream_t stream);
// A batch of chunks and decode rows (bf16) in one launch: the chunk tiles first, then
// the decode workgroups of plan `dp` (planned with mixed = true), then the merges.
hipError_t launch_mixed(const AttnArgs &a, const PrefillPlan &pp, const DecodePlan &dp,
                        hipStream_t stream);
// Decode head group that the mixed launch pairs with a chunk head group (equal to the
// one plan_decode picks for the same GQA group).
constexpr int mixed_decode_head_group(int head_dim, int chunk_head_group) {
  return head_dim == 64 ? chunk_head_group : (chunk_head_group > 2 ? 2 : chunk_head_group);
}
// The shared-run pass (the prefill kernel in shared-run mode, partials only) and the
// private parts' decode workgroups (plan `dp`, planned with cascade and mixed set) in
// one launch: the shared-run tiles first (they also store a fused call's new rows),
// then the decode workgroups.
hipError_t launch_shared_run_mixed(const AttnArgs &a, const PrefillPlan &sp, int shared_keys,
                                   const DecodePlan &dp, hipStream_t stream);
// Merge of a shared-prefix batch: per (row, q head), the decode pieces of the private
// part (plan `dp`, launched with cascade set) and the shared run's splits (plan `sp`).
hipError_t launch_cascade_merge(const AttnArgs &a, const DecodePlan &dp,
                                const PrefillPlan &sp, hipStream_t stream);

// Row-tile count bound of the prefill launch: the sequences' ceil(q_len / BM) row tiles
// add up to at most floor(total_q / BM) plus one per sequence.
inline int prefill_tile_slots(int total_q, int num_seqs, int rows_per_tile) {
  return total_q / rows_per_tile + num_seqs;
}

// Index of the prefill tile of row tile j and head unit h (kv head * head groups + head
// group) among `units` head units: row tiles are the slow index, so with the tiles
// launched in index order every XCD's real tiles come before the empty slots.
__host__ __device__ inline int prefill_tile_index(int j, int h, int units) {
  return j * units + h;
}

}  // namespace pkv
