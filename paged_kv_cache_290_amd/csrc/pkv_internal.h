// Internal declarations shared by the HIP translation units of libpagedkv.
// Not part of the public ABI (that is include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;  // tokens per physical block
constexpr int kWaves = 4;               // waves per workgroup in every kernel
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// Decode (one query row per work item) split-K plan.
//
// A work item is (row, kv head, head group, split).  Rows are sequences with one
// query (bf16) or every query row (fp32, where prefill rows also take this path).
// A split covers `blocks_per_split` consecutive logical blocks; the four waves of a
// workgroup take its blocks round-robin and merge in LDS.  Rows with more than one
// split leave partial results in the workspace for the merge kernel.
// ---------------------------------------------------------------------------
struct DecodePlan {
  int items;            // work rows: num_seqs (bf16) or total_q (fp32)
  int group;            // G = num_q_heads / num_kv_heads
  int head_group;       // q heads handled together by one workgroup (divides G)
  int num_head_groups;  // G / head_group
  int blocks_per_split;
  int num_splits;       // upper bound over rows, from max_context_len
  size_t ws_o_offset, ws_lse_offset, ws_bytes;
};

DecodePlan plan_decode(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len, pkv_dtype dtype);

struct AttnArgs {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;
  float *ws_o;    // [items][Hq][num_splits][D] normalised partial outputs
  float *ws_lse;  // [items][Hq][num_splits] log2-sum-exp of each partial
  int num_seqs, total_q, num_blocks, max_blocks_per_seq;
  int num_q_heads, num_kv_heads, head_dim;
  int max_query_len;
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_kv_write(const void *k_new, const void *v_new, void *k_pool,
                           void *v_pool, const int32_t *slot_mapping, int num_tokens,
                           int num_blocks, int num_kv_heads, int head_dim, pkv_dtype dtype,
                           hipStream_t stream);

hipError_t launch_decode(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                         hipStream_t stream);

hipError_t launch_prefill(const AttnArgs &a, pkv_dtype dtype, hipStream_t stream);

// Work-slot count of the prefill launch: an upper bound on the number of query tiles
// over all sequences (each sequence's tiles fit between floor(qsl[s]/BM) + s and the
// next sequence's start).
inline int prefill_tile_slots(int total_q, int num_seqs, int rows_per_tile) {
  return total_q / rows_per_tile + num_seqs;
}

}  // namespace pkv
