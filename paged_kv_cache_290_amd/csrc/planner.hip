// Chunked-prefill step planning (host): which tokens of which requests run in one
// engine step under a token budget, and the varlen batch that step hands to the
// paged-attention path.
//
// Method (pages cited by title and section):
//  * Inference-engine page (xiaohu-jiedu), Chunked Prefill subsection: each step has a
//    token budget; a long prompt is cut into consecutive slices that fit it, and the
//    active users' single decode tokens are packed into every step.
//  * Serving-engine KV page (ttlab), section 3, "the new problem": chunked prefill
//    with decode-first filling; the page's per-step input-token limit counts every
//    token of the step.
//
// One step: every decoding request (prompt fully cached) gets one token, in request
// order, while the budget lasts; what is left goes to requests still prefilling, in
// request order, each taking min(remaining prompt, remaining budget) tokens.
#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <unordered_map>

#include "pkv_internal.h"

using pkv::kBlock;

extern "C" {

pkv_status pkv_plan_step(int32_t num_requests, const int32_t *prompt_len,
                         const int32_t *num_computed, int32_t token_budget,
                         int32_t *query_len) {
  if (num_requests < 0 || token_budget < 0) return PKV_ERR_INVALID_ARG;
  if (num_requests == 0) return PKV_OK;
  if (!prompt_len || !num_computed || !query_len) return PKV_ERR_INVALID_ARG;
  for (int32_t r = 0; r < num_requests; ++r)
    if (prompt_len[r] < 0 || num_computed[r] < 0) return PKV_ERR_INVALID_ARG;
  int64_t left = token_budget;
  for (int32_t r = 0; r < num_requests; ++r) {
    const bool decoding = prompt_len[r] > 0 && num_computed[r] >= prompt_len[r];
    query_len[r] = 0;
    if (decoding && left > 0) {
      query_len[r] = 1;
      --left;
    }
  }
  for (int32_t r = 0; r < num_requests && left > 0; ++r) {
    if (num_computed[r] < prompt_len[r]) {
      const int64_t want = (int64_t)prompt_len[r] - num_computed[r];
      const int64_t take = want < left ? want : left;
      query_len[r] = (int32_t)take;
      left -= take;
    }
  }
  return PKV_OK;
}

pkv_status pkv_build_step(pkv_block_allocator *alloc, int32_t num_requests, int32_t *tables,
                          int32_t max_blocks_per_seq, const int32_t *num_computed,
                          const int32_t *query_len, int32_t *seq_request,
                          int32_t *block_tables, int32_t *query_start_loc,
                          int32_t *context_lens, int32_t *slot_mapping, int32_t max_tokens,
                          int32_t *copies, int32_t *num_seqs, int32_t *num_copies) {
  if (num_seqs) *num_seqs = 0;
  if (num_copies) *num_copies = 0;
  if (!alloc || num_requests < 0 || max_blocks_per_seq <= 0 || max_tokens < 0 ||
      !num_seqs || !num_copies)
    return PKV_ERR_INVALID_ARG;
  if (num_requests == 0) return PKV_OK;
  if (!tables || !num_computed || !query_len || !seq_request || !block_tables ||
      !query_start_loc || !context_lens || !copies || (max_tokens > 0 && !slot_mapping))
    return PKV_ERR_INVALID_ARG;
  // Exact block need of the whole step (copy decisions see the earlier requests'
  // copies), so the step either fits completely or changes nothing.
  int64_t tokens = 0, need = 0;
  std::unordered_map<int32_t, int32_t> moved;  // block -> references moved off it
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t q = query_len[r], c = num_computed[r];
    if (q < 0 || c < 0) return PKV_ERR_INVALID_ARG;
    if (q == 0) continue;
    tokens += q;
    const int64_t end = (int64_t)c + q;
    if (end > INT32_MAX || (end + kBlock - 1) / kBlock > max_blocks_per_seq)
      return PKV_ERR_INVALID_ARG;
    const int32_t used = (c + kBlock - 1) / kBlock;
    const int32_t *row = tables + (size_t)r * max_blocks_per_seq;
    for (int32_t lb = 0; lb < used; ++lb)
      if (!pkv::held(alloc, row[lb])) return PKV_ERR_INVALID_ARG;
    need += (end + kBlock - 1) / kBlock - used;
    if (c % kBlock != 0) {
      const int32_t last = row[used - 1];
      if (alloc->ref[last] > 1) {
        int32_t &m = moved[last];
        if (alloc->ref[last] - m > 1) {
          ++need;
          ++m;
        }
      }
    }
  }
  if (tokens > max_tokens) return PKV_ERR_INVALID_ARG;
  if (need > pkv::available(alloc)) return PKV_ERR_OUT_OF_BLOCKS;

  int32_t s = 0, t = 0, nc = 0;
  query_start_loc[0] = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t q = query_len[r];
    if (q == 0) continue;
    int32_t *row = tables + (size_t)r * max_blocks_per_seq;
    nc += pkv::append_unchecked(alloc, row, num_computed[r], q, slot_mapping + t,
                                copies + 2 * nc);
    seq_request[s] = r;
    const int32_t ctx = num_computed[r] + q;
    context_lens[s] = ctx;
    const int32_t nb = (ctx + kBlock - 1) / kBlock;
    int32_t *out_row = block_tables + (size_t)s * max_blocks_per_seq;
    std::copy(row, row + nb, out_row);
    std::fill(out_row + nb, out_row + max_blocks_per_seq, -1);
    t += q;
    query_start_loc[++s] = t;
  }
  *num_seqs = s;
  *num_copies = nc;
  return PKV_OK;
}

}  // extern "C"
