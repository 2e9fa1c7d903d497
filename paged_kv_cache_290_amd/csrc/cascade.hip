// Merge step of shared-prefix attention: every decode row's output from the partial
// results of its private keys (the decode kernel's pieces) and of the shared run (the
// shared-run pass's key splits).
//
// Method (pages cited by title and section):
//  * Serving-engine KV page (ttlab), section 2, "block sharing", and section 4 (prefix
//    cache): requests with a common prefix name the same physical blocks in their
//    tables.  Attention over the whole context is then the log-sum-exp combination of
//    attention over the shared blocks and attention over each request's own blocks,
//    so the shared blocks can be read once for all requests.
//  * With per-part (o_i, lse_i) in log2 units, the row's output is
//    sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

struct CascadeArgs {
  // key ranges of the private keys (the decode kernel's partials)
  const float *dec_o;    // [segment][range][dec_hg][D]
  const float *dec_lse;  // [segment][range][dec_hg]
  int dec_hg, dec_nhg;   // query heads per decode segment, segments per kv head
  int dec_splits;        // ranges per segment
  // shared-run splits
  const float *sh_o;     // [tile][split][column][D]
  const float *sh_lse;   // [tile][split][column]
  int sh_hg, sh_nhg, sh_splits;
};

constexpr int kBatch = 8;  // parts whose loads are issued together

}  // namespace

// One wave per (decode row, q head); lane l owns dims l + 64*e.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void cascade_merge_kernel(AttnArgs a, CascadeArgs c) {
  constexpr int DW = D / 64;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= a.num_seqs * a.num_q_heads) return;
  const int item = gw / a.num_q_heads;  // the sequence (one decode row each)
  const int h = gw - item * a.num_q_heads;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / group;
  const int w = h - kvh * group;
  // Private ranges: segment (decode head group, item), range i at slot dbase + i*hg.
  const int seg = (kvh * c.dec_nhg + w / c.dec_hg) * a.num_seqs + item;
  const int npieces = c.dec_splits;
  const int row = a.query_start_loc[item];
  const int q_len = a.query_start_loc[item + 1] - row;
  const int ctx = a.context_lens[item];
  if (q_len != 1 || row < 0 || row >= a.total_q) return;
  T *out = static_cast<T *>(a.out) + ((size_t)row * a.num_q_heads + h) * D;
  if (ctx < q_len) {  // precondition broken: defined as zeros
#pragma unroll
    for (int e = 0; e < DW; ++e) out[lane + 64 * e] = T(0);
    return;
  }
  const size_t dbase = (size_t)seg * c.dec_splits * c.dec_hg + (w % c.dec_hg);
  // Shared splits: the row is column (w % sh_hg) * bm + row % bm of row tile row / bm.
  const int bm = kPrefillCols / c.sh_hg;
  const int tile = prefill_tile_index(row / bm, kvh * c.sh_nhg + w / c.sh_hg,
                                      a.num_kv_heads * c.sh_nhg);
  const size_t sbase = (size_t)tile * c.sh_splits * kPrefillCols + (w % c.sh_hg) * bm + row % bm;
  const int nparts = npieces + c.sh_splits;

  // One pass in batches: each batch's lse and o values are loaded together, and the
  // running sums are rescaled when the running maximum rises.  Part j < npieces is a
  // private piece, the others are shared splits.
  float M = -INFINITY, L = 0.f;
  float o[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) o[e] = 0.f;
  for (int j0 = 0; j0 < nparts; j0 += kBatch) {
    float v[kBatch][DW];
    float lv[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = min(j0 + jj, nparts - 1);
      const float *src;
      if (j < npieces) {
        const size_t slot = dbase + (size_t)j * c.dec_hg;
        lv[jj] = c.dec_lse[slot];
        src = c.dec_o + slot * D;
      } else {
        const size_t pc = sbase + (size_t)(j - npieces) * kPrefillCols;
        lv[jj] = c.sh_lse[pc];
        src = c.sh_o + pc * D;
      }
#pragma unroll
      for (int e = 0; e < DW; ++e) v[jj][e] = src[lane + 64 * e];
    }
    float bm_ = M;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      if (j0 + jj < nparts) bm_ = fmaxf(bm_, lv[jj]);
    if (bm_ == -INFINITY) continue;  // nothing with weight yet
    const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - bm_);
    L *= r;
#pragma unroll
    for (int e = 0; e < DW; ++e) o[e] *= r;
    M = bm_;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      // Unused or empty parts weigh 0 (their values may be anything, even NaN).
      const bool use = j0 + jj < nparts && lv[jj] != -INFINITY;
      const float wj = use ? fast_exp2(lv[jj] - M) : 0.f;
      L += wj;
#pragma unroll
      for (int e = 0; e < DW; ++e) o[e] = use ? fmaf(wj, v[jj][e], o[e]) : o[e];
    }
  }
#pragma unroll
  for (int e = 0; e < DW; ++e) {
    const float res = (L > 0.f) ? o[e] / L : 0.f;
    if constexpr (std::is_same<T, float>::value) out[lane + 64 * e] = res;
    else out[lane + 64 * e] = f32_to_bf16(res);
  }
}

hipError_t launch_cascade_merge(const AttnArgs &a, const DecodePlan &dp, const PrefillPlan &sp,
                                hipStream_t stream) {
  CascadeArgs c{};
  char *dw = static_cast<char *>(dp.workspace);
  c.dec_o = reinterpret_cast<const float *>(dw + dp.ws_o_offset);
  c.dec_lse = reinterpret_cast<const float *>(dw + dp.ws_lse_offset);
  c.dec_hg = dp.head_group;
  c.dec_nhg = dp.num_head_groups;
  c.dec_splits = dp.splits;
  char *sw = static_cast<char *>(sp.workspace);
  c.sh_o = reinterpret_cast<const float *>(sw + sp.ws_o_offset);
  c.sh_lse = reinterpret_cast<const float *>(sw + sp.ws_lse_offset);
  c.sh_hg = sp.head_group;
  c.sh_nhg = sp.num_head_groups;
  c.sh_splits = sp.splits;
  const int waves = a.num_seqs * a.num_q_heads;
  const dim3 grid((waves + kWaves - 1) / kWaves);
  if (a.head_dim == 64)
    cascade_merge_kernel<uint16_t, 64><<<grid, dim3(kThreads), 0, stream>>>(a, c);
  else if (a.head_dim == 128)
    cascade_merge_kernel<uint16_t, 128><<<grid, dim3(kThreads), 0, stream>>>(a, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
