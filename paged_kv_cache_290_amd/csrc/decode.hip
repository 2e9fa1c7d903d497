// Decode attention over the paged KV pool: one workgroup per (row, kv-head group)
// segment, its waves taking the segment's blocks in turn and merging their states in
// LDS; long segments are cut into a few key ranges whose partial results a merge
// kernel combines.
//
// Method (pages cited by title and section):
//  * Inference-engine page (xiaohu-jiedu), prefill/decode section: a decode step has
//    one new query per request and must read the whole cached context, so it is
//    bound by memory bandwidth, not arithmetic.
//  * Serving-engine KV page (ttlab), section 2, "blocks and block table": K/V sit in
//    16-token blocks anywhere in the pool; the kernel follows the request's block
//    table and must give the same result as a contiguous cache.
//
// Work decomposition.  A segment is (row, kv-head group g): the blocks one row reads
// for the HG query heads of group g.  Its blocks are cut into `splits` contiguous
// ranges (one unless a wave would get more than kBlocksPerWave blocks, or the
// segments alone cannot fill the GPU), one workgroup of NW waves per range; wave w
// takes blocks w, w+NW, w+2NW, ... of the range, so the waves of a workgroup stream
// within one block of each other whatever the segment's length.  The waves' online-
// softmax states meet in LDS at the end: with one range the workgroup writes the
// output itself (no scan over the batch, no second launch); with several each range
// leaves a normalised partial (o, log2-sum-exp) for the merge kernel.
//
// Per block a wave reads one contiguous (block, kv head) tile of K and of V (2-8 KB
// each) with 16-byte-per-lane raw buffer loads and uses it for all HG query heads
// (grouped-query reuse), keeping the next block in flight in a register ring while it
// computes one.  Softmax runs in log2 units (scores times scale*log2 e, exp2).  Every
// lane keeps running sums for its own tokens, all scaled by one wave-uniform reference
// max per head; the reference is raised only when some score exceeds it by more than
// kRescaleSlack (then every lane rescales), so the usual per-block cross-lane max is
// replaced by one ballot.  Terms stay below 2^kRescaleSlack, far from fp32 overflow.
//
// bf16 tiles with head_dim 64 run both products of a block on the matrix cores: the
// scores as S^T = K Q^T (v_mfma_f32_16x16x32_bf16: 16 tokens x 16 columns, the
// group's HG heads in the first columns), whose accumulator layout is the B operand
// layout of the second product O^T += V^T P^T (v_mfma_f32_16x16x16_bf16), so the
// weights stay in the lanes that computed them; V^T comes from the wave's V tile in
// LDS through transposing reads.  Each column keeps its own lazily raised reference.
// The other cases use packed bf16 dot products (v_dot2_f32_bf16) or fp32 FMAs.
#include <type_traits>

#include "decode_body.h"

namespace pkv {

template <typename T, int D, int HG, int NW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<T>(), decode_waves_per_simd<T>())))
void decode_kernel(AttnArgs a, SegArgs p) {
  using L = DecodeLds<T, D, HG, NW>;
  __shared__ typename L::Red s_red;
  __shared__ typename L::Pw s_pw;
  __shared__ typename L::V s_v;
  __shared__ typename L::O s_o;
  __shared__ typename L::Ml s_ml;
  const L sh{s_red, s_pw, s_v, s_o, s_ml};
  // Fused call: the launch stores every new row; each decode row's newest key and
  // value come from k_new / v_new.
  if (a.k_new != nullptr) fused_slot_write<T, D>(a, blockIdx.x, gridDim.x, 64 * NW);

  // Virtual order (g, item, split): the workgroups of one kv-head group sit on one
  // XCD, sharing its L2 for shared blocks.
  decode_segment<T, D, HG, NW>(a, p, xcd_remap(blockIdx.x, gridDim.x), sh);
}

// Log-sum-exp merge of the key ranges of each segment cut into several: with per-range
// (o_i, lse_i) in log2 units, out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M),
// M = max_i lse_i.  One wave per (segment, q head of its group).
template <typename T, int D, int HG>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a, SegArgs p) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int DW = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= p.items * p.groups * HG) return;
  const int hh = gw % HG;
  const int seg = gw / HG;
  const int g = seg / p.items;
  const int item = seg - g * p.items;
  int seq, row, keys;
  bool zero;
  if (!item_row<kF32>(a, item, seq, row, keys, zero) || zero) return;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = g / p.num_head_groups;
  const int h = kvh * group + (g - kvh * p.num_head_groups) * HG + hh;
  const size_t base = (size_t)seg * p.splits * HG + hh;  // range i: base + i * HG

  // One pass in batches of 16 ranges (indices past the end are clamped to the last
  // range and weighted 0): each batch's lse and o values are loaded together, and the
  // running sums are rescaled when the running maximum rises.
  constexpr int kBatch = 16;
  float M = -INFINITY, L = 0.f;
  float o[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
    float v[kBatch][DW];
    float lv[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = min(s0 + jj, p.splits - 1);
      const size_t slot = base + (size_t)j * HG;
      lv[jj] = p.ws_lse[slot];
      const float *src = p.ws_o + slot * D;
#pragma unroll
      for (int e = 0; e < DW; ++e) v[jj][e] = src[lane + 64 * e];
    }
    float bm = M;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      if (s0 + jj < p.splits) bm = fmaxf(bm, lv[jj]);
    if (bm == -INFINITY) continue;  // nothing with weight yet
    const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - bm);
    L *= r;
#pragma unroll
    for (int e = 0; e < DW; ++e) o[e] *= r;
    M = bm;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const float wj = (s0 + jj < p.splits && lv[jj] != -INFINITY) ? fast_exp2(lv[jj] - M) : 0.f;
      L += wj;
#pragma unroll
      for (int e = 0; e < DW; ++e) o[e] = fmaf(wj, v[jj][e], o[e]);
    }
  }
  T *out = static_cast<T *>(a.out) + ((size_t)row * a.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < DW; ++e) {
    const float res = (L > 0.f) ? o[e] / L : 0.f;
    if constexpr (kF32) out[lane + 64 * e] = res;
    else out[lane + 64 * e] = f32_to_bf16(res);
  }
}

SegArgs decode_seg_args(const DecodePlan &pl, int num_kv_heads) {
  SegArgs p{};
  p.items = pl.items;
  p.num_head_groups = pl.num_head_groups;
  p.groups = num_kv_heads * pl.num_head_groups;
  p.splits = pl.splits;
  p.skip_blocks = pl.skip_blocks;
  p.partials = (pl.splits > 1 || pl.cascade) ? 1 : 0;
  if (p.partials) {
    p.ws_o = reinterpret_cast<float *>(static_cast<char *>(pl.workspace) + pl.ws_o_offset);
    p.ws_lse = reinterpret_cast<float *>(static_cast<char *>(pl.workspace) + pl.ws_lse_offset);
  }
  return p;
}

template <typename T, int D, int HG>
static hipError_t launch_merge_t(const AttnArgs &a, const SegArgs &p, hipStream_t st) {
  const int64_t waves = (int64_t)p.items * p.groups * HG;
  merge_kernel<T, D, HG><<<dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                           st>>>(a, p);
  return hipGetLastError();
}

template <typename T, int D, int HG, int NW>
static hipError_t launch_decode_t(const AttnArgs &a, const DecodePlan &pl, hipStream_t st) {
  const SegArgs p = decode_seg_args(pl, a.num_kv_heads);
  const int64_t wgs = (int64_t)p.items * p.groups * p.splits;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  decode_kernel<T, D, HG, NW><<<dim3((unsigned)wgs), dim3(64 * NW), 0, st>>>(a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1 || pl.cascade) return e;
  return launch_merge_t<T, D, HG>(a, p, st);
}

template <typename T, int D, int HG>
static hipError_t launch_decode_w(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  if constexpr (!std::is_same<T, float>::value) {  // fp32 rows always take 8 waves
    if (p.waves == kDecodeWavesMax) return launch_decode_t<T, D, HG, kDecodeWavesMax>(a, p, st);
  }
  if (p.waves == kDecodeWavesMin) return launch_decode_t<T, D, HG, kDecodeWavesMin>(a, p, st);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_decode_d(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  // Only the head groups the planner can pick for this element type and head_dim.
  constexpr int kMaxHG = (512 / (D * (int)sizeof(T))) < 4 ? (512 / (D * (int)sizeof(T))) : 4;
  switch (p.head_group) {
    case 1: return launch_decode_w<T, D, 1>(a, p, st);
    case 2:
      if constexpr (kMaxHG >= 2) return launch_decode_w<T, D, 2>(a, p, st);
      break;
    case 4:
      if constexpr (kMaxHG >= 4) return launch_decode_w<T, D, 4>(a, p, st);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                               hipStream_t stream) {
  if (p.items == 0 || p.splits == 1 || p.cascade) return hipSuccess;
  if (dtype != PKV_BF16) return hipErrorInvalidValue;
  const SegArgs sp = decode_seg_args(p, a.num_kv_heads);
  if (a.head_dim == 64) {
    if (p.head_group == 4) return launch_merge_t<uint16_t, 64, 4>(a, sp, stream);
    if (p.head_group == 2) return launch_merge_t<uint16_t, 64, 2>(a, sp, stream);
    if (p.head_group == 1) return launch_merge_t<uint16_t, 64, 1>(a, sp, stream);
  } else if (a.head_dim == 128) {
    if (p.head_group == 2) return launch_merge_t<uint16_t, 128, 2>(a, sp, stream);
    if (p.head_group == 1) return launch_merge_t<uint16_t, 128, 1>(a, sp, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                         hipStream_t stream) {
  if (p.items == 0) return hipSuccess;
  if (dtype == PKV_F32) {
    if (a.head_dim == 64) return launch_decode_d<float, 64>(a, p, stream);
    if (a.head_dim == 128) return launch_decode_d<float, 128>(a, p, stream);
  } else {
    if (a.head_dim == 64) return launch_decode_d<uint16_t, 64>(a, p, stream);
    if (a.head_dim == 128) return launch_decode_d<uint16_t, 128>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
