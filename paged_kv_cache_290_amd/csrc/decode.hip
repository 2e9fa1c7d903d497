// Decode attention over the paged KV pool: balanced split-K (stream-K) over the
// context, then a log-sum-exp merge.
//
// Method (pages cited by title and section):
//  * Inference-engine page (xiaohu-jiedu), prefill/decode section: a decode step has
//    one new query per request and must read the whole cached context, so it is
//    bound by memory bandwidth, not arithmetic.
//  * Serving-engine KV page (ttlab), section 2, "blocks and block table": K/V sit in
//    16-token blocks anywhere in the pool; the kernel follows the request's block
//    table and must give the same result as a contiguous cache.
//
// Work decomposition.  A segment is (kv-head group g, row): the blocks one row must
// read for the HG query heads of group g.  All segments, concatenated in (g, row,
// block) order, form one sequence of T blocks.  The grid is persistent (a fixed
// number of workgroups per CU) and wave w of the W waves takes the contiguous range
// [w*T/W, (w+1)*T/W), so every wave streams the same number of blocks whatever the
// context lengths.  A segment that lies inside one wave is finished there; a segment
// cut across waves leaves one normalised partial (o, log2-sum-exp) per piece, in
// workspace slot (segment + wave), and the merge kernel combines them.  Slots of
// different segments never collide: segment s+1 starts at or after the last wave of
// segment s, so its slots start past segment s's.
//
// Per block a wave reads one contiguous (block, kv head) tile of K and of V (2-8 KB
// each) with 16-byte-per-lane raw buffer loads and uses it for all HG query heads
// (grouped-query reuse), keeping PF blocks in flight in a register ring while it
// computes one.  Softmax runs in log2 units (scores times scale*log2 e, exp2).  Every
// lane keeps running sums for its own tokens, all scaled by one wave-uniform reference
// max per head; the reference is raised only when some score exceeds it by more than
// kRescaleSlack (then every lane rescales), so the usual per-block cross-lane max is
// replaced by one ballot.  Terms stay below 2^kRescaleSlack, far from fp32 overflow.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Set-up cost of a segment (query load, flush of a partial) for the static split of the
// work, in K/V bytes streamed in the same time: measured best at 4-6 blocks of 4 KiB
// (d=64 bf16) and ~2 blocks of 8 KiB (d=128 bf16).
constexpr int kSegCostBytes = 20 * 1024;

constexpr float kRescaleSlack = 8.0f;

// Lane mapping for one (block, kv head) tile of 16 tokens x D elements, row R bytes.
// Load instruction j of a wave reads the tile's j-th contiguous KiB: lane l gets the
// 16 bytes at 1024*j + 16*l, i.e. chunk c = l % CPR (EPC elements) of token
// TPI*j + l / CPR.  A lane thus owns the same EPC dims of NV tokens, and each token's
// dot product is summed over its CPR lanes.
template <typename T, int D>
struct DecodeMap {
  static constexpr int R = D * (int)sizeof(T);  // bytes per token row
  static constexpr int CPR = R / 16;            // lanes (16-byte chunks) per token
  static constexpr int TPI = 64 / CPR;          // tokens per load instruction
  static constexpr int NV = 16 / TPI;           // load instructions per tile
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int WPC = 4;                 // dwords per chunk
};

// Sum over the CPR lanes of a token (lanes l with equal l / CPR).
template <int CPR>
__device__ __forceinline__ float sum_over_token_lanes(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if constexpr (CPR >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (CPR >= 16) x += dpp<kRowMirror>(x);
  if constexpr (CPR >= 32) x += shfl_xor(x, 16);
  return x;
}

// Sum over the lanes that own the same chunk (l % CPR equal), i.e. across tokens.
template <int CPR>
__device__ __forceinline__ float sum_over_chunk_lanes(float x) {
  if constexpr (CPR <= 8) x += dpp<kRowRor8>(x);
  if constexpr (CPR <= 16) x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

// v_perm_b32 selectors: (s0, s1) -> (s1.lo16, s0.lo16) and (s1.hi16, s0.hi16) (selector
// bytes 0-3 pick bytes of the second operand, 4-7 of the first).
constexpr uint32_t kPermLo = 0x05040100u;
constexpr uint32_t kPermHi = 0x07060302u;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

// Row geometry of work item `item`: the query row, its sequence, and how many keys it
// sees.  Items are sequences for bf16 (only single-query sequences are decode rows;
// chunks go to the MFMA kernel) and query rows for fp32.  `zero` marks rows that break
// q_len <= context_len, whose output is defined as zeros.
template <bool kRows>
__device__ __forceinline__ bool item_row(const AttnArgs &a, int item, int &seq, int &row,
                                         int &keys, bool &zero) {
  if constexpr (kRows) {
    row = item;
    seq = find_seq(a.query_start_loc, a.num_seqs, row);
  } else {
    seq = item;
    row = a.query_start_loc[seq];
    if (a.query_start_loc[seq + 1] - row != 1 || row < 0 || row >= a.total_q) return false;
  }
  const int q_begin = a.query_start_loc[seq];
  const int q_len = a.query_start_loc[seq + 1] - q_begin;
  const int ctx = a.context_lens[seq];
  zero = ctx < q_len;
  keys = zero ? 0 : min(ctx - q_len + (row - q_begin) + 1, a.max_blocks_per_seq * kBlock);
  return true;
}

// Per-item block counts -> exclusive prefix in LDS (s_pref[0..items], s_pref[items] =
// total), visible keys in s_keys, query row and sequence in s_row / s_seq.  Whole
// workgroup; ends with a barrier.
template <bool kRows>
__device__ __forceinline__ void scan_items(const AttnArgs &a, int base, int items,
                                           int skip_blocks, int *s_pref, int *s_keys,
                                           int *s_row, int *s_seq, int *s_tmp) {
  const int tid = threadIdx.x;
  const int per = (items + kThreads - 1) / kThreads;
  const int i0 = min(items, tid * per);
  const int i1 = min(items, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    int seq = 0, row = 0, keys;
    bool zero;
    if (!item_row<kRows>(a, base + i, seq, row, keys, zero)) keys = 0;
    s_keys[i] = keys;
    s_row[i] = row;
    s_seq[i] = seq;
    const int n = max((keys + kBlock - 1) / kBlock - skip_blocks, 0);
    s_pref[i] = n;
    local += n;
  }
  s_tmp[tid] = local;
  __syncthreads();
  if (tid < 64) {  // exclusive scan of the 256 thread totals by one wave
    int v0 = s_tmp[4 * tid], v1 = s_tmp[4 * tid + 1], v2 = s_tmp[4 * tid + 2],
        v3 = s_tmp[4 * tid + 3];
    const int sum = v0 + v1 + v2 + v3;
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
    int ex = incl - sum;
    s_tmp[4 * tid] = ex; ex += v0;
    s_tmp[4 * tid + 1] = ex; ex += v1;
    s_tmp[4 * tid + 2] = ex; ex += v2;
    s_tmp[4 * tid + 3] = ex; ex += v3;
    if (tid == 63) s_pref[items] = ex;
  }
  __syncthreads();
  int run = s_tmp[tid];
  for (int i = i0; i < i1; ++i) {
    const int n = s_pref[i];
    s_pref[i] = run;
    run += n;
  }
  __syncthreads();
}

template <typename T, int D, int HG, int PF>
__global__ __launch_bounds__(kThreads) void decode_streamk_kernel(AttnArgs a, StreamArgs p) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  using M = DecodeMap<T, D>;
  constexpr int CPR = M::CPR, TPI = M::TPI, NV = M::NV, EPC = M::EPC, WPC = M::WPC;
  constexpr int kTileBytes = kBlock * D * (int)sizeof(T);
  // Segment set-up cost in blocks (one block = a K tile and a V tile).
  constexpr int kSegCost =
      kSegCostBytes / (2 * kTileBytes) > 1 ? kSegCostBytes / (2 * kTileBytes) : 1;

  __shared__ int s_pref[kMaxStreamItems + 1];
  __shared__ int s_keys[kMaxStreamItems];
  __shared__ int s_row[kMaxStreamItems];
  __shared__ int s_seq[kMaxStreamItems];
  __shared__ int s_tmp[kThreads];
  // bf16 path: per wave and ring slot, partial scores [j*HG + hh][lane] and the bf16
  // weights [token group][head][j] exchanged between the lanes of the wave.
  constexpr int kRed = kF32 ? 1 : NV * HG * 64;
  constexpr int kPw = kF32 ? 1 : 16 * HG / 2;
  __shared__ float s_red[kWaves][PF + 1][kRed];
  __shared__ uint32_t s_pw[kWaves][PF + 1][kPw];

  if (a.k_new != nullptr && p.item_base == 0) {
    // Fused slot write of every new row (16-byte pieces spread over the grid); its
    // latency overlaps the item scan.  Nothing in this launch reads those slots.
    constexpr int kRowVecs = D * (int)sizeof(T) / 16;
    const int64_t total = (int64_t)a.total_q * a.num_kv_heads * kRowVecs;
    const int64_t per_token = (int64_t)a.num_kv_heads * kRowVecs;
    const int64_t num_slots = (int64_t)a.num_blocks * kBlock;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kThreads) {
      const int64_t t = idx / per_token;
      const int rem = (int)(idx - t * per_token);
      const int h = rem / kRowVecs;
      const int piece = rem - h * kRowVecs;
      const uint4 kx = static_cast<const uint4 *>(a.k_new)[idx];
      const uint4 vx = static_cast<const uint4 *>(a.v_new)[idx];
      const int64_t slot = a.slot_mapping[t];
      if (slot < 0 || slot >= num_slots) continue;
      const int64_t dst = ((slot / kBlock * a.num_kv_heads + h) * kBlock + slot % kBlock) *
                              kRowVecs + piece;
      static_cast<uint4 *>(const_cast<void *>(a.k_pool))[dst] = kx;
      static_cast<uint4 *>(const_cast<void *>(a.v_pool))[dst] = vx;
    }
  }
  scan_items<kF32>(a, p.item_base, p.items, p.skip_blocks, s_pref, s_keys, s_row, s_seq,
                   s_tmp);
  const int rows_total = s_pref[p.items];
  const int64_t T_all = (int64_t)rows_total * p.groups;
  // With fewer blocks than waves only the first T_all waves work.
  const int W = (int)min<int64_t>((int64_t)gridDim.x * kWaves, T_all);
  // The static split balances cost, not blocks: each segment costs its blocks plus
  // kSegCost block-equivalents of set-up (query load, a partial's flush), so a wave
  // whose range crosses segment starts gets fewer blocks.  In cost order a segment
  // (g, item) starts at g*rows_cost + s_pref[item] + kSegCost*item, and its block lb
  // sits at that start + kSegCost + lb.  Wave w owns the cost range
  // [w*T_cost/W, (w+1)*T_cost/W); its blocks stay one contiguous run in block order.
  const int64_t rows_cost = (int64_t)rows_total + (int64_t)kSegCost * p.items;
  const int64_t T_cost = rows_cost * p.groups;
  // Every product and quotient below fits in 31 bits for all but huge batches; then
  // the divisions run in 32-bit arithmetic (64-bit division is a long instruction
  // sequence on the GPU, and these sit on the path to the first block).
  const bool narrow = T_cost * (int64_t)(W + 1) < (int64_t)INT32_MAX;
  auto quot = [narrow](int64_t x, int64_t y) -> int64_t {
    return narrow ? (int64_t)((uint32_t)x / (uint32_t)y) : x / y;
  };
  auto wave_of_cost = [&](int64_t c) { return (int)quot((c + 1) * W - 1, T_cost); };
  // Blocks (in block order) whose cost position is below c (c wave-uniform).  The
  // item holding c is found with one LDS read and a ballot when there are at most 64
  // items (lane i tests item i), else by binary search.
  auto blocks_before = [&](int64_t c) -> int64_t {
    const int64_t g = quot(c, rows_cost);
    const int64_t cc = c - g * rows_cost;
    int lo;  // last item whose cost start is <= cc (item 0 starts at 0)
    if (p.items <= 64) {
      const int ln = threadIdx.x & 63;
      const bool le = ln < p.items && s_pref[ln] + (int64_t)kSegCost * ln <= cc;
      lo = 63 - __builtin_clzll(__builtin_amdgcn_ballot_w64(le));
    } else {
      lo = 0;
      int hi = p.items - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] + (int64_t)kSegCost * mid <= cc) lo = mid; else hi = mid - 1;
      }
    }
    const int64_t off = cc - (s_pref[lo] + (int64_t)kSegCost * lo);
    return g * rows_total + s_pref[lo] + (off > kSegCost ? off - kSegCost : 0);
  };
  if (blockIdx.x == 0) {
    // Rows of sequences that break q_len <= context_len: defined as zeros.
    for (int i = threadIdx.x; i < p.items; i += kThreads) {
      int seq, row, keys;
      bool zero;
      if (item_row<kF32>(a, p.item_base + i, seq, row, keys, zero) && zero)
        for (int e = 0; e < a.num_q_heads * D; ++e)
          static_cast<T *>(a.out)[(size_t)row * a.num_q_heads * D + e] = T(0);
    }
    // Per segment (g, item): first partial slot and piece count for the merge kernel
    // (0 pieces: nothing to merge, the segment was finished in one wave or is empty;
    // with all_partial a segment finished in one wave is one piece).
    for (int sg = threadIdx.x; sg < p.items * p.groups; sg += kThreads) {
      const int g = sg / p.items;
      const int item = sg - g * p.items;
      int first = 0, pieces = 0;
      if (s_pref[item + 1] > s_pref[item]) {
        const int64_t c0 = (int64_t)g * rows_cost + s_pref[item] + (int64_t)kSegCost * item +
                           kSegCost;  // cost position of the segment's first block
        const int w0 = wave_of_cost(c0);
        const int w1 = wave_of_cost(c0 + (s_pref[item + 1] - s_pref[item]) - 1);
        if (w1 > w0 || p.all_partial) {
          first = sg + w0;
          pieces = w1 - w0 + 1;
        }
      }
      p.seginfo[2 * sg] = first;
      p.seginfo[2 * sg + 1] = pieces;
    }
  }
  if (T_all == 0) return;

  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep everything
  // derived from it (block range, loop bounds, buffer descriptors) in scalar registers
  // instead of wrapping each buffer load in a loop over distinct descriptor values.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = lane % CPR;
  const int tok0 = lane / CPR;  // token of load j is TPI*j + tok0
  const int w = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave;
  if (w >= W) return;
  // The wave's blocks: [wb0, wb0 + nbw) in block order (possibly none).
  const int64_t wb0 = blocks_before(quot((int64_t)w * T_cost, W));
  const int nbw = (int)(blocks_before(quot((int64_t)(w + 1) * T_cost, W)) - wb0);
  if (nbw == 0) return;
  const int group = a.num_q_heads / a.num_kv_heads;
  const char *kpool = static_cast<const char *>(a.k_pool);
  const char *vpool = static_cast<const char *>(a.v_pool);
  const bool fused = !kF32 && a.k_new != nullptr;
  const char *knew = static_cast<const char *>(a.k_new);
  const char *vnew = static_cast<const char *>(a.v_new);

  // bf16: after the exchange lane `lane` < NSC owns the score of token tau_s (of the
  // current block) and head hh_s.  The softmax scale enters as |scale| with the sign
  // of a negative scale folded into q (exact for bf16).
  constexpr int NSC = 16 * HG;
  const int k_s = lane / TPI;
  const int j_s = k_s / HG;
  const int hh_s = k_s - j_s * HG;
  const int tau_s = TPI * j_s + (lane - k_s * TPI);
  const bool scoring = lane < NSC;
  const float sc = fabsf(a.scale_log2);
  const uint32_t qflip = (!kF32 && a.scale_log2 < 0.f) ? 0x80008000u : 0u;

  // State of the open piece (the wave's blocks of one segment).
  uint32_t qw[HG][WPC];  // its query fragment: this lane's EPC dims of each head
  uint32_t qn[HG][WPC];  // query fragment prefetched for the next piece
  int qn_block = -1;     // wave block at which that next piece starts
  float acc[HG][EPC];
  float lsum[HG];   // fp32: per head, over this lane's tokens
  float mref[HG];   // reference max per head (wave-uniform)
  float my_m = -INFINITY;  // bf16: mref of this lane's score head
  float my_l = 0.f;        // bf16: this lane's share of its head's weight sum
  bool pc_open = false, pc_whole = false;
  int pc_row = 0, pc_h0 = 0, pc_keys = 0, pc_seg = 0;

  auto load_q = [&](uint32_t (&dst)[HG][WPC], int row, int h0) {
    const T *qp = static_cast<const T *>(a.q) + ((size_t)row * a.num_q_heads + h0) * D +
                  chunk * EPC;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const uint4 x = *reinterpret_cast<const uint4 *>(qp + hh * D);
      dst[hh][0] = x.x ^ qflip; dst[hh][1] = x.y ^ qflip;
      dst[hh][2] = x.z ^ qflip; dst[hh][3] = x.w ^ qflip;
    }
  };
  auto head0 = [&](int g) {
    const int kvh = g / p.num_head_groups;
    return kvh * group + (g - kvh * p.num_head_groups) * HG;
  };

  // Totals of the open piece: the whole segment goes straight to `out`, a part of one
  // to its partial slot (normalised o and log2-sum-exp per head).
  auto flush = [&]() {
    if constexpr (!kF32) {
      // bf16: the weight sum of head hh is spread over the lanes that scored it.
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) lsum[hh] = wave_sum((scoring && hh_s == hh) ? my_l : 0.f);
    }
    // fp32: each token's weight was counted on all CPR lanes of the token; summing over
    // the lanes of one chunk (one per token group) gives the piece's totals.  The
    // accumulators of both paths hold one chunk's dims per lane and token group.
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      if constexpr (kF32) lsum[hh] = sum_over_chunk_lanes<CPR>(lsum[hh]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[hh][e] = sum_over_chunk_lanes<CPR>(acc[hh][e]);
    }
    if (lane < CPR) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float inv = lsum[hh] > 0.f ? 1.f / lsum[hh] : 0.f;
        if (pc_whole) {
          T *dst = static_cast<T *>(a.out) +
                   ((size_t)pc_row * a.num_q_heads + pc_h0 + hh) * D + chunk * EPC;
          if constexpr (kF32) {
            *reinterpret_cast<float4 *>(dst) =
                float4{acc[hh][0] * inv, acc[hh][1] * inv, acc[hh][2] * inv, acc[hh][3] * inv};
          } else {
            uint4 pk;
            pk.x = pack_bf16x2(acc[hh][0] * inv, acc[hh][1] * inv);
            pk.y = pack_bf16x2(acc[hh][2] * inv, acc[hh][3] * inv);
            pk.z = pack_bf16x2(acc[hh][4] * inv, acc[hh][5] * inv);
            pk.w = pack_bf16x2(acc[hh][6] * inv, acc[hh][7] * inv);
            *reinterpret_cast<uint4 *>(dst) = pk;
          }
        } else {
          const size_t slot = (size_t)(pc_seg + w) * HG + hh;
          float *dst = p.ws_o + slot * D + chunk * EPC;
#pragma unroll
          for (int e = 0; e < EPC; e += 4)
            *reinterpret_cast<float4 *>(dst + e) =
                float4{acc[hh][e] * inv, acc[hh][e + 1] * inv, acc[hh][e + 2] * inv,
                       acc[hh][e + 3] * inv};
          if (lane == 0)
            p.ws_lse[slot] =
                lsum[hh] > 0.f ? mref[hh] + __builtin_amdgcn_logf(lsum[hh]) : -INFINITY;
        }
      }
    }
  };

  for (int c0 = 0; c0 < nbw; c0 += 64) {
    const int nc = min(64, nbw - c0);
    // Lane i describes wave block c0 + i: its kv-head group g, item, logical block and
    // physical block (invalid table entries read block 0 and are masked).  All table
    // entries of the chunk are fetched at once, whatever pieces the chunk spans.
    int m_g = 0, m_item = 0, m_lb = 0, m_pb = 0, m_ok = 0, m_keys = 0;
    // Item of the chunk's first block (last item with s_pref[item] <= r): a ballot
    // over lanes for up to 64 items, else a binary search.  Each lane then walks
    // forward from it to its own block's item; a chunk spans few items, and a lane
    // already in the next kv-head group starts from item 0 near that group's start.
    const int64_t b_first = wb0 + c0;
    const int g_first = (int)quot(b_first, rows_total);
    const int r_first = (int)(b_first - (int64_t)g_first * rows_total);
    int it0;
    if (p.items <= 64) {
      it0 = 63 - __builtin_clzll(
                     __builtin_amdgcn_ballot_w64(lane < p.items && s_pref[lane] <= r_first));
    } else {
      int lo = 0, hi = p.items - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= r_first) lo = mid; else hi = mid - 1;
      }
      it0 = lo;
    }
    if (lane < nc) {
      const int64_t bi = wb0 + c0 + lane;
      m_g = (int)quot(bi, rows_total);
      const int r = (int)(bi - (int64_t)m_g * rows_total);
      int lo = m_g == g_first ? it0 : 0;  // last item with s_pref[item] <= r
      while (lo + 1 < p.items && s_pref[lo + 1] <= r) ++lo;
      m_item = lo;
      m_lb = r - s_pref[lo] + p.skip_blocks;
      m_keys = s_keys[lo];
      const int pb = a.block_tables[(size_t)s_seq[lo] * a.max_blocks_per_seq + m_lb];
      m_ok = pb >= 0 && pb < a.num_blocks;
      m_pb = m_ok ? pb : 0;
    }
    // Pieces start at a segment's first block, and at the wave's first block.
    uint64_t starts = __builtin_amdgcn_ballot_w64(lane < nc && m_lb == p.skip_blocks);
    if (c0 == 0) starts |= 1ull;

    // Raw buffer loads through a per-tile descriptor.  Prefetches past the chunk (and
    // tiles of invalid table entries) get a descriptor with no records: those loads
    // fetch nothing and return zeros, yet every path issues the same number of
    // loads, so the compiler's wait counts stay exact.
    auto load = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], uint4 &kn, uint4 &vn, int i) {
      const int ic = min(i, nc - 1);
      const int pb = readlane(m_pb, ic);
      const bool ok = i < nc && readlane(m_ok, ic) != 0;
      const int kvh = readlane(m_g, ic) / p.num_head_groups;
      const size_t off = ((size_t)pb * a.num_kv_heads + kvh) * kTileBytes;
      const int nrec = ok ? kTileBytes : 0;
      const buffer_rsrc_t rk = make_rsrc(kpool + off, nrec);
      const buffer_rsrc_t rv = make_rsrc(vpool + off, nrec);
#pragma unroll
      for (int j = 0; j < NV; ++j) kr[j] = buffer_load16(rk, 1024 * j + 16 * lane);
#pragma unroll
      for (int j = 0; j < NV; ++j) vr[j] = buffer_load16(rv, 1024 * j + 16 * lane);
      if constexpr (!kF32) {
        // Fused write: the lanes of a decode row's newest token (in its last block) also
        // fetch that row from k_new / v_new; every other lane's offset is out of range,
        // so the load fetches nothing (issued on every block to keep wait counts exact).
        const int keys = readlane(m_keys, ic);
        const int lb = readlane(m_lb, ic);
        const int row = s_row[readlane(m_item, ic)];
        const bool has_new = fused && i < nc && (keys - 1) / kBlock == lb;
        const bool mine = has_new && (keys - 1) % TPI == tok0;
        const size_t noff = ((size_t)row * a.num_kv_heads + kvh) * D * sizeof(T);
        const buffer_rsrc_t rkn = make_rsrc(knew + noff, has_new ? D * (int)sizeof(T) : 0);
        const buffer_rsrc_t rvn = make_rsrc(vnew + noff, has_new ? D * (int)sizeof(T) : 0);
        const int o = mine ? 16 * chunk : D * (int)sizeof(T);
        kn = buffer_load16(rkn, o);
        vn = buffer_load16(rvn, o);
      }
    };

    // A new piece at chunk block i: flush the open one, set up the new one, and
    // prefetch the query of the piece after it (if that one starts in this chunk).
    auto begin_piece = [&](int i) {
      if (pc_open) flush();
      const int g = readlane(m_g, i);
      const int item = readlane(m_item, i);
      const int lb0 = readlane(m_lb, i) - p.skip_blocks;  // first block, counted from the skip
      pc_row = s_row[item];
      pc_keys = s_keys[item];
      pc_h0 = head0(g);
      pc_seg = g * p.items + item;
      const int n_item = s_pref[item + 1] - s_pref[item];
      const int len = min(n_item - lb0, nbw - (c0 + i));
      pc_whole = !p.all_partial && lb0 == 0 && len == n_item;
      pc_open = true;
      if (qn_block == c0 + i) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
#pragma unroll
          for (int k = 0; k < WPC; ++k) qw[hh][k] = qn[hh][k];
      } else {
        load_q(qw, pc_row, pc_h0);
      }
      if constexpr (kF32) {  // fold the softmax scale into q once
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
#pragma unroll
          for (int k = 0; k < WPC; ++k)
            qw[hh][k] = __float_as_uint(__uint_as_float(qw[hh][k]) * a.scale_log2);
      }
      const uint64_t later = i < 63 ? starts & (~0ull << (i + 1)) : 0ull;
      if (later) {
        const int j = __builtin_ctzll(later);
        const int gj = readlane(m_g, j);
        load_q(qn, s_row[readlane(m_item, j)], head0(gj));
        qn_block = c0 + j;
      }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        lsum[hh] = 0.f;
        mref[hh] = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
      }
      my_m = -INFINITY;
      my_l = 0.f;
    };

    // bf16 block update.  Each lane forms the partial dot products of its chunk for
    // its NV tokens and HG heads and parks them in LDS; lane `lane` < NSC then adds the
    // CPR partials of one (token, head) score, so the softmax work (scale, mask, exp)
    // is done once per score.  The weights go back through LDS as bf16, laid out so a
    // lane reads its token pairs as packed words and P.V is one dot2 per (head, dim,
    // token pair).  The denominator sums the same rounded weights.
    auto compute_bf16 = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], const uint4 &kn,
                            const uint4 &vn, int i, int u) {
      const int lb = readlane(m_lb, i);
      const bool bad = readlane(m_ok, i) == 0;
      const int keys = pc_keys;
      float *red = s_red[wave][u];
      uint32_t *pw = s_pw[wave][u];
      if (fused && (keys - 1) / kBlock == lb) {
        // The newest token (position keys-1) comes from k_new / v_new, not the pool.
        const int jn = ((keys - 1) % kBlock) / TPI;
        const bool mine = (keys - 1) % TPI == tok0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (j == jn && mine) {
            kr[j] = kn;
            vr[j] = vn;
          }
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float x = 0.f;
#pragma unroll
          for (int k = 0; k < WPC; ++k) x = dot2_bf16(qw[hh][k], kw[k], x);
          red[(j * HG + hh) * 64 + lane] = x;
        }
      }
      float xs = -INFINITY;
      if (scoring) {
        const float4 *src = reinterpret_cast<const float4 *>(red + lane * CPR);
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < CPR / 4; ++c) {
          const float4 v4 = src[c];
          x += (v4.x + v4.y) + (v4.z + v4.w);
        }
        if (!bad && lb * kBlock + tau_s < keys) xs = x * sc;
      }
      if (wave_any(xs > my_m + kRescaleSlack)) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          const float mn = fmaxf(mref[hh], wave_max(hh_s == hh ? xs : -INFINITY));
          const float alpha = (mref[hh] == -INFINITY) ? 0.f : fast_exp2(mref[hh] - mn);
          mref[hh] = mn;
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[hh][e] *= alpha;
          if (hh_s == hh) {
            my_l *= alpha;
            my_m = mn;
          }
        }
      }
      if (scoring) {
        const float pr = (xs == -INFINITY) ? 0.f : fast_exp2(xs - my_m);
        const uint16_t pb = f32_to_bf16(pr);
        my_l += __uint_as_float((uint32_t)pb << 16);
        reinterpret_cast<uint16_t *>(pw)[((tau_s % TPI) * HG + hh_s) * NV + tau_s / TPI] = pb;
      }
      // Slots past the context (and tiles of invalid blocks) may hold anything,
      // including NaN: their weight is 0 and their values are replaced by 0.
      const bool edge = bad || (lb + 1) * kBlock > keys;
      uint32_t vw[NV][4];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        vw[j][0] = vr[j].x; vw[j][1] = vr[j].y; vw[j][2] = vr[j].z; vw[j][3] = vr[j].w;
        if (edge) {
          const bool valid = !bad && lb * kBlock + TPI * j + tok0 < keys;
#pragma unroll
          for (int k = 0; k < 4; ++k) vw[j][k] = valid ? vw[j][k] : 0u;
        }
      }
      // Weights of this lane's tokens: word (hh, jp) = (p[TPI*2jp + tok0], p[TPI*(2jp+1)
      // + tok0]) of head hh.
      uint32_t pp[HG][NV / 2];
      {
        const uint32_t *src = pw + tok0 * (HG * NV / 2);
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
#pragma unroll
          for (int jp = 0; jp < NV / 2; ++jp) pp[hh][jp] = src[hh * (NV / 2) + jp];
      }
#pragma unroll
      for (int jp = 0; jp < NV / 2; ++jp) {
#pragma unroll
        for (int k = 0; k < WPC; ++k) {
          const uint32_t lo = __builtin_amdgcn_perm(vw[2 * jp + 1][k], vw[2 * jp][k], kPermLo);
          const uint32_t hi = __builtin_amdgcn_perm(vw[2 * jp + 1][k], vw[2 * jp][k], kPermHi);
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            acc[hh][2 * k] = dot2_bf16(pp[hh][jp], lo, acc[hh][2 * k]);
            acc[hh][2 * k + 1] = dot2_bf16(pp[hh][jp], hi, acc[hh][2 * k + 1]);
          }
        }
      }
    };

    auto compute = [&](const uint4 (&kr)[NV], const uint4 (&vr)[NV], int i) {
      const int lb = readlane(m_lb, i);
      const bool bad = readlane(m_ok, i) == 0;
      const int key0 = lb * kBlock + tok0;
      const int keys = pc_keys;
      float s[NV][HG];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float x = 0.f;
#pragma unroll
          for (int k = 0; k < WPC; ++k) {
            if constexpr (kF32)
              x = fmaf(__uint_as_float(qw[hh][k]), __uint_as_float(kw[k]), x);
            else
              x = dot2_bf16(qw[hh][k], kw[k], x);
          }
          s[j][hh] = x;
        }
      }
      bool need = false;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool valid = !bad && (key0 + TPI * j) < keys;
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float x = sum_over_token_lanes<CPR>(s[j][hh]);
          if constexpr (!kF32) x *= a.scale_log2;
          x = valid ? x : -INFINITY;
          s[j][hh] = x;
          need |= x > mref[hh] + kRescaleSlack;
        }
      }
      if (wave_any(need)) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float mx = s[0][hh];
#pragma unroll
          for (int j = 1; j < NV; ++j) mx = fmaxf(mx, s[j][hh]);
          const float mn = fmaxf(mref[hh], wave_max(mx));
          const float alpha = (mref[hh] == -INFINITY) ? 0.f : fast_exp2(mref[hh] - mn);
          mref[hh] = mn;
          lsum[hh] *= alpha;
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[hh][e] *= alpha;
        }
      }
      // Slots past the context (and tiles of invalid blocks) may hold anything,
      // including NaN: their weight is 0 and their values are replaced by 0.
      const bool edge = bad || (lb + 1) * kBlock > keys;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool valid = !bad && (key0 + TPI * j) < keys;
        uint32_t vw[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
        if (edge) {
#pragma unroll
          for (int k = 0; k < 4; ++k) vw[k] = valid ? vw[k] : 0u;
        }
        float pr[HG];
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          pr[hh] = valid ? fast_exp2(s[j][hh] - mref[hh]) : 0.f;
          lsum[hh] += pr[hh];
        }
#pragma unroll
        for (int k = 0; k < WPC; ++k) {
          if constexpr (kF32) {
            const float x = __uint_as_float(vw[k]);
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) acc[hh][k] = fmaf(pr[hh], x, acc[hh][k]);
          } else {
            const float lo = bf16_lo(vw[k]);
            const float hi = bf16_hi(vw[k]);
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
              acc[hh][2 * k] = fmaf(pr[hh], lo, acc[hh][2 * k]);
              acc[hh][2 * k + 1] = fmaf(pr[hh], hi, acc[hh][2 * k + 1]);
            }
          }
        }
      }
    };

    // Ring of PF+1 register buffers: while block i is computed, blocks i+1..i+PF are
    // in flight, across piece boundaries.
    uint4 kb[PF + 1][NV], vb[PF + 1][NV], knb[PF + 1], vnb[PF + 1];
#pragma unroll
    for (int q = 0; q < PF; ++q) load(kb[q], vb[q], knb[q], vnb[q], q);
    for (int i0 = 0; i0 < nc; i0 += PF + 1) {
#pragma unroll
      for (int u = 0; u <= PF; ++u) {
        const int un = (u + PF) % (PF + 1);
        load(kb[un], vb[un], knb[un], vnb[un], i0 + u + PF);
        const int i = i0 + u;
        if (i < nc) {
          if ((starts >> i) & 1ull) begin_piece(i);
          if constexpr (kF32)
            compute(kb[u], vb[u], i);
          else
            compute_bf16(kb[u], vb[u], knb[u], vnb[u], i, u);
        }
      }
    }
  }
  if (pc_open) flush();
}

// Log-sum-exp merge of the pieces of each segment cut across waves: with per-piece
// (o_i, lse_i) in log2 units, out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M),
// M = max_i lse_i.  One wave per (segment, q head of its group); the decode kernel
// left each segment's first slot and piece count in `seginfo`.
template <typename T, int D, int HG>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a, StreamArgs p) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int DW = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= p.items * p.groups * HG) return;
  const int hh = gw % HG;
  const int seg = gw / HG;
  const int g = seg / p.items;
  const int item = seg - g * p.items;
  // The output row's lookup does not depend on the piece info; it is made to complete
  // before the branch on that info (the empty asm uses it), so that both round trips
  // overlap instead of the lookup following the branch.
  int seq, row, keys;
  bool zero;
  item_row<kF32>(a, p.item_base + item, seq, row, keys, zero);
  const int first = p.seginfo[2 * seg];
  const int npieces = p.seginfo[2 * seg + 1];
  asm volatile("" ::"s"(row));
  if (npieces == 0) return;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = g / p.num_head_groups;
  const int h = kvh * group + (g - kvh * p.num_head_groups) * HG + hh;
  const size_t base = (size_t)first * HG + hh;  // slot of piece i: base + i * HG

  // One pass in batches of 16 pieces (indices past the end are clamped to the last
  // piece and weighted 0): each batch's lse and o values are loaded together, and the
  // running sums are rescaled when the running maximum rises.
  constexpr int kBatch = 16;
  float M = -INFINITY, L = 0.f;
  float o[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < npieces; s0 += kBatch) {
    float v[kBatch][DW];
    float lv[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = min(s0 + jj, npieces - 1);
      const size_t slot = base + (size_t)j * HG;
      lv[jj] = p.ws_lse[slot];
      const float *src = p.ws_o + slot * D;
#pragma unroll
      for (int e = 0; e < DW; ++e) v[jj][e] = src[lane + 64 * e];
    }
    float bm = M;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      if (s0 + jj < npieces) bm = fmaxf(bm, lv[jj]);
    if (bm == -INFINITY) continue;  // nothing with weight yet
    const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - bm);
    L *= r;
#pragma unroll
    for (int e = 0; e < DW; ++e) o[e] *= r;
    M = bm;
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const float wj = (s0 + jj < npieces && lv[jj] != -INFINITY) ? fast_exp2(lv[jj] - M) : 0.f;
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

template <typename T, int D, int HG, int PF>
static hipError_t launch_decode_t(const AttnArgs &a, const DecodePlan &pl, hipStream_t st) {
  for (int base = 0; base < pl.items; base += kMaxStreamItems) {
    StreamArgs p{};
    p.item_base = base;
    p.items = min(kMaxStreamItems, pl.items - base);
    p.num_head_groups = pl.num_head_groups;
    p.groups = a.num_kv_heads * pl.num_head_groups;
    p.ws_o = reinterpret_cast<float *>(static_cast<char *>(pl.workspace) + pl.ws_o_offset);
    p.ws_lse = reinterpret_cast<float *>(static_cast<char *>(pl.workspace) + pl.ws_lse_offset);
    p.seginfo =
        reinterpret_cast<int *>(static_cast<char *>(pl.workspace) + pl.ws_seginfo_offset);
    p.skip_blocks = pl.skip_blocks;
    p.all_partial = pl.cascade ? 1 : 0;

    decode_streamk_kernel<T, D, HG, PF><<<dim3(pl.grid), dim3(kThreads), 0, st>>>(a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pl.cascade) continue;  // one launch (at most kMaxStreamItems rows); merged later
    const int waves = p.items * p.groups * HG;
    merge_kernel<T, D, HG><<<dim3((waves + kWaves - 1) / kWaves), dim3(kThreads), 0, st>>>(
        a, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D, int HG>
static hipError_t launch_decode_p(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  if (p.prefetch != 1) return hipErrorInvalidValue;
  return launch_decode_t<T, D, HG, 1>(a, p, st);
}

template <typename T, int D>
static hipError_t launch_decode_d(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  // Only the head groups the planner can pick for this element type and head_dim.
  constexpr int kMaxHG = (512 / (D * (int)sizeof(T))) < 4 ? (512 / (D * (int)sizeof(T))) : 4;
  switch (p.head_group) {
    case 1: return launch_decode_p<T, D, 1>(a, p, st);
    case 2:
      if constexpr (kMaxHG >= 2) return launch_decode_p<T, D, 2>(a, p, st);
      break;
    case 4:
      if constexpr (kMaxHG >= 4) return launch_decode_p<T, D, 4>(a, p, st);
      break;
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
