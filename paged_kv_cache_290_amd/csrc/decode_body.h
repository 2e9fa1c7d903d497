// Decode attention of one segment key range by one workgroup: the body of the decode
// kernel, also run by the workgroups of the mixed launch that follow the chunk tiles.
// Design and the pages it follows are described in decode.hip.
#pragma once
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

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

// Matrix-core path (bf16, head_dim 64), lane l = 16 * lg + l16.  MFMA operand layout:
// A row l16 and B column l16 each hold the k-slots (lg, e); the accumulator holds rows
// 4 lg .. 4 lg + 3 of column l16.  K tiles are loaded straight into A fragments
// (token l16, dims 32 j + 8 lg .. + 7 for load j); V tiles go to LDS row-major, each
// row's 32-byte chunk pairs permuted by vslot so that the 8 rows that one transposing
// read pass touches fall on distinct banks.
template <int D>
__device__ __forceinline__ int vslot(int t, int c) {
  const int f = D == 64 ? ((t >> 1) & 3) : (t & 7);
  return c ^ (2 * f);
}

__device__ __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_k16(v4i16_t a, v4i16_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

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


// Waves per SIMD the decode kernel is compiled for: bf16 rows four (128 registers
// each: one 16-wave workgroup or two 8-wave workgroups per compute unit), fp32 rows two
// (their wider tiles need more registers per wave).
template <typename T>
constexpr int decode_waves_per_simd() {
  return std::is_same<T, float>::value ? 2 : 4;
}

// Fused slot write: every new row's key and value (D elements of T per kv head) stored
// at its slot, in 16-byte pieces spread over the workgroups of the calling launch
// (workgroup wg of nwg, nthr threads each).  Slots outside the pool are skipped.  The
// launch reads none of these slots from the pool: the attention work of the same
// launch takes this step's keys and values from k_new / v_new.
template <typename T, int D>
__device__ __forceinline__ void fused_slot_write(const AttnArgs &a, int64_t wg, int64_t nwg,
                                                 int nthr) {
  constexpr int kRowVecs = D * (int)sizeof(T) / 16;
  const int64_t total = (int64_t)a.total_q * a.num_kv_heads * kRowVecs;
  const int64_t per_token = (int64_t)a.num_kv_heads * kRowVecs;
  const int64_t num_slots = (int64_t)a.num_blocks * kBlock;
  for (int64_t idx = wg * nthr + threadIdx.x; idx < total; idx += nwg * nthr) {
    const int64_t t = idx / per_token;
    const int rem = (int)(idx - t * per_token);
    const int h = rem / kRowVecs;
    const int piece = rem - h * kRowVecs;
    const uint4 kx = static_cast<const uint4 *>(a.k_new)[idx];
    const uint4 vx = static_cast<const uint4 *>(a.v_new)[idx];
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t dst =
        ((slot / kBlock * a.num_kv_heads + h) * kBlock + slot % kBlock) * kRowVecs + piece;
    static_cast<uint4 *>(const_cast<void *>(a.k_pool))[dst] = kx;
    static_cast<uint4 *>(const_cast<void *>(a.v_pool))[dst] = vx;
  }
}

// LDS of one decode workgroup of NW waves.  bf16 dot-product path: per wave and ring
// slot, partial scores [j*HG + hh][lane] and the bf16 weights [token group][head][j]
// exchanged between the lanes of the wave; matrix-core path: each wave's current V
// tile (rows permuted by vslot); both: the waves' states for the merge (unnormalised
// outputs, reference max, weight sum).  The decode kernel declares the five arrays as
// __shared__ arrays of its own; the mixed launch lays them over its tile buffers.
template <typename T, int D, int HG, int NW>
struct DecodeLds {
  using M = DecodeMap<T, D>;
  static constexpr bool kF32 = std::is_same<T, float>::value;
  static constexpr bool kMfma = !kF32 && D == 64;
  static constexpr int PF = 1;
  static constexpr int kTileBytes = kBlock * D * (int)sizeof(T);
  static constexpr int kRed = (kF32 || kMfma) ? 1 : M::NV * HG * 64;
  static constexpr int kPw = (kF32 || kMfma) ? 1 : 16 * HG / 2;
  static constexpr int kV = kMfma ? NW * kTileBytes / 16 : 1;
  typedef float Red[NW][PF + 1][kRed];
  typedef uint32_t Pw[NW][PF + 1][kPw];
  typedef uint4 V[kV];
  typedef float O[NW][HG][D];
  typedef float Ml[NW][HG][2];
  Red &red;
  Pw &pw;
  V &v;
  O &o;
  Ml &ml;
  // Bytes of the five arrays laid out one after another (16-byte aligned each).
  static constexpr size_t bytes() {
    return al(sizeof(Red)) + al(sizeof(Pw)) + al(sizeof(V)) + al(sizeof(O)) + al(sizeof(Ml));
  }
  // The arrays laid out from `base` (16-byte aligned LDS of at least bytes()).
  static __device__ DecodeLds over(char *base) {
    char *p = base;
    Red &r = *reinterpret_cast<Red *>(p); p += al(sizeof(Red));
    Pw &w = *reinterpret_cast<Pw *>(p); p += al(sizeof(Pw));
    V &vv = *reinterpret_cast<V *>(p); p += al(sizeof(V));
    O &oo = *reinterpret_cast<O *>(p); p += al(sizeof(O));
    Ml &m = *reinterpret_cast<Ml *>(p);
    return DecodeLds{r, w, vv, oo, m};
  }
  static constexpr size_t al(size_t n) { return (n + 15) / 16 * 16; }
};

// The work of decode workgroup v (a segment's key range) by the calling workgroup of
// NW waves, with its LDS in `sh`.
template <typename T, int D, int HG, int NW>
__device__ __forceinline__ void decode_segment(AttnArgs a, SegArgs p, int64_t v,
                                               DecodeLds<T, D, HG, NW> sh) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  using M = DecodeMap<T, D>;
  constexpr int CPR = M::CPR, TPI = M::TPI, NV = M::NV, EPC = M::EPC, WPC = M::WPC;
  constexpr int kTileBytes = kBlock * D * (int)sizeof(T);
  constexpr int PF = 1;  // blocks in flight per wave while one is computed
  constexpr bool kMfma = !kF32 && D == 64;  // both products on the matrix cores
  constexpr int MT = D / 16;                // 16-dim tiles of O^T (matrix-core path)

  auto &s_red = sh.red;
  auto &s_pw = sh.pw;
  auto &s_v = sh.v;
  auto &s_o = sh.o;
  auto &s_ml = sh.ml;

  // Segment and range of virtual workgroup v (uniform over the workgroup, so every
  // early return below is taken by all its waves), in the order (g, item, split).
  const int64_t total_wg = (int64_t)p.items * p.groups * p.splits;
  if (v >= total_wg) return;
  const int split = (int)(v % p.splits);
  v /= p.splits;
  const int item = (int)(v % p.items);
  const int g = (int)(v / p.items);
  const int seg = g * p.items + item;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = g / p.num_head_groups;
  const int h0 = kvh * group + (g - kvh * p.num_head_groups) * HG;
  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep everything
  // derived from it in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = lane % CPR;
  const int tok0 = lane / CPR;  // token of load j is TPI*j + tok0
  const int l16 = lane & 15;    // matrix-core path: token (K) or column (head) of the lane
  const int lg = lane >> 4;
  const uint32_t qflip = (!kF32 && a.scale_log2 < 0.f) ? 0x80008000u : 0u;

  // bf16 items are sequences, so the table row is known before any load: with one key
  // range per segment this wave's first blocks are skip + wave + NW*i, and their table
  // entries are requested together with the row's lengths (one round trip less before
  // the first K/V request).  Likewise the query is fetched from row `item`, the row of
  // every sequence in a batch of decode rows only, and fetched again below if the
  // batch says otherwise.
  const bool early_tbl = !kF32 && p.splits == 1;
  int early_pb = 0;
  if (early_tbl) {
    const int lb = p.skip_blocks + wave + NW * lane;
    if (lb < a.max_blocks_per_seq)
      early_pb = a.block_tables[(size_t)item * a.max_blocks_per_seq + lb];
  }
  uint32_t qw[HG][WPC];
  auto load_q = [&](int r) {
    const T *qp = static_cast<const T *>(a.q) + ((size_t)r * a.num_q_heads + h0) * D +
                  chunk * EPC;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const uint4 x = *reinterpret_cast<const uint4 *>(qp + hh * D);
      qw[hh][0] = x.x ^ qflip; qw[hh][1] = x.y ^ qflip;
      qw[hh][2] = x.z ^ qflip; qw[hh][3] = x.w ^ qflip;
    }
  };
  // Matrix-core path: Q^T fragments, column l16 = head h0 + l16 (zeros past the group's
  // HG heads), dims 32 j + 8 lg .. + 7.
  uint4 qf[NV];
  auto load_qf = [&](int r) {
    const T *qp = static_cast<const T *>(a.q) +
                  ((size_t)r * a.num_q_heads + h0 + min(l16, HG - 1)) * D + 8 * lg;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint4 x = *reinterpret_cast<const uint4 *>(qp + 32 * j);
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      qf[j] = l16 < HG ? x : uint4{0u, 0u, 0u, 0u};
    }
  };
  const int row_guess = min(item, a.total_q - 1);
  if constexpr (kMfma) load_qf(row_guess);
  else if constexpr (!kF32) load_q(row_guess);

  int seq, row, keys;
  bool zero;
  if (!item_row<kF32>(a, item, seq, row, keys, zero)) return;  // not a decode row
  const size_t part = ((size_t)seg * p.splits + split) * HG;  // partial slot of head 0
  if (zero) {
    // Rows of sequences that break q_len <= context_len: defined as zeros.
    for (int e = threadIdx.x; e < HG * D; e += 64 * NW) {
      if (split == 0)
        static_cast<T *>(a.out)[((size_t)row * a.num_q_heads + h0) * D + e] = T(0);
      if (p.partials) {
        p.ws_o[part * D + e] = 0.f;
        if (e % D == 0) p.ws_lse[part + e / D] = -INFINITY;
      }
    }
    return;
  }
  const int nb = max((keys + kBlock - 1) / kBlock - p.skip_blocks, 0);
  const int b0 = p.skip_blocks + (int)((int64_t)split * nb / p.splits);
  const int b1 = p.skip_blocks + (int)((int64_t)(split + 1) * nb / p.splits);

  // This wave's blocks: b0 + wave + NW*i, i < nmine.
  const int nmine = b1 - b0 > wave ? (b1 - b0 - wave + NW - 1) / NW : 0;
  const char *kpool = static_cast<const char *>(a.k_pool);
  const char *vpool = static_cast<const char *>(a.v_pool);
  const bool fused = !kF32 && a.k_new != nullptr;
  const char *knew = static_cast<const char *>(a.k_new);
  const char *vnew = static_cast<const char *>(a.v_new);
  const int32_t *tbl = a.block_tables + (size_t)seq * a.max_blocks_per_seq;

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

  // Query fragment: this lane's EPC dims of each head (fp32: the scale folded in).
  if constexpr (kF32) {
    load_q(row);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int k = 0; k < WPC; ++k)
        qw[hh][k] = __float_as_uint(__uint_as_float(qw[hh][k]) * a.scale_log2);
  } else if (row != row_guess) {
    if constexpr (kMfma) load_qf(row);
    else load_q(row);
  }
  float acc[HG][EPC];
  float lsum[HG];   // fp32: per head, over this lane's tokens
  float mref[HG];   // reference max per head (wave-uniform)
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    lsum[hh] = 0.f;
    mref[hh] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
  }
  float my_m = -INFINITY;  // bf16: mref of this lane's score head (column)
  float my_l = 0.f;        // bf16: this lane's share of its head's weight sum
  float mneg = 0.f;        // matrix-core path: -my_m, or 0 while my_m is -inf
  f32x4_t oacc[kMfma ? MT : 1];  // matrix-core path: O^T tiles (dims 16 mt + 4 lg + r)
#pragma unroll
  for (int mt = 0; mt < (kMfma ? MT : 1); ++mt) oacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fused write: the row's newest token (position keys-1, in block lb_new) comes from
  // k_new / v_new, not the pool, which this launch is still writing.  The wave holding
  // that block loads it once; the lanes of that token get the row's 16-byte chunk, all
  // other loads are out of range and fetch nothing.
  const int lb_new = (keys - 1) / kBlock;
  uint4 kn{}, vn{};
  if constexpr (!kF32) {
    const bool has_new = fused && lb_new >= b0 && lb_new < b1 && (lb_new - b0) % NW == wave;
    const bool mine = has_new && (keys - 1) % TPI == tok0;
    const size_t noff = ((size_t)row * a.num_kv_heads + kvh) * D * sizeof(T);
    const buffer_rsrc_t rkn = make_rsrc(knew + noff, has_new ? D * (int)sizeof(T) : 0);
    const buffer_rsrc_t rvn = make_rsrc(vnew + noff, has_new ? D * (int)sizeof(T) : 0);
    const int o = mine ? 16 * chunk : D * (int)sizeof(T);
    kn = buffer_load16(rkn, o);
    vn = buffer_load16(rvn, o);
  }

  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int nc = min(64, nmine - c0);
    // Lane i looks up the table entry of this wave's block c0 + i (all at once);
    // invalid entries read block 0 and are masked.
    int m_lb = 0, m_pb = 0, m_ok = 0;
    if (lane < nc) {
      m_lb = b0 + wave + NW * (c0 + lane);
      const int pb = (early_tbl && c0 == 0) ? early_pb : tbl[m_lb];
      m_ok = pb >= 0 && pb < a.num_blocks;
      m_pb = m_ok ? pb : 0;
    }

    // Raw buffer loads through a per-tile descriptor.  Prefetches past the chunk (and
    // tiles of invalid table entries) get a descriptor with no records: those loads
    // fetch nothing and return zeros, yet every path issues the same number of
    // loads, so the compiler's wait counts stay exact.
    auto load = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], int i) {
      const int ic = min(i, nc - 1);
      const int pb = readlane(m_pb, ic);
      const bool ok = i < nc && readlane(m_ok, ic) != 0;
      const size_t off = ((size_t)pb * a.num_kv_heads + kvh) * kTileBytes;
      const int nrec = ok ? kTileBytes : 0;
      const buffer_rsrc_t rk = make_rsrc(kpool + off, nrec);
      const buffer_rsrc_t rv = make_rsrc(vpool + off, nrec);
#pragma unroll
      for (int j = 0; j < NV; ++j)
        kr[j] = buffer_load16(rk, kMfma ? l16 * M::R + 64 * j + 16 * lg : 1024 * j + 16 * lane);
#pragma unroll
      for (int j = 0; j < NV; ++j) vr[j] = buffer_load16(rv, 1024 * j + 16 * lane);
    };

    // bf16 block update.  Each lane forms the partial dot products of its chunk for
    // its NV tokens and HG heads and parks them in LDS; lane `lane` < NSC then adds the
    // CPR partials of one (token, head) score, so the softmax work (scale, mask, exp)
    // is done once per score.  The weights go back through LDS as bf16, laid out so a
    // lane reads its token pairs as packed words and P.V is one dot2 per (head, dim,
    // token pair).  The denominator sums the same rounded weights.
    auto compute_bf16 = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], int i, int u) {
      const int lb = readlane(m_lb, i);
      const bool bad = readlane(m_ok, i) == 0;
      float *red = s_red[wave][u];
      uint32_t *pw = s_pw[wave][u];
      if (fused && lb == lb_new) {
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

    // Matrix-core block update (bf16, head_dim 64).  The weights are rounded to bf16 for
    // P.V and the denominator sums the same rounded values.  Columns past the group's
    // heads score 0 and accumulate harmless sums that are never stored.
    auto compute_mfma = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], int i) {
      const int lb = readlane(m_lb, i);
      const bool bad = readlane(m_ok, i) == 0;
      char *vt = reinterpret_cast<char *>(s_v) + wave * kTileBytes;
      if (fused && lb == lb_new) {
        // The newest token comes from k_new / v_new, not the pool.  Its K chunks sit in
        // the lanes of kn that load it (token tn % TPI of the load layout); the A-layout
        // lanes of token tn fetch them from there.
        const int tn = (keys - 1) % kBlock;
        const int src = (tn % TPI) * CPR;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int sl = (src + 4 * j + lg) * 4;
          uint4 x;
          x.x = __builtin_amdgcn_ds_bpermute(sl, (int)kn.x);
          x.y = __builtin_amdgcn_ds_bpermute(sl, (int)kn.y);
          x.z = __builtin_amdgcn_ds_bpermute(sl, (int)kn.z);
          x.w = __builtin_amdgcn_ds_bpermute(sl, (int)kn.w);
          if (l16 == tn) kr[j] = x;
        }
        const int jn = tn / TPI;
        const bool mine = tn % TPI == tok0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (j == jn && mine) vr[j] = vn;
      }
      // V tile to LDS; slots past the context (and tiles of invalid blocks) may hold
      // anything, including NaN: they become 0 (their weight is 0).
      const bool edge = bad || (lb + 1) * kBlock > keys;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int t = TPI * j + tok0;
        uint4 x = vr[j];
        if (edge && (bad || lb * kBlock + t >= keys)) x = uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4 *>(vt + t * M::R + vslot<D>(t, chunk) * 16) = x;
      }
      // S^T = K Q^T: lane (lg, l16) holds tokens 4 lg + r of column l16.
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NV; ++j) sacc = mfma_k32(kr[j], qf[j], sacc);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = sacc[r] * sc;
        if (edge && (bad || lb * kBlock + 4 * lg + r >= keys)) x[r] = -INFINITY;
      }
      const float m4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (wave_any(m4 > my_m + kRescaleSlack)) {
        // Raise the reference of every column to its new maximum (over the four lane
        // groups that share the column).
        float mc = fmaxf(m4, shfl_xor(m4, 16));
        mc = fmaxf(mc, shfl_xor(mc, 32));
        const float mn = fmaxf(my_m, mc);
        const float alpha = (my_m == -INFINITY) ? 0.f : fast_exp2(my_m - mn);
        my_m = mn;
        mneg = (mn == -INFINITY) ? 0.f : -mn;
        my_l *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
      }
      const uint32_t pk0 = pack_bf16x2(fast_exp2(x[0] + mneg), fast_exp2(x[1] + mneg));
      const uint32_t pk1 = pack_bf16x2(fast_exp2(x[2] + mneg), fast_exp2(x[3] + mneg));
      my_l = dot2_bf16(pk0, 0x3F803F80u, my_l);
      my_l = dot2_bf16(pk1, 0x3F803F80u, my_l);
      const v4i16_t pb = __builtin_bit_cast(v4i16_t, uint2{pk0, pk1});
      // O^T += V^T P^T: the transposing read gives lane (lg, i) dim 16 mt + i of tokens
      // 4 lg + 0..3; lane (lg, 4 jj + q) addresses token 4 lg + jj, dims 16 mt + 4 q..+3.
      const int vt_tok = 4 * lg + (l16 >> 2);
      const int vt_q = l16 & 3;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const v4i16_t av = lds_read_tr16(vt + vt_tok * M::R +
                                         vslot<D>(vt_tok, 2 * mt + (vt_q >> 1)) * 16 +
                                         (vt_q & 1) * 8);
        oacc[mt] = mfma_k16(av, pb, oacc[mt]);
      }
    };

    // fp32 block update: per-lane fp32 dot products summed over the lanes of a token,
    // fp32 FMAs for P.V (every lane keeps its own tokens' weights).
    auto compute = [&](const uint4 (&kr)[NV], const uint4 (&vr)[NV], int i) {
      const int lb = readlane(m_lb, i);
      const bool bad = readlane(m_ok, i) == 0;
      const int key0 = lb * kBlock + tok0;
      float s[NV][HG];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float x = 0.f;
#pragma unroll
          for (int k = 0; k < WPC; ++k)
            x = fmaf(__uint_as_float(qw[hh][k]), __uint_as_float(kw[k]), x);
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
          const float x = __uint_as_float(vw[k]);
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) acc[hh][k] = fmaf(pr[hh], x, acc[hh][k]);
        }
      }
    };

    // Ring of PF+1 register buffers: while block i is computed, block i+1 is in flight.
    uint4 kb[PF + 1][NV], vb[PF + 1][NV];
#pragma unroll
    for (int q = 0; q < PF; ++q) load(kb[q], vb[q], q);
    for (int i0 = 0; i0 < nc; i0 += PF + 1) {
#pragma unroll
      for (int u = 0; u <= PF; ++u) {
        const int un = (u + PF) % (PF + 1);
        load(kb[un], vb[un], i0 + u + PF);
        const int i = i0 + u;
        if (i < nc) {
          if constexpr (kF32)
            compute(kb[u], vb[u], i);
          else if constexpr (kMfma)
            compute_mfma(kb[u], vb[u], i);
          else
            compute_bf16(kb[u], vb[u], i, u);
        }
      }
    }
  }

  // The wave's totals: bf16 weight sums are spread over the lanes that scored them;
  // fp32 counted each token's weight on all CPR lanes of the token, so summing over the
  // lanes of one chunk gives the totals.  The accumulators hold one chunk's dims per
  // lane and token group: summed over the token groups, lanes < CPR hold them all.
  if constexpr (kMfma) {
    // Column l16's totals: the weight sum over its four lane groups; its O^T tiles hold
    // dims 16 mt + 4 lg + r.
    float lt = my_l + shfl_xor(my_l, 16);
    lt += shfl_xor(lt, 32);
    if (l16 < HG) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[wave][l16][16 * mt + 4 * lg + r] = oacc[mt][r];
      if (lg == 0) {
        s_ml[wave][l16][0] = my_m;
        s_ml[wave][l16][1] = lt;
      }
    }
  } else {
    if constexpr (!kF32) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
        lsum[hh] = wave_sum((scoring && hh_s == hh) ? my_l : 0.f);
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      if constexpr (kF32) lsum[hh] = sum_over_chunk_lanes<CPR>(lsum[hh]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[hh][e] = sum_over_chunk_lanes<CPR>(acc[hh][e]);
    }
    // Lanes < CPR hold chunk `lane` (indexing by lane rather than the chunk index
    // computed before the loop keeps that index from staying live across it: at 128
    // registers it was spilled).
    if (lane < CPR) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_o[wave][hh][lane * EPC + e] = acc[hh][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        s_ml[wave][hh][0] = mref[hh];
        s_ml[wave][hh][1] = lsum[hh];
      }
    }
  }
  __syncthreads();
  // Merge of the waves: thread t owns (head t / D, dim t % D).
  for (int t = threadIdx.x; t < HG * D; t += 64 * NW) {
    const int hh = t / D;
    const int d = t - hh * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_ml[w][hh][0]);
    float L = 0.f, o = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float m = s_ml[w][hh][0];
        const float wt = m == -INFINITY ? 0.f : fast_exp2(m - mx);
        L = fmaf(wt, s_ml[w][hh][1], L);
        o = fmaf(wt, s_o[w][hh][d], o);
      }
    }
    const float res = L > 0.f ? o / L : 0.f;
    if (p.partials) {
      p.ws_o[(part + hh) * D + d] = res;
      if (d == 0) p.ws_lse[part + hh] = L > 0.f ? mx + __builtin_amdgcn_logf(L) : -INFINITY;
    } else {
      T *dst = static_cast<T *>(a.out) + ((size_t)row * a.num_q_heads + h0 + hh) * D + d;
      if constexpr (kF32) *dst = res;
      else *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16(res);
    }
  }
}


}  // namespace pkv
