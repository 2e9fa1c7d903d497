// Prefill-chunk attention (query chunks of two or more rows) with bf16 MFMA.
//
// Method (pages cited by title and section):
//  * Inference-engine page (xiaohu-jiedu), prefill/decode section: prefill handles
//    many positions at once with large matrix products and is compute bound.
//  * Same page, Chunked Prefill subsection: a long prompt is split into consecutive
//    slices processed over several steps, each following the positions already in
//    the cache, mixed with other requests' decode tokens.  So row i of a chunk of q
//    rows over c keys is position c-q+i and sees keys 0..c-q+i.
//  * Serving-engine KV page (ttlab), section 2, "blocks and block table": keys and
//    values are read from 16-token blocks through the block table.
//
// One workgroup (8 waves, two per SIMD) owns 128 columns = (query row, q head) pairs
// of one KV head: HGP heads x (128/HGP) consecutive rows.  The keys are walked in
// 128-key steps (8 physical blocks).  Waves 0-3 take the first 64 keys of a step and
// waves 4-7 the second 64, each wave over 32 columns, so every SIMD holds one wave of
// each half and can run one wave's softmax while the other's matrix products issue.
// The two halves keep separate online-softmax states (an in-workgroup split of the
// key range) that are merged through LDS at the end.
//
// K and V are staged in LDS row-major (each with its own XOR swizzle of the 16-byte
// chunks, so that the K fragment reads and the transposing V fragment reads are free
// of bank conflicts); the next step's global loads are in flight
// while the current step is computed (double-buffered LDS).  Each wave computes the
// transposed score tile S^T = K Q^T and the update O^T += V^T P^T with
// v_mfma_f32_16x16x32_bf16.  Working on transposes lets the score accumulator feed
// the second product directly: both hold one column per lane%16 and the same key
// slots.
//
// MFMA 16x16x32 operand layout (lane l, g = l/16): A row l%16 and B column l%16 each
// hold 8 k-slots (g, e); the contraction pairs equal slots, so any fixed assignment
// of k indices to slots is valid as long as A and B agree.  The accumulator holds
// rows 4g..4g+3 of column l%16.
//
// Softmax is the online form in log2 units with a lazily raised per-column reference
// max (raised only when a score exceeds it by more than kSlack, so the cross-lane
// maximum is only formed then).  P is rounded to bf16 for the second product and the
// softmax denominator sums those same rounded weights (dot2 with ones), accumulation
// is fp32, output is bf16 (RNE).  A negative scale is folded into the
// sign of q (exact in bf16) so the kernel works with |scale|.
#include <algorithm>
#include <climits>

#include "decode_body.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kPThreads = 512;  // 8 waves
constexpr int kHalfKeys = 64;   // keys per wave group per step
constexpr int kStepKeys = kPrefillStepKeys;  // keys per step (128)
constexpr int kCols = kPrefillCols;  // columns per workgroup
constexpr int kTblCache = 256;  // block-table entries cached in LDS (4,096 keys)
constexpr float kSlack = 8.0f;  // log2 units
constexpr uint32_t kBf16Ones = 0x3F803F80u;  // two bf16 1.0

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) {
  return __builtin_bit_cast(bf16x8_t, x);
}

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land at LDS
// byte address lds_byte + 16*L (lds_byte is wave-uniform; it travels in M0).  Written
// as asm so that the compiler, which cannot tell the two LDS buffers apart, does not
// hold this step's LDS reads until the next step's loads have landed; the kernel waits
// for these loads itself (vmcnt) before the barrier that publishes the buffer.
__device__ __forceinline__ void load_lds16(const void *g, uint32_t lds_byte) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_byte));
}

typedef short v8i16_t __attribute__((ext_vector_type(8)));

// Slot of 16-byte chunk c of a K row in LDS: c ^ swz_k(row), of a V row: c ^
// swz_v(row).  Both depend on the row mod 16 only (every row that one thread stages
// shares them).  The K fragment read sends 16 consecutive rows, one chunk each, to a
// quarter-wave; the V^T read sends 8 consecutive rows, two adjacent chunks each, to
// half a wave.  The functions make the 16 (row, slot) pairs of each such group land on
// different banks, with 16-lane passes over 32 four-byte banks and with 32-lane passes
// over 64 banks alike (checked exhaustively for both head sizes).  For d = 128 the K
// slot is c ^ row (rows are 256 bytes, so each starts at bank 0); the V slot uses
// 2*row, because the same XOR by row would put rows 2j and 2j+1, whose chunk pairs
// are the same two slots, on the same banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 15;
  else return ((row >> 1) & 3) | (((row ^ (row >> 3)) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return (row << 1) & 15;
  else return (row & 2) | (((row ^ (row >> 2)) & 1) << 2);
}

// Item and index of element j of a sequence of n items in which item i holds count(i)
// elements, numbered over the items in order (item = -1 when j is past the last
// element).  Every thread of the workgroup calls it (two barriers): thread t counts the
// elements of a run of ceil(n / threads) consecutive items, an exclusive scan over the
// threads finds the run holding j, and that thread walks it.  s_find holds at least
// waves + 2 ints.
template <typename CF>
__device__ __forceinline__ void find_in_runs(int n, int j, CF &&count, int *s_find,
                                             int &item, int &local) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kW = kPThreads / 64;
  const int per = (n + kPThreads - 1) / kPThreads;
  const int s0 = min(tid * per, n);
  const int s1 = min(s0 + per, n);
  int cnt = 0;
  for (int s = s0; s < s1; ++s) cnt += count(s);
  int inc = cnt;  // inclusive prefix over the wave's lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) s_find[wave] = inc;
  if (tid == 0) s_find[kW] = -1;
  __syncthreads();
  int excl = inc - cnt;
  for (int w = 0; w < wave; ++w) excl += s_find[w];
  if (j >= excl && j < excl + cnt) {
    int r = j - excl;
    for (int s = s0; s < s1; ++s) {
      const int c = count(s);
      if (r < c) {
        s_find[kW] = s;
        s_find[kW + 1] = r;
        break;
      }
      r -= c;
    }
  }
  __syncthreads();
  item = s_find[kW];
  local = s_find[kW + 1];
}

// Row tiles of a batch: a sequence with q_len >= 2 query rows (q_len <= total_q) has
// ceil(q_len / BM) of them, numbered over the sequences in order; decode rows and
// broken lengths have none.  Finds the sequence of row tile j and j's index among that
// sequence's tiles (seq = -1 when j is past the last one).
template <int BM>
__device__ __forceinline__ void find_row_tile(const int32_t *qsl, int num_seqs, int total_q,
                                              int j, int *s_find, int &seq, int &local) {
  auto tiles_of = [&](int s) {
    const int q = qsl[s + 1] - qsl[s];
    return (q >= 2 && q <= total_q) ? (q + BM - 1) / BM : 0;
  };
  find_in_runs(num_seqs, j, tiles_of, s_find, seq, local);
}

// Decode workgroup k of a mixed launch -> the virtual workgroup of the decode plan it
// runs, rows longest first (the workgroups are dispatched in order, so long pieces start
// while the chunk's shorter row tiles end, and short ones fill the end).  All pieces
// of a row are equally long (its key ranges are equal fractions), so workgroup k takes
// piece k % (groups * splits) of the row of rank k / (groups * splits) in descending
// context length; rows that are no decode row (the chunks, whose pieces do nothing)
// come last.  The rank comes from a counting sort on buckets of `bucket_keys` keys
// (rows of one bucket in index order) that every decode workgroup computes on its own:
// a histogram of the 256 buckets, a scan of it, and a pass over the rows of the
// bucket that holds the rank.  Returns a value past the plan's workgroups for padding
// workgroups.  s_hist holds 256 ints, s_find at least waves + 2.
__device__ __forceinline__ int64_t mixed_decode_piece(const AttnArgs &a, const SegArgs &dp, int k,
                                                      int bucket_keys, int *s_hist,
                                                      int *s_find) {
  const int tid = threadIdx.x;
  const int per_row = dp.groups * dp.splits;
  const int r = k / per_row;
  const int rem = k - r * per_row;
  if (r >= dp.items) return (int64_t)dp.items * per_row;  // padding
  auto bucket = [&](int i) {
    const int q = a.query_start_loc[i + 1] - a.query_start_loc[i];
    if (q != 1) return 255;
    return 254 - min(253, max(a.context_lens[i], 0) / bucket_keys);
  };
  if (tid < 256) s_hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < dp.items; i += kPThreads) atomicAdd(&s_hist[bucket(i)], 1);
  __syncthreads();
  int b = -1, off = 0;
  find_in_runs(256, r, [&](int x) { return s_hist[x]; }, s_find, b, off);
  __syncthreads();  // every thread has read the result before s_find is reused
  int row = -1, idx = 0;
  find_in_runs(dp.items, off, [&](int i) { return bucket(i) == b ? 1 : 0; }, s_find, row,
               idx);
  if (row < 0) return (int64_t)dp.items * per_row;
  const int g = rem / dp.splits;
  const int split = rem - g * dp.splits;
  return ((int64_t)g * dp.items + row) * dp.splits + split;
}

// One wave's update with a 64-key tile: kb and vb = K and V tiles, each row-major
// [key][16-byte chunk slot] (slots as above); kbase = position of the tile's first key.  MASK
// applies the causal and length masks (tiles that reach past the first column's
// position or past kv_end).  mid(ks) is called after the score products of k-step ks
// (the caller issues one part of the next step's staging there, so that the staging
// loads do not stall the wave in one burst ahead of the products).
template <int D, bool MASK, typename FM>
__device__ __forceinline__ void tile_update(FM &&mid, const uint4 *kb, const uint4 *vb,
                                            const bf16x8_t (&qf)[2][D / 32],
                                            f32x4_t (&o)[D / 16][2], float (&mref)[2],
                                            float (&mneg)[2], float (&lsum)[2], float sc,
                                            int kbase, const int (&col_pos)[2], int kv_end,
                                            int l16, int lg) {
  constexpr int KS = D / 32;
  constexpr int MT = D / 16;
  constexpr int NCH = D / 8;

  // S^T tile: sacc[sub][cg] element r <-> key kbase + 16*sub + 4*lg + r, column cg.
  f32x4_t sacc[4][2];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) sacc[sub][cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int key = sub * 16 + l16;
      const bf16x8_t af = as_bf16x8(kb[key * NCH + ((4 * ks + lg) ^ swz_k<D>(key))]);
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) sacc[sub][cg] = mfma16(af, qf[cg][ks], sacc[sub][cg]);
    }
    mid(ks);
  }

  // Masked scores (MASK: past a column's position or past kv_end) become -inf.
  if (MASK) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + sub * 16 + 4 * lg + r;
          if (key > col_pos[cg] || key >= kv_end) sacc[sub][cg][r] = -INFINITY;
        }
  }
  // P = exp2(s * sc - mref), first with the current reference: the exponentials need
  // only this step's scores, so they can issue while the last score products finish
  // and before the reference check below.  Where that check raises the reference (it
  // does whenever a score exceeds the reference by more than kSlack, in particular on
  // a wave's first keys), the weights are recomputed; otherwise every weight is at most
  // 2^kSlack.
  float p[2][16];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg)
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p[cg][sub * 4 + r] = fast_exp2(fmaf(sacc[sub][cg][r], sc, mneg[cg]));

  // Per-lane maximum of the scaled scores (log2 units).
  float lmx[2];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    float m = sacc[0][cg][0];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (sub | r) m = fmaxf(m, sacc[sub][cg][r]);
    lmx[cg] = m * sc;
  }
  const bool need = (lmx[0] > mref[0] + kSlack) || (lmx[1] > mref[1] + kSlack);
  if (wave_any(need)) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      float m = lmx[cg];
      m = fmaxf(m, shfl_xor(m, 16));
      m = fmaxf(m, shfl_xor(m, 32));
      const float mn = fmaxf(mref[cg], m);
      const float alpha = (mref[cg] == -INFINITY) ? 0.f : fast_exp2(mref[cg] - mn);
      mref[cg] = mn;
      mneg[cg] = (mn == -INFINITY) ? 0.f : -mn;
      lsum[cg] *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt][cg] *= alpha;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p[cg][sub * 4 + r] = fast_exp2(fmaf(sacc[sub][cg][r], sc, mneg[cg]));
    }
  }

  // P in bf16, packed in the k-slot order of the V^T fragments.
  bf16x8_t pf[2][2];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      uint4 packed;
      packed.x = pack_bf16x2(p[cg][8 * ks2 + 0], p[cg][8 * ks2 + 1]);
      packed.y = pack_bf16x2(p[cg][8 * ks2 + 2], p[cg][8 * ks2 + 3]);
      packed.z = pack_bf16x2(p[cg][8 * ks2 + 4], p[cg][8 * ks2 + 5]);
      packed.w = pack_bf16x2(p[cg][8 * ks2 + 6], p[cg][8 * ks2 + 7]);
      pf[cg][ks2] = as_bf16x8(packed);
      // The denominator sums the same bf16-rounded weights the numerator uses.
      lsum[cg] = dot2_bf16(packed.x, kBf16Ones, lsum[cg]);
      lsum[cg] = dot2_bf16(packed.y, kBf16Ones, lsum[cg]);
      lsum[cg] = dot2_bf16(packed.z, kBf16Ones, lsum[cg]);
      lsum[cg] = dot2_bf16(packed.w, kBf16Ones, lsum[cg]);
    }
  }

  // O^T += V^T P^T: A row = dim, k-slots (lg, e) <-> keys 32*ks2 + 4*lg + e (e < 4)
  // and 32*ks2 + 16 + 4*lg + (e - 4), matching the slots of pf.  Each half of an A
  // fragment is one transposing LDS read (ds_read_b64_tr_b16): within a 16-lane group
  // g, lane i receives element i%4 of the 4-element rows addressed by lanes
  // 16g + 4j + i/4, j = 0..3.  So lane (g, j = l16/4, q = l16%4) addresses dims
  // 16*mt + 4q..4q+3 of key 4g + j (+16 for the second half), and lane (g, i) receives
  // dim 16*mt + i of keys 4g + 0..3.
  const int vj = l16 >> 2;
  const int vq = l16 & 3;
  const int vkey = 4 * lg + vj;
  const int vsw = (vq >> 1) ^ swz_v<D>(vkey);  // chunk of dims 16*mt + 4q is 2mt + q/2
  const char *vrow = reinterpret_cast<const char *>(vb) + vkey * (NCH * 16) + (vq & 1) * 8;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const char *vp = vrow + ((2 * mt) ^ vsw) * 16;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const v4i16_t lo = lds_read_tr16(vp + (32 * ks2) * (NCH * 16));
      const v4i16_t hi = lds_read_tr16(vp + (32 * ks2 + 16) * (NCH * 16));
      const bf16x8_t af = __builtin_bit_cast(
          bf16x8_t, (v8i16_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) o[mt][cg] = mfma16(af, pf[cg][ks2], o[mt][cg]);
    }
  }
}

}  // namespace

// MIXED: the workgroups past the chunk's tiles each run one decode workgroup of plan
// `dp` (kDecodeWavesMin = 8 waves, the decode kernel's body, its LDS laid over this
// kernel's tiles), so the decode rows of a mixed batch fill the compute units that the
// chunk's shorter row tiles leave idle.
// The workgroups of a mixed launch are, in order: the first `mix_first` chunk
// workgroups (row tiles that surely exist), the `mix_dec` decode workgroups, then the
// other chunk workgroups (slots that may be empty), so that the units freed by short
// row tiles go to decode work rather than to empty slots; mix_bucket is the bucket
// width (keys) of the decode rows' longest-first order (0: the plan's order).  Without decode workgroups
// mix_dec is 0 and mix_first the number of row-tile workgroups that surely exist (at
// least one).
template <int D, int HGP, bool MIXED, bool FUSED>
__global__ __launch_bounds__(kPThreads) void prefill_mfma_kernel(AttnArgs a,
                                                                 int num_head_groups,
                                                                 int tile_slots,
                                                                 PrefillSplit ps, SegArgs dp,
                                                                 int mix_first, int mix_dec,
                                                                 int mix_bucket) {
  constexpr int BMQ = kCols / HGP;  // query rows per workgroup
  constexpr int KS = D / 32;        // k-steps of S^T over head_dim
  constexpr int MT = D / 16;        // 16-dim row tiles of O^T
  constexpr int NCH = D / 8;        // 16-byte chunks per K row
  constexpr int K_U4 = kHalfKeys * NCH;               // uint4 per K (or V) tile
  constexpr int KCH = kStepKeys * NCH / kPThreads;    // chunks per thread per step, each pool
  constexpr int LDS_U4 = 8 * K_U4;                    // [buf][half] K tiles, then V tiles
  constexpr int XF = MT * 8 + 4;                      // floats per lane in the merge
  static_assert(4 * XF * 64 * 4 <= LDS_U4 * 16, "merge exchange must fit the tiles");
  __shared__ uint4 lds[LDS_U4];
  __shared__ int s_tbl[kTblCache];  // block-table entries of this workgroup
  __shared__ int s_find[kPThreads / 64 + 2];  // row-tile and decode-order lookups
  uint4 *const k_lds = lds;             // [buf*2+half][K_U4]
  uint4 *const v_lds = lds + 4 * K_U4;  // [buf*2+half][K_U4]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = wave >> 2;  // which 64 keys of each step
  const int cw = wave & 3;     // which 32 columns
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // Workgroup u computes split u % splits of tile u / splits, and tile = row tile j *
  // units + head unit (prefill_tile_index), the row tiles numbered densely (below).
  // Workgroups go to the XCDs round-robin by index and, inside an XCD, to its shader
  // engines round-robin, each waiting for a free compute unit of its own engine.  With
  // dense numbering every XCD starts its real tiles first, spread over all its engines
  // (with an empty slot after each real tile, as a batch of 64-row chunks had when the
  // tiles were numbered by query offset, the real tiles all fell on two of the four
  // engines and ran in two rounds, taking twice as long).
  const int units = a.num_kv_heads * num_head_groups;
  const int total = tile_slots * units * ps.splits;
  int u = blockIdx.x;
  // Fused calls store this step's new rows in this launch, the first mix_first
  // workgroups a share each (those dispatched first: the row tiles that surely exist).
  // FUSED (the chunk launch of a fused call with one sequence): the chunk tiles read
  // those keys and values from k_new / v_new.  MIXED with k_new (a shared prefix's
  // fused call): the shared-run tiles read none of them, and each decode row's newest
  // key and value come from k_new / v_new.  (In the shared-run launch the tiles come
  // first and end earlier than the second round of decode workgroups, so the write
  // stays off the launch's longest chain.)
  if constexpr (FUSED || MIXED) {
    if ((FUSED || a.k_new != nullptr) && (int)blockIdx.x < mix_first)
      fused_slot_write<uint16_t, D>(a, blockIdx.x, mix_first, kPThreads);
  }
  if constexpr (MIXED) {
    if (u >= mix_first) {
      if (u < mix_first + mix_dec) {
        constexpr int HGD = mixed_decode_head_group(D, HGP);
        using DL = DecodeLds<uint16_t, D, HGD, kDecodeWavesMin>;
        static_assert(kPThreads == 64 * kDecodeWavesMin, "one decode workgroup per workgroup");
        static_assert(DL::bytes() <= sizeof(lds), "the decode LDS must fit in the tiles");
        // Longest rows first (mix_bucket > 0), else in the plan's order.
        const int64_t v =
            mix_bucket > 0 ? mixed_decode_piece(a, dp, u - mix_first, mix_bucket, s_tbl, s_find)
                           : (int64_t)(u - mix_first);
        decode_segment<uint16_t, D, HGD, kDecodeWavesMin>(
            a, dp, v, DL::over(reinterpret_cast<char *>(lds)));
        return;
      }
      u -= mix_dec;
    }
  }
  if (u >= total) return;
  const int split = u % ps.splits;
  const int tile = u / ps.splits;
  const int tid = threadIdx.x;
  const bool shared = ps.shared_keys > 0;  // the shared-run pass of a shared prefix
  const bool partials = ps.splits > 1 || shared;
  // Split partials: until this tile's columns are known, mark them all unused, so the
  // merge skips tiles that end early (decode rows, empty slots, broken lengths).
  if (partials && split == 0 && tid < kCols) ps.col[(size_t)tile * kCols + tid] = -1;
  const int j = tile / units;
  const int hu = tile - j * units;
  const int hgi = hu % num_head_groups;
  const int kvh = hu / num_head_groups;

  int seq, q_begin, q_len, qtile, ctx;
  if (shared) {
    // Every row of the batch is a column of one chunk over the shared run (table row
    // 0's first blocks); row tile j holds rows [j*BMQ, (j+1)*BMQ).
    seq = 0;
    q_begin = 0;
    q_len = a.total_q;
    if (j * BMQ >= q_len) return;
    qtile = j;
    ctx = ps.shared_keys;
  } else {
    // Decode rows (one query) have no row tile: they run in the split-K kernel.
    int local;
    find_row_tile<BMQ>(a.query_start_loc, a.num_seqs, a.total_q, j, s_find, seq, local);
    if (seq < 0) return;  // past the batch's last row tile
    q_begin = a.query_start_loc[seq];
    q_len = a.query_start_loc[seq + 1] - q_begin;
    if (q_begin < 0 || q_begin + q_len > a.total_q) return;
    const int ntiles = (q_len + BMQ - 1) / BMQ;
    qtile = ntiles - 1 - local;  // tiles that see the most keys go first
    ctx = a.context_lens[seq];
  }
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hbase = kvh * group + hgi * HGP;
  const int qi0 = qtile * BMQ;
  const int nq = min(BMQ, q_len - qi0);
  uint16_t *out = static_cast<uint16_t *>(a.out);

  // Columns of this lane (one per 16-column group).
  int col_row[2], col_head[2], col_pos[2];
  bool col_ok[2];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    const int c = cw * 32 + cg * 16 + l16;
    const int g = c / BMQ;
    int qi = c - g * BMQ;
    col_ok[cg] = qi < nq;
    qi = min(qi, nq - 1);  // padding columns repeat a real row; never stored
    col_row[cg] = q_begin + qi0 + qi;
    col_head[cg] = hbase + g;
    // A shared run has no causal limit: every row sees all of its keys.
    col_pos[cg] = shared ? ctx - 1 : ctx - q_len + qi0 + qi;
  }

  if (!shared && ctx < q_len) {  // precondition broken: defined as zeros
    if (half == 0) {
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
        if (col_ok[cg])
          for (int d = lg; d < D; d += 4)
            out[((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D + d] = 0;
    }
    return;
  }

  // Q^T fragments (B operand of S^T): column's row, dims 32*ks + 8*lg + 0..7, with
  // the sign of a negative scale folded in.
  const float sc = fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) +
        ((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 x = src[4 * ks + lg];
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      qf[cg][ks] = as_bf16x8(x);
    }
  }

  const int pos_first = shared ? ctx - 1 : ctx - q_len + qi0;
  const int ctx_eff = min(ctx, a.max_blocks_per_seq * kBlock);
  const int kv_end = min(pos_first + nq, ctx_eff);
  const int nst_tile = (kv_end + kStepKeys - 1) / kStepKeys;
  // This split's steps [st0, nst) of the tile's nst_tile (the split-K of short chunks
  // over long contexts; one split covers them all otherwise).
  const int st0 = (int)((int64_t)split * nst_tile / ps.splits);
  const int nst = (int)((int64_t)(split + 1) * nst_tile / ps.splits);
  const int32_t *tbl = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);

  f32x4_t o[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) o[mt][cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  float mneg[2] = {0.f, 0.f};
  float lsum[2] = {0.f, 0.f};

  // Block-table entries of the keys this workgroup reads, cached in LDS kTblCache at a
  // time (refilled every kTblCache/8 steps); invalid entries read block 0.
  const int nblk = (kv_end + kBlock - 1) / kBlock;
#define PKV_FILL_TBL(first_blk)                                                          \
  do {                                                                                   \
    if (tid < kTblCache) {                                                               \
      const int lb_ = (first_blk) + tid;                                                 \
      const int pb_ = lb_ < nblk ? tbl[lb_] : 0;                                         \
      s_tbl[tid] = (pb_ < 0 || pb_ >= a.num_blocks) ? 0 : pb_;                           \
    }                                                                                    \
  } while (0)

  // Staging of a 128-key step: K and V rows go from global memory straight into LDS
  // buffer `buf` (keys 0-63 of the step to half 0, 64-127 to half 1), both row-major
  // with the 16-byte chunk slots swizzled (swz_k, swz_v).  One wave's 16-byte loads
  // land at consecutive LDS addresses (lane L at 16*L), i.e. rows kw0 + L/NCH, slot
  // L%NCH, so a lane fetches the chunk that the row's swizzle puts in its slot.  Thread
  // tid handles key kkey0 + KSTRIDE*i (i < KCH) of the step, slot kch; the row's
  // residue mod 16, hence its swizzle, and its row inside the block are those of kkey0
  // for every i (KSTRIDE is a multiple of 16).  Every load is unconditional: a key past kv_end reads a row of
  // its block, or of block 0 when its table entry is past the sequence.  Scores of
  // such keys are masked; their V rows are zeroed after landing (a stale NaN times a
  // zero weight would still be NaN), by the wave that loaded them, once its loads
  // have completed.
  constexpr int KSTRIDE = kPThreads / NCH;
  static_assert(KSTRIDE % kBlock == 0, "rows must stay fixed across a thread's chunks");
  const uint32_t blk_bytes = (uint32_t)a.num_kv_heads * kBlock * D * 2;
  const int kch = tid % NCH;
  const int kkey0 = tid / NCH;
  const int kw0 = __builtin_amdgcn_readfirstlane(tid >> 6) * (64 / NCH);
  const size_t row_off = ((size_t)kvh * kBlock + kkey0 % kBlock) * D * 2;
  const char *kthr = reinterpret_cast<const char *>(kpool) + row_off +
                     (kch ^ swz_k<D>(kkey0)) * 16;
  const char *vthr = reinterpret_cast<const char *>(vpool) + row_off +
                     (kch ^ swz_v<D>(kkey0)) * 16;
  // Fused call: this step's rows (positions new0 = ctx - q_len onward) are read from
  // k_new / v_new, position p at row q_begin + p - new0, since this launch is still
  // writing their slots.  Otherwise new0 lies past every key.
  const bool new_rows = FUSED && !shared;
  const int new0 = new_rows ? ctx - q_len : INT_MAX;
  const size_t nrow_bytes = (size_t)a.num_kv_heads * D * 2;
  const size_t nrow_off = (size_t)kvh * D * 2;
  const char *knthr = new_rows ? static_cast<const char *>(a.k_new) + nrow_off +
                                     (kch ^ swz_k<D>(kkey0)) * 16
                               : nullptr;
  const char *vnthr = new_rows ? static_cast<const char *>(a.v_new) + nrow_off +
                                     (kch ^ swz_v<D>(kkey0)) * 16
                               : nullptr;
  // Part i of the staging of step s into buffer b.  Fused call: a step that holds new
  // positions (uniform over the workgroup) reads those from k_new / v_new; positions
  // past the sequence's last row (masked keys of the last step) read that row.
  auto fetch = [&](int s, int b, int i) {
    const int k0 = s * kStepKeys;
    const int key_ = kw0 + KSTRIDE * i;
    const int row_ = (b * 2 + key_ / kHalfKeys) * K_U4 + (key_ % kHalfKeys) * NCH;
    const uint64_t off_ =
        (uint64_t)(uint32_t)s_tbl[(s * (kStepKeys / kBlock)) % kTblCache +
                                  (kkey0 + KSTRIDE * i) / kBlock] * blk_bytes;
    const char *ks = kthr + off_;
    const char *vs = vthr + off_;
    if constexpr (FUSED) {
      if (k0 + kStepKeys > new0) {
        const int pos = k0 + kkey0 + KSTRIDE * i;
        const int r = min(max(pos, new0), ctx - 1) - new0;
        const size_t noff = (size_t)(q_begin + r) * nrow_bytes;
        if (pos >= new0) {
          ks = knthr + noff;
          vs = vnthr + noff;
        }
      }
    }
    load_lds16(ks, (uint32_t)(uintptr_t)(k_lds + row_));
    load_lds16(vs, (uint32_t)(uintptr_t)(v_lds + row_));
  };
  // After this wave's loads of step st have completed: zero its V slots past kv_end
  // (only the last step has any).
#define PKV_ZERO_TAIL(st, buf)                                                           \
  do {                                                                                   \
    const int k0_ = (st) * kStepKeys;                                                    \
    if (k0_ + kStepKeys > kv_end) {                                                      \
      _Pragma("unroll") for (int i = 0; i < KCH; ++i) {                                  \
        const int key_ = kkey0 + KSTRIDE * i;                                            \
        if (k0_ + key_ >= kv_end)                                                        \
          v_lds[((buf) * 2 + key_ / kHalfKeys) * K_U4 + (key_ % kHalfKeys) * NCH + kch] = \
              uint4{};                                                                   \
      }                                                                                  \
    }                                                                                    \
  } while (0)

  PKV_FILL_TBL((st0 * (kStepKeys / kBlock)) / kTblCache * kTblCache);
  __syncthreads();
  if (partials && split == 0) {  // after the unused marks: a barrier lies between
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
      if (half == 0 && lg == 0 && col_ok[cg])
        ps.col[(size_t)tile * kCols + cw * 32 + cg * 16 + l16] =
            col_row[cg] * a.num_q_heads + col_head[cg];
  }
  if (st0 < nst) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) fetch(st0, st0 & 1, i);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed in LDS
    PKV_ZERO_TAIL(st0, st0 & 1);
  }
  __syncthreads();
  // Retire every outstanding load (the query fragments in particular) on all paths
  // here.  Otherwise the wait counters merged at the loop head still see the query
  // loads in flight, and each MFMA that reads them waits for the next step's
  // prefetch as well, which undoes the overlap.
  __builtin_amdgcn_s_waitcnt(0);

  for (int st = st0; st < nst; ++st) {
    const int buf = st & 1;
    // Refill the table cache before the first fetch that needs new entries.
    if (st + 1 < nst && ((st + 1) * (kStepKeys / kBlock)) % kTblCache == 0) {
      PKV_FILL_TBL((st + 1) * (kStepKeys / kBlock));
      __syncthreads();
    }
    // The staging of step st+1 (into the buffer step st-1 used, free since the last
    // barrier) in KCH parts, one per k-step of this step's score products; KCH equals
    // the number of k-steps (D / 32).  The last step stages too, without a branch
    // around each part: the table cache then names blocks of the current window (or
    // block 0), so those loads read valid pool rows into the buffer no step reads any
    // more, and they have landed before the barrier that ends the loop.
    static_assert(KCH == KS, "one staging part per k-step");
    auto fetch_part = [&](int i) { fetch(st + 1, buf ^ 1, i); };

    const int kbase = st * kStepKeys + half * kHalfKeys;
    if (kbase < kv_end) {
      const uint4 *kb = k_lds + (buf * 2 + half) * K_U4;
      const uint4 *vb = v_lds + (buf * 2 + half) * K_U4;
      const bool edge = (kbase + kHalfKeys - 1 > pos_first) || (kbase + kHalfKeys > kv_end);
      if (edge)
        tile_update<D, true>(fetch_part, kb, vb, qf, o, mref, mneg, lsum, sc, kbase, col_pos,
                             kv_end, l16, lg);
      else
        tile_update<D, false>(fetch_part, kb, vb, qf, o, mref, mneg, lsum, sc, kbase, col_pos,
                              kv_end, l16, lg);
    } else {
#pragma unroll
      for (int i = 0; i < KCH; ++i) fetch_part(i);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of step st+1 have landed
    if (st + 1 < nst) PKV_ZERO_TAIL(st + 1, buf ^ 1);
    __syncthreads();  // step st+1 staged; everyone is done reading step st
  }

  // Merge the two halves' states through LDS (the tiles are no longer read: the loop
  // ended on a barrier), then normalise and store bf16, 4 consecutive dims per tile.
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    lsum[cg] += shfl_xor(lsum[cg], 16);
    lsum[cg] += shfl_xor(lsum[cg], 32);
  }
  float *xch = reinterpret_cast<float *>(lds) + cw * XF * 64 + lane;
  if (half == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int r = 0; r < 4; ++r) xch[((mt * 2 + cg) * 4 + r) * 64] = o[mt][cg][r];
    xch[(MT * 8 + 0) * 64] = mref[0];
    xch[(MT * 8 + 1) * 64] = mref[1];
    xch[(MT * 8 + 2) * 64] = lsum[0];
    xch[(MT * 8 + 3) * 64] = lsum[1];
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    const float m1 = xch[(MT * 8 + cg) * 64];
    const float l1 = xch[(MT * 8 + 2 + cg) * 64];
    const float mx = fmaxf(mref[cg], m1);
    const float a0 = (mref[cg] == -INFINITY) ? 0.f : fast_exp2(mref[cg] - mx);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - mx);
    const float L = a0 * lsum[cg] + a1 * l1;
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    if (!col_ok[cg]) continue;
    if (partials) {
      // This split's normalised output and log2-sum-exp (-inf when it saw no key).
      const size_t pc = ((size_t)tile * ps.splits + split) * kCols + cw * 32 + cg * 16 + l16;
      float *po = ps.o + pc * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float4 y;
        y.x = (a0 * o[mt][cg][0] + a1 * xch[((mt * 2 + cg) * 4 + 0) * 64]) * inv;
        y.y = (a0 * o[mt][cg][1] + a1 * xch[((mt * 2 + cg) * 4 + 1) * 64]) * inv;
        y.z = (a0 * o[mt][cg][2] + a1 * xch[((mt * 2 + cg) * 4 + 2) * 64]) * inv;
        y.w = (a0 * o[mt][cg][3] + a1 * xch[((mt * 2 + cg) * 4 + 3) * 64]) * inv;
        *reinterpret_cast<float4 *>(po + mt * 16 + 4 * lg) = y;
      }
      if (lg == 0) ps.lse[pc] = L > 0.f ? mx + __builtin_amdgcn_logf(L) : -INFINITY;
      continue;
    }
    uint16_t *dst = out + ((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        y[r] = (a0 * o[mt][cg][r] + a1 * xch[((mt * 2 + cg) * 4 + r) * 64]) * inv;
      uint2 packed;
      packed.x = pack_bf16x2(y[0], y[1]);
      packed.y = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<uint2 *>(dst + mt * 16 + 4 * lg) = packed;
    }
  }
}

#undef PKV_FILL_TBL
#undef PKV_ZERO_TAIL

// Log-sum-exp merge of the splits of each tile column: out = sum_s 2^(lse_s - M) o_s /
// sum_s 2^(lse_s - M), M = max_s lse_s.  Each thread owns four dims of one column
// (D/4 threads per column), so a tile spreads over kCols*D/4/256 workgroups.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(AttnArgs a, PrefillSplit ps) {
  constexpr int TPC = D / 4;      // threads per column
  constexpr int CPW = 256 / TPC;  // columns per workgroup
  constexpr int WPT = kCols / CPW;  // workgroups per tile
  const int tile = blockIdx.x / WPT;
  const int c = (blockIdx.x % WPT) * CPW + threadIdx.x / TPC;
  const int d0 = (threadIdx.x % TPC) * 4;
  const int dst = ps.col[(size_t)tile * kCols + c];
  if (dst < 0) return;
  const size_t base = (size_t)tile * ps.splits * kCols + c;  // column c of split 0
  float M = -INFINITY;
  for (int s = 0; s < ps.splits; ++s) M = fmaxf(M, ps.lse[base + (size_t)s * kCols]);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = 0; s < ps.splits; ++s) {
      const size_t ps_ = base + (size_t)s * kCols;
      const float ls = ps.lse[ps_];
      const float4 x = *reinterpret_cast<const float4 *>(ps.o + ps_ * D + d0);
      const float w = ls == -INFINITY ? 0.f : fast_exp2(ls - M);
      L += w;
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint2 packed;
  packed.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  packed.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)dst * D + d0) = packed;
}

template <int D, int HGP>
static hipError_t launch_prefill_t(const AttnArgs &a, const PrefillPlan &pl, int shared_keys,
                                   hipStream_t st, const DecodePlan *dpl = nullptr) {
  const int total = pl.tiles * pl.splits;
  int64_t dec_wgs = 0;
  SegArgs dp{};
  if (dpl) {
    if (dpl->head_group != mixed_decode_head_group(D, HGP) || dpl->waves != kDecodeWavesMin)
      return hipErrorInvalidValue;
    dp = decode_seg_args(*dpl, a.num_kv_heads);
    // Padded to a multiple of the XCD count, so that the chunk workgroups after the
    // decode ones keep their XCD (workgroups go to XCDs round-robin by index).
    dec_wgs = ((int64_t)dp.items * dp.groups * dp.splits + 7) / 8 * 8;
  }
  // Row tiles that surely exist: the chunk sequences hold at least total_q -
  // (num_seqs - 1) rows (every other sequence has at most one), so the batch has at
  // least ceil((total_q - num_seqs + 1) / BM) row tiles (a shared run: all its rows).
  const int bm = kCols / HGP;
  const int sure = std::max(1, (a.total_q - a.num_seqs + 1 + bm - 1) / bm);
  const int first = (int)std::min<int64_t>(
      total, (int64_t)std::min(sure, pl.tile_slots) * a.num_kv_heads * pl.num_head_groups *
                 pl.splits);
  if (total + dec_wgs > INT32_MAX) return hipErrorInvalidValue;
  // The new rows of a fused call are stored by the first `first` workgroups.
  if (a.k_new != nullptr && first == 0) return hipErrorInvalidValue;
  if (total + dec_wgs == 0) return hipSuccess;
  PrefillSplit ps{};
  ps.splits = pl.splits;
  ps.shared_keys = shared_keys;
  if (pl.splits > 1 || shared_keys > 0) {
    char *w = static_cast<char *>(pl.workspace);
    ps.o = reinterpret_cast<float *>(w + pl.ws_o_offset);
    ps.lse = reinterpret_cast<float *>(w + pl.ws_lse_offset);
    ps.col = reinterpret_cast<int *>(w + pl.ws_col_offset);
  }
  // Fused calls (k_new given) store the new rows in this launch: the chunk tiles of a
  // single sequence (FUSED), or the shared-run tiles of a shared prefix's launch.
  const bool fused = a.k_new != nullptr && shared_keys == 0;
  const dim3 grid((unsigned)(total + dec_wgs)), block(kPThreads);
  const int nhg = pl.num_head_groups, slots = pl.tile_slots, ndec = (int)dec_wgs;
  // A mixed launch reads the new rows from the pools (the caller writes them first):
  // with k_new in a mixed launch, the chunk steps that read k_new and the stores of
  // the new rows cost more than the separate write launch they save.
  if (dpl && fused) return hipErrorInvalidValue;
  // Buckets of the decode rows' longest-first order: 254 of them over the longest
  // context (a longer row falls in the first).  A shared run's decode rows (the
  // private tails, all short) keep the plan's order: the order costs each decode
  // workgroup a dependent read of every row's lengths, on the launch's longest chain.
  const int bucket =
      shared_keys > 0 ? 0 : std::max(1, (dpl ? dpl->max_context_len : 0) / 254 + 1);
  if (dpl)
    prefill_mfma_kernel<D, HGP, true, false><<<grid, block, 0, st>>>(a, nhg, slots, ps, dp,
                                                                     first, ndec, bucket);
  else if (fused)
    prefill_mfma_kernel<D, HGP, false, true><<<grid, block, 0, st>>>(a, nhg, slots, ps, dp,
                                                                     first, 0, 1);
  else
    prefill_mfma_kernel<D, HGP, false, false><<<grid, block, 0, st>>>(a, nhg, slots, ps, dp,
                                                                      first, 0, 1);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && dpl) e = launch_decode_merge(a, *dpl, PKV_BF16, st);
  // A shared run's partials are merged with the rows' other parts elsewhere.
  if (e != hipSuccess || pl.splits == 1 || shared_keys > 0) return e;
  prefill_merge_kernel<D><<<dim3(pl.tiles * (kCols * D / 4 / 256)), dim3(256), 0, st>>>(a, ps);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const AttnArgs &a, const PrefillPlan &pl, int shared_keys,
                                   hipStream_t st, const DecodePlan *dpl = nullptr) {
  switch (pl.head_group) {
    case 4: return launch_prefill_t<D, 4>(a, pl, shared_keys, st, dpl);
    case 2: return launch_prefill_t<D, 2>(a, pl, shared_keys, st, dpl);
    case 1: return launch_prefill_t<D, 1>(a, pl, shared_keys, st, dpl);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const AttnArgs &a, const PrefillPlan &pl, pkv_dtype dtype,
                          hipStream_t stream) {
  if (dtype != PKV_BF16) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch_prefill_d<64>(a, pl, 0, stream);
  if (a.head_dim == 128) return launch_prefill_d<128>(a, pl, 0, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mixed(const AttnArgs &a, const PrefillPlan &pp, const DecodePlan &dp,
                        hipStream_t stream) {
  if (a.head_dim == 64) return launch_prefill_d<64>(a, pp, 0, stream, &dp);
  if (a.head_dim == 128) return launch_prefill_d<128>(a, pp, 0, stream, &dp);
  return hipErrorInvalidValue;
}

hipError_t launch_shared_run_mixed(const AttnArgs &a, const PrefillPlan &sp, int shared_keys,
                                   const DecodePlan &dp, hipStream_t stream) {
  if (shared_keys <= 0) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch_prefill_d<64>(a, sp, shared_keys, stream, &dp);
  if (a.head_dim == 128) return launch_prefill_d<128>(a, sp, shared_keys, stream, &dp);
  return hipErrorInvalidValue;
}

}  // namespace pkv
