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
// One workgroup (4 waves) owns 128 columns = (query row, q head) pairs of one KV
// head: HGP heads x (128/HGP) consecutive rows.  Each wave owns 32 columns.  The
// workgroup walks 64-key tiles (4 physical blocks): K is staged in LDS row-major and
// V transposed (both XOR-swizzled so the MFMA fragment reads are bank-conflict free),
// then each wave computes the transposed score tile S^T = K Q^T and the update
// O^T += V^T P^T with v_mfma_f32_16x16x32_bf16.  Working on transposes lets the
// score accumulator be reused directly as the B operand of the second product: both
// hold one column per lane%16 and the same key slots.
//
// MFMA 16x16x32 operand layout (lane l, g = l/16): A row l%16 and B column l%16 each
// hold 8 k-slots (g, e); the contraction pairs equal slots, so any fixed assignment
// of k indices to slots is valid as long as A and B agree.  The accumulator holds
// rows 4g..4g+3 of column l%16.
//
// Softmax is the online form in log2 units with a lazily raised per-column reference
// max (raised only when a score exceeds it by more than kSlack), P is rounded to
// bf16 for the second product, accumulation is fp32, output is bf16 (RNE).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kBN = 64;         // keys per tile
constexpr int kCols = 128;      // columns per workgroup
constexpr float kSlack = 8.0f;  // log2 units

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) {
  return __builtin_bit_cast(bf16x8_t, x);
}

}  // namespace

template <int D, int HGP>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(AttnArgs a,
                                                                int num_head_groups,
                                                                int tile_slots) {
  constexpr int BMQ = kCols / HGP;  // query rows per workgroup
  constexpr int KS = D / 32;        // k-steps of S^T over head_dim
  constexpr int MT = D / 16;        // 16-dim row tiles of O^T
  constexpr int NCH = D / 8;        // 16-byte chunks per K row

  __shared__ uint4 k_lds[kBN * NCH];     // [key][chunk ^ (key % NCH)]
  __shared__ uint2 vt_lds[D * (kBN / 4)];  // [dim][keygroup ^ (dim % 16)], 4 keys each

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int total = tile_slots * a.num_kv_heads * num_head_groups;
  int v = xcd_remap(blockIdx.x, total);
  if (v >= total) return;
  const int slot = v % tile_slots;
  v /= tile_slots;
  const int hgi = v % num_head_groups;
  const int kvh = v / num_head_groups;

  // Sequence owning this tile slot: the last s with qsl[s]/BMQ + s <= slot.
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.query_start_loc[mid] / BMQ + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int seq = lo;
  const int q_begin = a.query_start_loc[seq];
  const int q_len = a.query_start_loc[seq + 1] - q_begin;
  if (q_len <= 1) return;  // decode rows run in the split-K kernel
  if (q_begin < 0 || q_begin + q_len > a.total_q) return;
  const int ntiles = (q_len + BMQ - 1) / BMQ;
  const int local = slot - (q_begin / BMQ + seq);
  if (local >= ntiles) return;
  const int qtile = ntiles - 1 - local;  // tiles that see the most keys go first
  const int ctx = a.context_lens[seq];
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
    const int c = wave * 32 + cg * 16 + l16;
    const int g = c / BMQ;
    int qi = c - g * BMQ;
    col_ok[cg] = qi < nq;
    qi = min(qi, nq - 1);  // padding columns repeat a real row; never stored
    col_row[cg] = q_begin + qi0 + qi;
    col_head[cg] = hbase + g;
    col_pos[cg] = ctx - q_len + qi0 + qi;
  }

  if (ctx < q_len) {  // precondition broken: defined as zeros
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
      if (col_ok[cg])
        for (int d = lg; d < D; d += 4)
          out[((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D + d] = 0;
    return;
  }

  // Q^T fragments (B operand of S^T): column's row, dims 32*ks + 8*lg + 0..7.
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) +
        ((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cg][ks] = as_bf16x8(src[4 * ks + lg]);
  }

  const int pos_first = ctx - q_len + qi0;
  const int ctx_eff = min(ctx, a.max_blocks_per_seq * kBlock);
  const int kv_end = min(pos_first + nq, ctx_eff);
  const int nkt = (kv_end + kBN - 1) / kBN;
  const int32_t *tbl = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);

  f32x4_t o[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) o[mt][cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  auto row_ptr = [&](const uint16_t *pool, int kidx) {
    int pb = tbl[kidx / kBlock];
    pb = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
    return reinterpret_cast<const uint4 *>(
        pool + (((size_t)pb * a.num_kv_heads + kvh) * kBlock + (kidx % kBlock)) * D);
  };

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBN;
    __syncthreads();  // the previous tile is no longer read
    // Stage K: 64 keys x NCH chunks, chunk index XOR-swizzled by key.
    for (int c = threadIdx.x; c < kBN * NCH; c += kThreads) {
      const int key = c / NCH;
      const int ch = c - key * NCH;
      uint4 val = {0u, 0u, 0u, 0u};
      if (k0 + key < kv_end) val = row_ptr(kpool, k0 + key)[ch];
      k_lds[key * NCH + (ch ^ (key % NCH))] = val;
    }
    // Stage V transposed: task = (group of 4 keys, chunk of 8 dims).
    for (int t = threadIdx.x; t < 16 * NCH; t += kThreads) {
      const int kg = t & 15;
      const int j = t >> 4;
      uint32_t w[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kidx = k0 + 4 * kg + i;
        uint4 x = {0u, 0u, 0u, 0u};
        if (kidx < kv_end) x = row_ptr(vpool, kidx)[j];
        w[i][0] = x.x; w[i][1] = x.y; w[i][2] = x.z; w[i][3] = x.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = 8 * j + 2 * e;
        const int d1 = d0 + 1;
        const uint2 even = {(w[0][e] & 0xffffu) | (w[1][e] << 16),
                            (w[2][e] & 0xffffu) | (w[3][e] << 16)};
        const uint2 odd = {(w[0][e] >> 16) | (w[1][e] & 0xffff0000u),
                           (w[2][e] >> 16) | (w[3][e] & 0xffff0000u)};
        vt_lds[d0 * 16 + (kg ^ (d0 & 15))] = even;
        vt_lds[d1 * 16 + (kg ^ (d1 & 15))] = odd;
      }
    }
    __syncthreads();

    // S^T tile: sacc[sub][cg] element r <-> key k0 + 16*sub + 4*lg + r, column cg.
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
        const bf16x8_t af = as_bf16x8(k_lds[key * NCH + ((4 * ks + lg) ^ (key % NCH))]);
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) sacc[sub][cg] = mfma16(af, qf[cg][ks], sacc[sub][cg]);
      }
    }

    const bool edge = (k0 + kBN - 1 > pos_first) || (k0 + kBN > kv_end);
    float p[2][16];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[sub][cg][r] * a.scale_log2;
          if (edge) {
            const int key = k0 + sub * 16 + 4 * lg + r;
            if (key > col_pos[cg] || key >= kv_end) x = -INFINITY;
          }
          p[cg][sub * 4 + r] = x;
        }
    }
    float mx[2];
    bool need = false;
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      float m = p[cg][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, p[cg][i]);
      m = fmaxf(m, shfl_xor(m, 16));
      m = fmaxf(m, shfl_xor(m, 32));
      mx[cg] = m;
      need |= m > mref[cg] + kSlack;
    }
    if (wave_any(need)) {
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const float mn = fmaxf(mref[cg], mx[cg]);
        const float alpha = (mref[cg] == -INFINITY) ? 0.f : fast_exp2(mref[cg] - mn);
        mref[cg] = mn;
        lsum[cg] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt][cg] *= alpha;
      }
    }
    bf16x8_t pf[2][2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[cg][i] = fast_exp2(p[cg][i] - mref[cg]);
        s += p[cg][i];
      }
      lsum[cg] += s;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        uint4 packed;
        packed.x = pack_bf16x2(p[cg][8 * ks2 + 0], p[cg][8 * ks2 + 1]);
        packed.y = pack_bf16x2(p[cg][8 * ks2 + 2], p[cg][8 * ks2 + 3]);
        packed.z = pack_bf16x2(p[cg][8 * ks2 + 4], p[cg][8 * ks2 + 5]);
        packed.w = pack_bf16x2(p[cg][8 * ks2 + 6], p[cg][8 * ks2 + 7]);
        pf[cg][ks2] = as_bf16x8(packed);
      }
    }

    // O^T += V^T P^T: A row = dim, k-slots (lg, e) <-> keys 32*ks2 + 4*lg + e (e < 4)
    // and 32*ks2 + 16 + 4*lg + (e - 4), matching the slots of pf.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int dim = mt * 16 + l16;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const uint2 a0 = vt_lds[dim * 16 + ((8 * ks2 + lg) ^ (dim & 15))];
        const uint2 a1 = vt_lds[dim * 16 + ((8 * ks2 + 4 + lg) ^ (dim & 15))];
        const bf16x8_t af = as_bf16x8(uint4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) o[mt][cg] = mfma16(af, pf[cg][ks2], o[mt][cg]);
      }
    }
  }

  // Epilogue: column totals, normalise, bf16 store of 4 consecutive dims per tile.
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    float L = lsum[cg];
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    if (!col_ok[cg]) continue;
    uint16_t *dst = out + ((size_t)col_row[cg] * a.num_q_heads + col_head[cg]) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint2 packed;
      packed.x = pack_bf16x2(o[mt][cg][0] * inv, o[mt][cg][1] * inv);
      packed.y = pack_bf16x2(o[mt][cg][2] * inv, o[mt][cg][3] * inv);
      *reinterpret_cast<uint2 *>(dst + mt * 16 + 4 * lg) = packed;
    }
  }
}

template <int D, int HGP>
static hipError_t launch_prefill_t(const AttnArgs &a, hipStream_t st) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int nhg = group / HGP;
  const int slots = prefill_tile_slots(a.total_q, a.num_seqs, kCols / HGP);
  const int total = slots * a.num_kv_heads * nhg;
  if (total == 0) return hipSuccess;
  const int grid = ((total + 7) / 8) * 8;
  prefill_mfma_kernel<D, HGP><<<dim3(grid), dim3(kThreads), 0, st>>>(a, nhg, slots);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const AttnArgs &a, hipStream_t st) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 4 == 0) return launch_prefill_t<D, 4>(a, st);
  if (group % 2 == 0) return launch_prefill_t<D, 2>(a, st);
  return launch_prefill_t<D, 1>(a, st);
}

hipError_t launch_prefill(const AttnArgs &a, pkv_dtype dtype, hipStream_t stream) {
  if (dtype != PKV_BF16) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch_prefill_d<64>(a, stream);
  if (a.head_dim == 128) return launch_prefill_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
