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
constexpr int kTblCache = 256;  // block-table entries cached in LDS (4,096 keys)
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

  constexpr int KCH = kBN * NCH / kThreads;          // K chunks per thread per tile
  constexpr int VTASK = 16 * NCH;                     // (4-key group, 8-dim chunk) tasks
  __shared__ uint4 k_lds[2][kBN * NCH];     // [buf][key][chunk ^ (key % NCH)]
  __shared__ uint2 vt_lds[2][D * (kBN / 4)];  // [buf][dim][keygroup ^ (dim % 16)]
  __shared__ int s_tbl[kTblCache];          // block-table entries of this workgroup

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

  // Block-table entries of the keys this workgroup reads, cached in LDS kTblCache at a
  // time (refilled every kTblCache/4 tiles); invalid entries read block 0.
  const int nblk = (kv_end + kBlock - 1) / kBlock;
  auto fill_tbl = [&](int first_blk) {
    for (int i = threadIdx.x; i < kTblCache; i += kThreads) {
      const int lb = first_blk + i;
      int pb = lb < nblk ? tbl[lb] : 0;
      s_tbl[i] = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
    }
  };
  // Staging of a 64-key tile, in two halves so the loads of tile kt+1 are in flight
  // while tile kt is computed.  fetch: global -> registers.  Every load is issued
  // unconditionally (a key past kv_end re-reads the last valid row and is zeroed
  // afterwards), so all of a tile's loads leave back to back.  stage: registers -> LDS
  // buffer `buf`: K row-major with the chunk index XOR-swizzled by key, V transposed
  // (4 keys of one dim per 8 bytes) with key groups swizzled by dim.
  uint4 kreg[KCH];
  uint4 vreg[4];
#define PKV_KEY_ROW(pool, kidx)                                                          \
  (reinterpret_cast<const uint4 *>(                                                      \
      (pool) + (((size_t)s_tbl[((kidx) / kBlock) % kTblCache] * a.num_kv_heads + kvh) *  \
                    kBlock + ((kidx) % kBlock)) * D))
#define PKV_FETCH(kt)                                                                    \
  do {                                                                                   \
    const int k0_ = (kt) * kBN;                                                          \
    _Pragma("unroll") for (int i = 0; i < KCH; ++i) {                                    \
      const int c = threadIdx.x + kThreads * i;                                          \
      const int key = c / NCH;                                                           \
      const int kidx = min(k0_ + key, kv_end - 1);                                       \
      kreg[i] = PKV_KEY_ROW(kpool, kidx)[c - key * NCH];                                 \
    }                                                                                    \
    if (threadIdx.x < VTASK) {                                                           \
      const int kg = threadIdx.x & 15;                                                   \
      const int j = threadIdx.x >> 4;                                                    \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
        const int kidx = min(k0_ + 4 * kg + i, kv_end - 1);                              \
        vreg[i] = PKV_KEY_ROW(vpool, kidx)[j];                                           \
      }                                                                                  \
    }                                                                                    \
  } while (0)
#define PKV_STAGE(kt, buf)                                                               \
  do {                                                                                   \
    const int k0_ = (kt) * kBN;                                                          \
    _Pragma("unroll") for (int i = 0; i < KCH; ++i) {                                    \
      const int c = threadIdx.x + kThreads * i;                                          \
      const int key = c / NCH;                                                           \
      const int ch = c - key * NCH;                                                      \
      const bool live = k0_ + key < kv_end;                                              \
      const uint4 x = kreg[i];                                                           \
      k_lds[buf][key * NCH + (ch ^ (key % NCH))] =                                       \
          uint4{live ? x.x : 0u, live ? x.y : 0u, live ? x.z : 0u, live ? x.w : 0u};     \
    }                                                                                    \
    if (threadIdx.x < VTASK) {                                                           \
      const int kg = threadIdx.x & 15;                                                   \
      const int j = threadIdx.x >> 4;                                                    \
      uint32_t w[4][4];                                                                  \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
        const bool live = k0_ + 4 * kg + i < kv_end;                                     \
        w[i][0] = live ? vreg[i].x : 0u;                                                 \
        w[i][1] = live ? vreg[i].y : 0u;                                                 \
        w[i][2] = live ? vreg[i].z : 0u;                                                 \
        w[i][3] = live ? vreg[i].w : 0u;                                                 \
      }                                                                                  \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                    \
        const int d0 = 8 * j + 2 * e;                                                    \
        const int d1 = d0 + 1;                                                           \
        vt_lds[buf][d0 * 16 + (kg ^ (d0 & 15))] =                                        \
            uint2{(w[0][e] & 0xffffu) | (w[1][e] << 16),                                 \
                  (w[2][e] & 0xffffu) | (w[3][e] << 16)};                                \
        vt_lds[buf][d1 * 16 + (kg ^ (d1 & 15))] =                                        \
            uint2{(w[0][e] >> 16) | (w[1][e] & 0xffff0000u),                             \
                  (w[2][e] >> 16) | (w[3][e] & 0xffff0000u)};                            \
      }                                                                                  \
    }                                                                                    \
  } while (0)

  fill_tbl(0);
  __syncthreads();
  if (nkt > 0) {
    PKV_FETCH(0);
    PKV_STAGE(0, 0);
  }
  __syncthreads();
  // Retire every outstanding load (the query fragments in particular) on all paths
  // here.  Otherwise the wait counters merged at the loop head still see the query
  // loads in flight, and each MFMA that reads them waits for the next tile's
  // prefetch as well, which undoes the overlap.
  __builtin_amdgcn_s_waitcnt(0);

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBN;
    const int buf = kt & 1;
    // Refill the table cache before the first fetch that needs new entries.
    if (kt + 1 < nkt && ((kt + 1) * (kBN / kBlock)) % kTblCache == 0) {
      fill_tbl((kt + 1) * (kBN / kBlock));
      __syncthreads();
    }
    if (kt + 1 < nkt) PKV_FETCH(kt + 1);  // in flight while this tile is computed

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
        const bf16x8_t af = as_bf16x8(k_lds[buf][key * NCH + ((4 * ks + lg) ^ (key % NCH))]);
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
        const uint2 a0 = vt_lds[buf][dim * 16 + ((8 * ks2 + lg) ^ (dim & 15))];
        const uint2 a1 = vt_lds[buf][dim * 16 + ((8 * ks2 + 4 + lg) ^ (dim & 15))];
        const bf16x8_t af = as_bf16x8(uint4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) o[mt][cg] = mfma16(af, pf[cg][ks2], o[mt][cg]);
      }
    }
    if (kt + 1 < nkt) PKV_STAGE(kt + 1, buf ^ 1);
    __syncthreads();  // tile kt+1 staged; everyone is done reading tile kt
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

#undef PKV_KEY_ROW
#undef PKV_FETCH
#undef PKV_STAGE

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
