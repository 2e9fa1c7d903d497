// Decode attention over the paged KV pool: split-K over the context, then a merge.
//
// Method (pages cited by title and section):
//  * Inference-engine page (xiaohu-jiedu), prefill/decode section: a decode step has
//    one new query per request and must read the whole cached context, so it is
//    bound by memory bandwidth, not arithmetic.
//  * Serving-engine KV page (ttlab), section 2, "blocks and block table": K/V sit in
//    16-token blocks anywhere in the pool; the kernel follows the request's block
//    table and must give the same result as a contiguous cache.
//
// Work item = (row, kv head, group of HG q heads, split of `bps` logical blocks).
// One workgroup of 4 waves per item; wave w takes blocks w, w+4, ... of the split.
// Lane mapping inside a wave, for one (block, kv head) tile of 16 x D elements:
// lane = 4*token + quarter, so a lane owns D/4 consecutive dims of one token, and a
// wave reads the whole contiguous tile (2-8 KB) with 16-byte loads.  Each K/V tile
// is loaded once and used for all HG query heads (grouped-query reuse).
//
// Softmax runs in log2 units (scores times scale*log2 e, exp2).  Every lane keeps
// its own running sum and accumulator for its token slot, all scaled by one
// wave-uniform reference max per head.  The reference is raised only when some
// score exceeds it by more than kRescaleSlack (then every lane rescales), so the
// usual per-block cross-lane max is replaced by one ballot.  Terms are at most
// 2^kRescaleSlack, far from fp32 overflow for any context length in int32.
// The lanes' partial sums are combined once at the end (DPP inside rows of 16 lanes,
// then LDS across rows and waves).
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr float kRescaleSlack = 8.0f;

template <typename T, int D>
struct DecodeFrag {
  static constexpr int kDimsPerLane = D / 4;
  static constexpr int kVecs = kDimsPerLane * (int)sizeof(T) / 16;  // uint4 per lane
  static constexpr int kWords = kVecs * 4;                          // dwords per lane
};

// Row handled by work item `item`, and how many keys it sees (0 when the sequence
// breaks q_len <= context_len).  Returns false when the item is not a decode row.
template <bool kRows>
__device__ __forceinline__ bool decode_row(const AttnArgs &a, int item, int &seq, int &row,
                                           int &row_keys) {
  if constexpr (kRows) {
    row = item;
    seq = find_seq(a.query_start_loc, a.num_seqs, row);
  } else {
    seq = item;
    row = a.query_start_loc[seq];
    if (a.query_start_loc[seq + 1] - row != 1) return false;  // prefill: MFMA path
    if (row < 0 || row >= a.total_q) return false;
  }
  const int q_begin = a.query_start_loc[seq];
  const int q_len = a.query_start_loc[seq + 1] - q_begin;
  const int ctx = a.context_lens[seq];
  row_keys = ctx - q_len + (row - q_begin) + 1;
  row_keys = min(row_keys, a.max_blocks_per_seq * kBlock);
  if (ctx < q_len) row_keys = 0;
  return true;
}

template <typename T, int D, int HG>
__global__ __launch_bounds__(kThreads) void decode_splitk_kernel(AttnArgs a, int items,
                                                                 int num_head_groups,
                                                                 int bps, int num_splits) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  using Fr = DecodeFrag<T, D>;
  constexpr int DPL = Fr::kDimsPerLane;
  constexpr int NV = Fr::kVecs;
  constexpr int NW = Fr::kWords;

  __shared__ float s_acc[kWaves][4][HG][D];
  __shared__ float s_l[kWaves][4][HG];
  __shared__ float s_m[kWaves][HG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok = lane >> 2;
  const int quarter = lane & 3;

  const int total = items * a.num_kv_heads * num_head_groups * num_splits;
  int v = xcd_remap(blockIdx.x, total);
  if (v >= total) return;
  const int item = v % items;
  v /= items;
  const int split = v % num_splits;
  v /= num_splits;
  const int hgi = v % num_head_groups;
  const int kvh = v / num_head_groups;

  int seq, row, row_keys;
  if (!decode_row<kF32>(a, item, seq, row, row_keys)) return;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int h0 = kvh * group + hgi * HG;
  T *out = static_cast<T *>(a.out);

  if (row_keys <= 0) {  // q_len > context_len: defined as zeros
    if (split == 0)
      for (int o = threadIdx.x; o < HG * D; o += kThreads)
        out[((size_t)row * a.num_q_heads + h0) * D + o] = T(0);
    return;
  }
  // The split plan comes from the host's max_context_len; a longer row is cut there.
  const int nblk = min((row_keys + kBlock - 1) / kBlock, num_splits * bps);
  row_keys = min(row_keys, nblk * kBlock);
  const int row_splits = (nblk + bps - 1) / bps;
  if (split >= row_splits) return;
  const int b0 = split * bps;
  const int b1 = min(nblk, b0 + bps);
  const int nb_w = (b1 - b0 > wave) ? (b1 - b0 - wave + kWaves - 1) / kWaves : 0;

  // Query fragment: this lane's D/4 dims of each of the HG heads.
  uint32_t qw[HG][NW];
  {
    const T *qp = static_cast<const T *>(a.q) + ((size_t)row * a.num_q_heads + h0) * D +
                  quarter * DPL;
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const uint4 *src = reinterpret_cast<const uint4 *>(qp + g * D);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint4 x = src[j];
        qw[g][4 * j + 0] = x.x;
        qw[g][4 * j + 1] = x.y;
        qw[g][4 * j + 2] = x.z;
        qw[g][4 * j + 3] = x.w;
      }
      if constexpr (kF32) {  // fold the softmax scale into q once
#pragma unroll
        for (int i = 0; i < NW; ++i)
          qw[g][i] = __float_as_uint(__uint_as_float(qw[g][i]) * a.scale_log2);
      }
    }
  }

  // Physical block ids of this wave's blocks: lane i holds the i-th (bps <= 256, so
  // a wave has at most 64 blocks in a split).
  int my_pb = 0;
  {
    const int32_t *tbl = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    if (lane < nb_w) my_pb = tbl[b0 + wave + kWaves * lane];
  }

  float acc[HG][DPL];
  float lsum[HG];
  float mref[HG];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    lsum[g] = 0.f;
    mref[g] = -INFINITY;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[g][d] = 0.f;
  }

  const size_t tile_elems = (size_t)kBlock * D;
  auto tile_base = [&](const void *pool, int pb) {
    return reinterpret_cast<const uint4 *>(static_cast<const T *>(pool) +
                                           ((size_t)pb * a.num_kv_heads + kvh) * tile_elems) +
           lane * NV;
  };
  auto load = [&](uint4 (&kr)[NV], uint4 (&vr)[NV], int i) {
    int pb = readlane(my_pb, i);
    pb = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
    const uint4 *kp = tile_base(a.k_pool, pb);
    const uint4 *vp = tile_base(a.v_pool, pb);
#pragma unroll
    for (int j = 0; j < NV; ++j) kr[j] = kp[j];
#pragma unroll
    for (int j = 0; j < NV; ++j) vr[j] = vp[j];
  };
  auto compute = [&](const uint4 (&kr)[NV], const uint4 (&vr)[NV], int i) {
    const int lb = b0 + wave + kWaves * i;
    const int pb = readlane(my_pb, i);
    const bool bad = pb < 0 || pb >= a.num_blocks;
    const bool valid = !bad && (lb * kBlock + tok) < row_keys;
    uint32_t kw[NW], vw[NW];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      kw[4 * j + 0] = kr[j].x; kw[4 * j + 1] = kr[j].y;
      kw[4 * j + 2] = kr[j].z; kw[4 * j + 3] = kr[j].w;
      vw[4 * j + 0] = vr[j].x; vw[4 * j + 1] = vr[j].y;
      vw[4 * j + 2] = vr[j].z; vw[4 * j + 3] = vr[j].w;
    }
    float s[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      float x = 0.f;
      if constexpr (kF32) {
#pragma unroll
        for (int w = 0; w < NW; ++w) x = fmaf(__uint_as_float(qw[g][w]), __uint_as_float(kw[w]), x);
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) x = dot2_bf16(qw[g][w], kw[w], x);
      }
      x += dpp<kQuadSwap1>(x);
      x += dpp<kQuadSwap2>(x);
      if constexpr (!kF32) x *= a.scale_log2;
      s[g] = valid ? x : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < HG; ++g) need |= s[g] > mref[g] + kRescaleSlack;
    if (wave_any(need)) {
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const float mx = wave_max_over_quads(s[g]);
        const float mn = fmaxf(mref[g], mx);
        const float alpha = (mref[g] == -INFINITY) ? 0.f : fast_exp2(mref[g] - mn);
        mref[g] = mn;
        lsum[g] *= alpha;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[g][d] *= alpha;
      }
    }
    float p[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      p[g] = valid ? fast_exp2(s[g] - mref[g]) : 0.f;
      lsum[g] += p[g];
    }
    // Slots past the context (and tiles of invalid blocks) may hold anything,
    // including NaN: their weight is 0 and their values are replaced by 0.
    if (bad || (lb + 1) * kBlock > row_keys) {
#pragma unroll
      for (int w = 0; w < NW; ++w) vw[w] = valid ? vw[w] : 0u;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if constexpr (kF32) {
        const float x = __uint_as_float(vw[w]);
#pragma unroll
        for (int g = 0; g < HG; ++g) acc[g][w] = fmaf(p[g], x, acc[g][w]);
      } else {
        const float lo = bf16_lo(vw[w]);
        const float hi = bf16_hi(vw[w]);
#pragma unroll
        for (int g = 0; g < HG; ++g) {
          acc[g][2 * w] = fmaf(p[g], lo, acc[g][2 * w]);
          acc[g][2 * w + 1] = fmaf(p[g], hi, acc[g][2 * w + 1]);
        }
      }
    }
  };

  if (nb_w > 0) {
    uint4 kA[NV], vA[NV], kB[NV], vB[NV];
    load(kA, vA, 0);
    int i = 0;
    for (; i + 1 < nb_w; i += 2) {
      load(kB, vB, i + 1);
      compute(kA, vA, i);
      if (i + 2 < nb_w) load(kA, vA, i + 2);
      compute(kB, vB, i + 1);
    }
    if (i < nb_w) compute(kA, vA, i);
  }

  // Combine the 4 token slots of each 16-lane row (same quarter = same dims).
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    lsum[g] += dpp<kRowRor4>(lsum[g]);
    lsum[g] += dpp<kRowRor8>(lsum[g]);
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      acc[g][d] += dpp<kRowRor4>(acc[g][d]);
      acc[g][d] += dpp<kRowRor8>(acc[g][d]);
    }
  }
  if ((lane & 15) < 4) {
    const int r = lane >> 4;
#pragma unroll
    for (int g = 0; g < HG; ++g) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) s_acc[wave][r][g][quarter * DPL + d] = acc[g][d];
      if (quarter == 0) s_l[wave][r][g] = lsum[g];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < HG; ++g) s_m[wave][g] = mref[g];
  }
  __syncthreads();

  for (int o = threadIdx.x; o < HG * D; o += kThreads) {
    const int g = o / D;
    const int d = o - g * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = (s_m[w][g] == -INFINITY) ? 0.f : fast_exp2(s_m[w][g] - mx);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        L = fmaf(wt, s_l[w][r][g], L);
        O = fmaf(wt, s_acc[w][r][g][d], O);
      }
    }
    const float res = (L > 0.f) ? O / L : 0.f;
    const int h = h0 + g;
    if (row_splits == 1) {
      if constexpr (kF32) out[((size_t)row * a.num_q_heads + h) * D + d] = res;
      else out[((size_t)row * a.num_q_heads + h) * D + d] = f32_to_bf16(res);
    } else {
      const size_t slot = ((size_t)item * a.num_q_heads + h) * num_splits + split;
      a.ws_o[slot * D + d] = res;
      if (d == 0) a.ws_lse[slot] = (L > 0.f) ? mx + __builtin_amdgcn_logf(L) : -INFINITY;
    }
  }
}

// Log-sum-exp merge of the split partials: with per-split (o_i, lse_i) in log2 units,
// out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i.  One wave per
// (row, q head); rows with a single split were finished by the decode kernel.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a, int items, int bps,
                                                         int num_splits) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int DW = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x * kWaves + wave;
  if (w >= items * a.num_q_heads) return;
  const int item = w / a.num_q_heads;
  const int h = w - item * a.num_q_heads;
  int seq, row, row_keys;
  if (!decode_row<kF32>(a, item, seq, row, row_keys)) return;
  if (row_keys <= 0) return;
  const int nblk = min((row_keys + kBlock - 1) / kBlock, num_splits * bps);
  const int row_splits = (nblk + bps - 1) / bps;
  if (row_splits <= 1) return;

  const size_t base = ((size_t)item * a.num_q_heads + h) * num_splits;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < row_splits; s0 += 64)
    if (s0 + lane < row_splits) mx = fmaxf(mx, a.ws_lse[base + s0 + lane]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mx = fmaxf(mx, shfl_xor(mx, m));

  float L = 0.f;
  float o[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < row_splits; s0 += 64) {
    const float lse = (s0 + lane < row_splits) ? a.ws_lse[base + s0 + lane] : -INFINITY;
    const float wt = (lse == -INFINITY) ? 0.f : fast_exp2(lse - mx);
    const int n = min(64, row_splits - s0);
    for (int j = 0; j < n; ++j) {
      const float wj = __int_as_float(readlane(__float_as_int(wt), j));
      L += wj;
      const float *src = a.ws_o + (base + s0 + j) * D;
#pragma unroll
      for (int e = 0; e < DW; ++e) o[e] = fmaf(wj, src[lane + 64 * e], o[e]);
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

template <typename T, int D, int HG>
static hipError_t launch_decode_t(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  const int total = p.items * a.num_kv_heads * p.num_head_groups * p.num_splits;
  if (total == 0) return hipSuccess;
  const int grid = ((total + 7) / 8) * 8;
  decode_splitk_kernel<T, D, HG><<<dim3(grid), dim3(kThreads), 0, st>>>(
      a, p.items, p.num_head_groups, p.blocks_per_split, p.num_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits <= 1) return e;
  const int waves = p.items * a.num_q_heads;
  merge_kernel<T, D><<<dim3((waves + kWaves - 1) / kWaves), dim3(kThreads), 0, st>>>(
      a, p.items, p.blocks_per_split, p.num_splits);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const AttnArgs &a, const DecodePlan &p, hipStream_t st) {
  switch (p.head_group) {
    case 1: return launch_decode_t<T, D, 1>(a, p, st);
    case 2: return launch_decode_t<T, D, 2>(a, p, st);
    case 4: return launch_decode_t<T, D, 4>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const AttnArgs &a, const DecodePlan &p, pkv_dtype dtype,
                         hipStream_t stream) {
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
