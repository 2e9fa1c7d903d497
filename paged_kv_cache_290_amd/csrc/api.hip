// extern "C" entry points of libpagedkv: argument checks, the split-K plan and the
// kernel launches on the caller's stream.  The library is stateless: it allocates
// nothing, frees nothing and never synchronises.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <unordered_set>

#include "pkv_internal.h"

namespace pkv {

namespace {

bool dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Query heads per decode workgroup: the largest of 4, 2, 1 dividing the group whose
// query fragment stays within 512 bytes per lane quarter (keeps registers in check).
int pick_head_group(int group, int head_dim, pkv_dtype dtype) {
  const int elem = dtype == PKV_F32 ? 4 : 2;
  for (int hg = 4; hg > 1; hg >>= 1)
    if (group % hg == 0 && hg * head_dim * elem <= 512) return hg;
  return 1;
}

}  // namespace

// Compute units of the current device (256 on MI355X; also the answer when no device
// is visible, so host-only size queries agree with the GPU).
static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

DecodePlan plan_decode(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len, pkv_dtype dtype, int skip_blocks,
                       bool cascade, bool mixed) {
  DecodePlan p{};
  p.group = num_q_heads / num_kv_heads;
  p.head_group = pick_head_group(p.group, head_dim, dtype);
  p.num_head_groups = p.group / p.head_group;
  p.items = dtype == PKV_F32 ? total_q : num_seqs;
  p.skip_blocks = skip_blocks;
  p.max_context_len = max_context_len;
  p.cascade = cascade;
  // Workgroup size: bf16 waves hold 128 registers (four per SIMD), so a compute unit
  // runs one 16-wave or two 8-wave workgroups.  16 waves per segment while the
  // segments fit the compute units one each; 8 once they do not (two per unit, and the
  // hardware spreads further rounds of workgroups as units free up).  fp32 rows: 8
  // waves of 256 registers, one workgroup per unit.
  const int64_t segments = (int64_t)p.items * num_kv_heads * p.num_head_groups;
  const int64_t cus = device_cus();
  // Decode rows of a mixed launch run in the chunk kernel's 8-wave workgroups.
  p.waves = (dtype == PKV_BF16 && segments <= cus && !mixed) ? kDecodeWavesMax
                                                              : kDecodeWavesMin;
  // Key ranges per segment: one, unless a wave would take more than kBlocksPerWave
  // (kMixedBlocksPerWave in a mixed launch) blocks of the longest row, or the segments
  // leave at least half of the compute units idle and the longest row gives every
  // wave 4 blocks or more (then as many ranges as fit the units in one round,
  // floor(cus / segments), each keeping a block per wave or more).  A second round
  // of workgroups, or a merge launch for a chip that is nearly full or for rows whose
  // workgroups are short chains of round trips, costs more than the idle units.
  const int64_t nb = std::max<int64_t>(
      (max_context_len + kBlock - 1) / kBlock - (int64_t)skip_blocks, 1);
  const int64_t cap = (int64_t)p.waves * (mixed ? kMixedBlocksPerWave : kBlocksPerWave);
  int64_t splits = (nb + cap - 1) / cap;
  if (segments > 0 && segments * splits < cus) {
    const int64_t fill = cus / segments;
    const int64_t keep =  // ranges with >= 1 block per wave, for long rows only
        nb >= 4 * (int64_t)p.waves ? (nb + p.waves - 1) / p.waves : 1;
    splits = std::max(splits, std::min(fill, keep));
  }
  p.splits = (int)std::max<int64_t>(1, std::min<int64_t>(splits, 1 << 16));
  const bool partials = p.splits > 1 || cascade;
  const size_t parts = (size_t)segments * p.splits * p.head_group;
  p.ws_o_offset = 0;
  p.ws_lse_offset = align256(parts * head_dim * sizeof(float));
  p.ws_bytes = (p.items > 0 && partials) ? p.ws_lse_offset + align256(parts * sizeof(float))
                                         : 0;
  return p;
}

PrefillPlan plan_prefill(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                         int head_dim, int max_context_len, pkv_dtype dtype,
                         size_t ws_offset) {
  PrefillPlan p{};
  const int group = num_q_heads / num_kv_heads;
  p.head_group = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  p.num_head_groups = group / p.head_group;
  p.tile_slots = prefill_tile_slots(total_q, num_seqs, kPrefillCols / p.head_group);
  p.tiles = p.tile_slots * num_kv_heads * p.num_head_groups;
  // Split the key range when the tiles cannot fill the compute units, keeping at
  // least two of the kernel's key steps per split.  Rounded up: chunk tiles are long
  // compute-bound workgroups, so a second round of split pieces plus the merge beats
  // units left idle (1,024 rows over 3,500 keys, 136 tiles: 49 us with two splits,
  // 65 us unsplit), unlike the short decode pieces above.
  const int cus = device_cus();
  const int steps = (max_context_len + kPrefillStepKeys - 1) / kPrefillStepKeys;
  p.splits = 1;
  if (dtype == PKV_BF16 && p.tiles > 0 && p.tiles < cus && steps >= 4)
    p.splits = std::max(1, std::min((cus + p.tiles - 1) / p.tiles, steps / 2));
  p.ws_end = ws_offset;
  if (p.splits > 1) {
    const size_t parts = (size_t)p.tiles * p.splits * kPrefillCols;
    p.ws_o_offset = align256(ws_offset);
    p.ws_lse_offset = p.ws_o_offset + align256(parts * head_dim * sizeof(float));
    p.ws_col_offset = p.ws_lse_offset + align256(parts * sizeof(float));
    p.ws_end = p.ws_col_offset + align256((size_t)p.tiles * kPrefillCols * sizeof(int));
  }
  return p;
}

PrefillPlan plan_shared_run(int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                            int shared_keys, size_t ws_offset) {
  PrefillPlan p{};
  const int group = num_q_heads / num_kv_heads;
  p.head_group = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  p.num_head_groups = group / p.head_group;
  const int bm = kPrefillCols / p.head_group;
  p.tile_slots = (total_q + bm - 1) / bm;
  p.tiles = p.tile_slots * num_kv_heads * p.num_head_groups;
  // Enough key splits to fill the compute units, two key steps or more each (fewer
  // splits also mean fewer partials to write and merge: one step per split made the
  // pass 1.1 us shorter and the merge 1.6 us longer on the 187-block workload).
  const int cus = device_cus();
  const int steps = (shared_keys + kPrefillStepKeys - 1) / kPrefillStepKeys;
  p.splits = std::max(1, std::min((cus + p.tiles - 1) / p.tiles, std::max(1, steps / 2)));
  const size_t parts = (size_t)p.tiles * p.splits * kPrefillCols;
  p.ws_o_offset = align256(ws_offset);
  p.ws_lse_offset = p.ws_o_offset + align256(parts * head_dim * sizeof(float));
  p.ws_col_offset = p.ws_lse_offset + align256(parts * sizeof(float));
  p.ws_end = p.ws_col_offset + align256((size_t)p.tiles * kPrefillCols * sizeof(int));
  return p;
}

// Workspace bytes one attention call uses: the decode partials, and after them the
// split-chunk partials when the batch may hold chunks (bf16 rows of q_len >= 2).
// A bf16 batch of several sequences with more query rows than sequences holds a chunk
// (q_len >= 2) and may hold decode rows: it runs as one mixed launch, the chunk tiles
// first and the decode rows in the workgroups after them.  (Batches with as many rows
// as sequences keep separate launches, so that the workspace of a decode batch does not
// depend on whether it could also hold chunks.)
static bool mixed_batch(int num_seqs, int total_q, int max_query_len, pkv_dtype dtype) {
  return dtype == PKV_BF16 && max_query_len > 1 && num_seqs > 1 && total_q > num_seqs;
}

static size_t required_workspace(int num_seqs, int total_q, int num_q_heads,
                                 int num_kv_heads, int head_dim, int max_context_len,
                                 int max_query_len, pkv_dtype dtype) {
  const DecodePlan plan =
      plan_decode(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, max_context_len,
                  dtype, 0, false, mixed_batch(num_seqs, total_q, max_query_len, dtype));
  if (!(dtype == PKV_BF16 && max_query_len > 1)) return plan.ws_bytes;
  return plan_prefill(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                      max_context_len, dtype, plan.ws_bytes)
      .ws_end;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char *pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
  }
  return "unknown status";
}

pkv_status paged_kv_write(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                          const int32_t *slot_mapping, int32_t num_tokens,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, pkv_dtype dtype, void *stream) {
  if (!dtype_ok(dtype) || block_size != kBlock || !head_dim_ok(head_dim))
    return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  const hipError_t e = launch_kv_write(k_new, v_new, k_pool, v_pool, slot_mapping,
                                       num_tokens, num_blocks, num_kv_heads, head_dim, dtype,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, pkv_dtype dtype) {
  if (num_seqs <= 0 || total_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) || !dtype_ok(dtype) ||
      max_context_len < 0)
    return 0;
  // Decode partials first (for a batch that can be mixed, the larger of the plain and
  // the mixed plan: the query does not know max_query_len), then the partials of split
  // prefill chunks.
  size_t dec = plan_decode(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                           max_context_len, dtype)
                   .ws_bytes;
  if (mixed_batch(num_seqs, total_q, 2, dtype))
    dec = std::max(dec, plan_decode(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                    max_context_len, dtype, 0, false, true)
                            .ws_bytes);
  return plan_prefill(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                      max_context_len, dtype, dec)
      .ws_end;
}

}  // extern "C"

namespace {

// Shared body of the two attention entry points.  k_new / v_new / slot_mapping are
// null for the plain call; for the fused call they carry this step's new rows.
pkv_status attention_impl(void *out, const void *q, const void *k_new, const void *v_new,
                          const void *k_pool, const void *v_pool,
                          const int32_t *slot_mapping, const int32_t *block_tables,
                          const int32_t *context_lens, const int32_t *query_start_loc,
                          int32_t num_seqs, int32_t total_q, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, float scale, pkv_dtype dtype,
                          void *workspace, size_t workspace_bytes, void *stream) {
  if (!dtype_ok(dtype) || block_size != kBlock || !head_dim_ok(head_dim))
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q < 0 || num_blocks <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_context_len < 0 ||
      max_query_len < 0 || !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens ||
      !query_start_loc)
    return PKV_ERR_INVALID_ARG;
  const bool with_write = k_new != nullptr;
  if (with_write && (!v_new || !slot_mapping)) return PKV_ERR_INVALID_ARG;

  const bool mixed = mixed_batch(num_seqs, total_q, max_query_len, dtype);
  DecodePlan plan = plan_decode(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                max_context_len, dtype, 0, false, mixed);
  PrefillPlan pplan = plan_prefill(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                   max_context_len, dtype, plan.ws_bytes);
  const size_t need = required_workspace(num_seqs, total_q, num_q_heads, num_kv_heads,
                                         head_dim, max_context_len, max_query_len, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  plan.workspace = workspace;
  pplan.workspace = workspace;

  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)

  const hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16 rows of chunks (q_len >= 2) go to the MFMA kernel, all other rows to the
  // decode kernel; a batch that may hold both runs them in one mixed launch, the slot
  // write first (the chunk tiles read this step's rows from the pool).
  const bool chunks = dtype == PKV_BF16 && max_query_len > 1;
  const bool decode_rows = !(chunks && num_seqs == 1 && total_q > 1);
  hipError_t e = hipSuccess;
  if (with_write) {
    if (dtype == PKV_BF16 && !mixed) {
      // The first bf16 attention launch (the decode kernel, or the chunk kernel of a
      // single sequence) stores the new rows itself and reads this step's keys and
      // values from k_new / v_new (the fused-call precondition places new row i of a
      // sequence at position context_len - q_len + i).  A mixed launch reads them from
      // the pools, written first.
      a.k_new = k_new;
      a.v_new = v_new;
      a.slot_mapping = slot_mapping;
    } else {
      e = launch_kv_write(k_new, v_new, const_cast<void *>(k_pool),
                          const_cast<void *>(v_pool), slot_mapping, total_q, num_blocks,
                          num_kv_heads, head_dim, dtype, st);
    }
  }
  if (mixed) {
    if (e == hipSuccess) e = launch_mixed(a, pplan, plan, st);
    return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  }
  if (e == hipSuccess && decode_rows) e = launch_decode(a, plan, dtype, st);
  if (e == hipSuccess && chunks) {
    AttnArgs ac = a;
    if (decode_rows) {  // the decode launch has stored the new rows
      ac.k_new = nullptr;
      ac.v_new = nullptr;
      ac.slot_mapping = nullptr;
    }
    e = launch_prefill(ac, pplan, dtype, st);
  }
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

pkv_status paged_attention_varlen(void *out, const void *q, const void *k_pool,
                                  const void *v_pool, const int32_t *block_tables,
                                  const int32_t *context_lens,
                                  const int32_t *query_start_loc, int32_t num_seqs,
                                  int32_t total_q, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, float scale, pkv_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  return attention_impl(out, q, nullptr, nullptr, k_pool, v_pool, nullptr, block_tables,
                        context_lens, query_start_loc, num_seqs, total_q, num_blocks,
                        max_blocks_per_seq, max_context_len, max_query_len, num_q_heads,
                        num_kv_heads, head_dim, block_size, scale, dtype, workspace,
                        workspace_bytes, stream);
}

pkv_status paged_attention_varlen_with_write(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    pkv_dtype dtype, void *workspace, size_t workspace_bytes, void *stream) {
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  return attention_impl(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                        context_lens, query_start_loc, num_seqs, total_q, num_blocks,
                        max_blocks_per_seq, max_context_len, max_query_len, num_q_heads,
                        num_kv_heads, head_dim, block_size, scale, dtype, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of the entry point for callers that cannot allocate.  One array per GPU
// (each device holds its own copy of this file-scope array from the moment the code
// object is loaded there until the process ends).  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is taken once per device
// with hipGetSymbolAddress, with that device current, and only that address is ever
// passed to a kernel.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array, or null on a runtime error.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_addr[dev] = ptr;
  }
  return g_scratch_addr[dev];
}

}  // namespace

extern "C" {

pkv_status paged_attention_varlen_with_write_noalloc(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    pkv_dtype dtype, void *stream) {
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  // The size check comes first and needs no device; shapes the attention call rejects
  // are left to its own checks (they need no scratch).
  const bool shapes_ok = dtype_ok(dtype) && block_size == kBlock && head_dim_ok(head_dim) &&
                         num_seqs > 0 && total_q > 0 && num_q_heads > 0 &&
                         num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 &&
                         max_context_len >= 0 && max_query_len >= 0;
  const size_t need = shapes_ok ? required_workspace(num_seqs, total_q, num_q_heads,
                                                     num_kv_heads, head_dim, max_context_len,
                                                     max_query_len, dtype)
                                : 0;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (!ws) return PKV_ERR_LAUNCH;
  }
  return attention_impl(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                        context_lens, query_start_loc, num_seqs, total_q, num_blocks,
                        max_blocks_per_seq, max_context_len, max_query_len, num_q_heads,
                        num_kv_heads, head_dim, block_size, scale, dtype, ws,
                        (size_t)PKV_NOALLOC_SCRATCH_BYTES, stream);
}

size_t paged_attention_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len,
                                                    int32_t shared_blocks, pkv_dtype dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) || dtype != PKV_BF16 ||
      shared_blocks <= 0 || max_context_len < 0)
    return 0;
  // Decode partials of the private keys (8-wave workgroups in the shared run's launch),
  // then the shared run's key splits.
  const DecodePlan dp = plan_decode(num_seqs, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    max_context_len, dtype, shared_blocks, true, true);
  return plan_shared_run(num_seqs, num_q_heads, num_kv_heads, head_dim,
                         shared_blocks * kBlock, dp.ws_bytes)
      .ws_end;
}

pkv_status paged_attention_varlen_shared_prefix(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t shared_blocks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, void *workspace, size_t workspace_bytes, void *stream) {
  const bool with_write = k_new || v_new || slot_mapping;
  if (with_write && !(k_new && v_new && slot_mapping)) return PKV_ERR_INVALID_ARG;
  if (shared_blocks < 0 || max_blocks_per_seq < 0 || shared_blocks > max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if (shared_blocks == 0)  // nothing shared: the plain call
    return attention_impl(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                          context_lens, query_start_loc, num_seqs, total_q, num_blocks,
                          max_blocks_per_seq, max_context_len, max_query_len, num_q_heads,
                          num_kv_heads, head_dim, block_size, scale, dtype, workspace,
                          workspace_bytes, stream);
  if (!dtype_ok(dtype) || block_size != kBlock || !head_dim_ok(head_dim))
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q < 0 || num_blocks <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_context_len < 0 ||
      max_query_len < 0 || !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  // Decode rows (one query per sequence) in bf16.
  if (dtype != PKV_BF16 || max_query_len != 1 || total_q != num_seqs)
    return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens ||
      !query_start_loc)
    return PKV_ERR_INVALID_ARG;

  DecodePlan dp = plan_decode(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                              max_context_len, dtype, shared_blocks, true, true);
  PrefillPlan sp = plan_shared_run(total_q, num_q_heads, num_kv_heads, head_dim,
                                   shared_blocks * kBlock, dp.ws_bytes);
  if (!workspace || workspace_bytes < sp.ws_end) return PKV_ERR_WORKSPACE;
  dp.workspace = workspace;
  sp.workspace = workspace;

  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  if (with_write) {  // the shared-run tiles store the new rows (all past the shared run)
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // The shared run once for every row and the private keys (each row's own blocks) in
  // one launch, then the merge of both parts per row and head.
  hipError_t e = launch_shared_run_mixed(a, sp, shared_blocks * kBlock, dp, st);
  if (e == hipSuccess) e = launch_cascade_merge(a, dp, sp, st);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

pkv_status pkv_validate_shared_prefix(const int32_t *block_tables, const int32_t *context_lens,
                                      const int32_t *query_start_loc, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int32_t shared_blocks,
                                      int32_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (num_seqs < 0 || shared_blocks < 0 || shared_blocks > max_blocks_per_seq ||
      (num_seqs > 0 && (!block_tables || !context_lens || !query_start_loc)))
    return PKV_ERR_INVALID_ARG;
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = query_start_loc[s + 1] - query_start_loc[s];
    bool ok = (int64_t)context_lens[s] - q_len >= (int64_t)shared_blocks * kBlock;
    for (int lb = 0; ok && lb < shared_blocks; ++lb)
      ok = block_tables[(size_t)s * max_blocks_per_seq + lb] == block_tables[lb];
    if (!ok) {
      if (bad_index) *bad_index = s;
      return PKV_ERR_INVALID_ARG;
    }
  }
  return PKV_OK;
}

pkv_status pkv_validate_metadata(const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *query_start_loc, const int32_t *slot_mapping,
                                 int32_t num_seqs, int32_t total_q, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t *bad_index) {
  auto fail = [&](int idx) {
    if (bad_index) *bad_index = idx;
    return PKV_ERR_INVALID_ARG;
  };
  if (bad_index) *bad_index = -1;
  if (num_seqs < 0 || total_q < 0 || num_blocks <= 0 || max_blocks_per_seq < 0)
    return fail(-1);
  if (num_seqs > 0 && (!block_tables || !context_lens || !query_start_loc)) return fail(-1);
  if (num_seqs > 0 && query_start_loc[0] != 0) return fail(0);
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = query_start_loc[s + 1] - query_start_loc[s];
    const int ctx = context_lens[s];
    if (q_len < 0 || q_len > ctx) return fail(s);
    if ((int64_t)ctx > (int64_t)max_blocks_per_seq * kBlock) return fail(s);
    const int used = (ctx + kBlock - 1) / kBlock;
    for (int lb = 0; lb < used; ++lb) {
      const int pb = block_tables[(size_t)s * max_blocks_per_seq + lb];
      if (pb < 0 || pb >= num_blocks) return fail(s);
    }
  }
  if (num_seqs > 0 && query_start_loc[num_seqs] != total_q) return fail(num_seqs);
  if (slot_mapping) {
    std::unordered_set<int64_t> seen;
    seen.reserve((size_t)total_q * 2);
    for (int t = 0; t < total_q; ++t) {
      const int64_t s = slot_mapping[t];
      if (s < 0) continue;
      if (s >= (int64_t)num_blocks * kBlock || !seen.insert(s).second) return fail(t);
    }
  }
  return PKV_OK;
}

pkv_status pkv_validate_fused_metadata(const int32_t *block_tables,
                                       const int32_t *context_lens,
                                       const int32_t *query_start_loc,
                                       const int32_t *slot_mapping, int32_t num_seqs,
                                       int32_t total_q, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (total_q > 0 && !slot_mapping) return PKV_ERR_INVALID_ARG;
  const pkv_status st =
      pkv_validate_metadata(block_tables, context_lens, query_start_loc, slot_mapping,
                            num_seqs, total_q, num_blocks, max_blocks_per_seq, bad_index);
  if (st != PKV_OK) return st;
  // Row i of sequence s (q rows, c keys) is position c - q + i; its slot must be that
  // position's table slot.
  for (int s = 0; s < num_seqs; ++s) {
    const int q0 = query_start_loc[s];
    const int q_len = query_start_loc[s + 1] - q0;
    const int ctx = context_lens[s];
    const int32_t *row = block_tables + (size_t)s * max_blocks_per_seq;
    for (int i = 0; i < q_len; ++i) {
      const int pos = ctx - q_len + i;
      const int64_t want = (int64_t)row[pos / kBlock] * kBlock + pos % kBlock;
      if (slot_mapping[q0 + i] != want) {
        if (bad_index) *bad_index = q0 + i;
        return PKV_ERR_INVALID_ARG;
      }
    }
  }
  return PKV_OK;
}

}  // extern "C"
