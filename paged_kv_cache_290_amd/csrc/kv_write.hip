// Slot-mapping write of this step's new K/V rows into the paged pool.
//
// Serving-engine KV page (ttlab), section 2 "PagedAttention", "blocks and block
// table": K/V are stored in fixed 16-token physical blocks; a token's home is
// (block, offset).  Inference-engine page (xiaohu-jiedu), KV-cache section: each step
// produces K/V only for its new tokens, which are appended to the cache.
//
// Each thread moves one 16-byte piece of one (token, kv head) row of K and the same
// piece of V.  Reads of k_new / v_new are fully coalesced; each written row is a
// contiguous run of head_dim * elem bytes inside a (block, kv head) tile.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int ROW_VECS>  // 16-byte pieces per (token, kv head) row
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
    uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
    const int32_t *__restrict__ slot_mapping, int64_t total_vecs, int num_kv_heads,
    int64_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total_vecs) return;
  const int64_t per_token = (int64_t)num_kv_heads * ROW_VECS;
  const int64_t t = i / per_token;
  const int rem = (int)(i - t * per_token);
  const int h = rem / ROW_VECS;
  const int piece = rem - h * ROW_VECS;
  // The row data does not depend on the slot: load both at once.
  const uint4 kx = k_new[i];
  const uint4 vx = v_new[i];
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped token (or out of range)
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot % kBlock);
  const int64_t dst = ((blk * num_kv_heads + h) * kBlock + off) * ROW_VECS + piece;
  k_pool[dst] = kx;
  v_pool[dst] = vx;
}

hipError_t launch_kv_write(const void *k_new, const void *v_new, void *k_pool,
                           void *v_pool, const int32_t *slot_mapping, int num_tokens,
                           int num_blocks, int num_kv_heads, int head_dim, pkv_dtype dtype,
                           hipStream_t stream) {
  const int row_bytes = head_dim * (dtype == PKV_F32 ? 4 : 2);
  const int row_vecs = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * row_vecs;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + kThreads - 1) / kThreads;
  const int64_t num_slots = (int64_t)num_blocks * kBlock;
  auto *kn = static_cast<const uint4 *>(k_new);
  auto *vn = static_cast<const uint4 *>(v_new);
  auto *kp = static_cast<uint4 *>(k_pool);
  auto *vp = static_cast<uint4 *>(v_pool);
  switch (row_vecs) {
    case 8:   // 64 x bf16
      kv_write_kernel<8><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
          kn, vn, kp, vp, slot_mapping, total, num_kv_heads, num_slots);
      break;
    case 16:  // 128 x bf16 or 64 x f32
      kv_write_kernel<16><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
          kn, vn, kp, vp, slot_mapping, total, num_kv_heads, num_slots);
      break;
    case 32:  // 128 x f32
      kv_write_kernel<32><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
          kn, vn, kp, vp, slot_mapping, total, num_kv_heads, num_slots);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
