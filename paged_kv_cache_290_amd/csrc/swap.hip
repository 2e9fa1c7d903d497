// KV swap between the GPU pools and host memory: whole blocks are gathered into a
// contiguous device staging buffer and copied to host memory with one asynchronous
// DMA copy (swap-out), or copied back and scattered into the blocks free at that time
// (swap-in).
//
// Method (pages cited by title and section):
//  * "How inference engines actually work" page (xiaohu-jiedu), agent-traffic section:
//    while a request waits on a tool, its KV cache moves to larger, cheaper CPU memory
//    and is brought back when its next turn arrives.
//  * Serving-engine KV page (ttlab), section 5: the alternative is preemption, where
//    the request drops its KV and is prefilled again later.
//
// Host image layout: K of the n blocks, then V of the n blocks, each block as it lies
// in a pool (num_kv_heads * 16 * head_dim elements).
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// staging[(pool * n + i) * block_vecs + piece] <-> pool[blocks[i] * block_vecs + piece]:
// gather (to_staging) or scatter, 16-byte pieces, grid-stride.  A block id outside the
// pool gathers zeros and scatters nothing.
template <bool kToStaging>
__global__ __launch_bounds__(kThreads) void swap_kernel(uint4 *__restrict__ k_pool,
                                                        uint4 *__restrict__ v_pool,
                                                        uint4 *__restrict__ staging,
                                                        const int32_t *__restrict__ blocks,
                                                        int n, int num_blocks,
                                                        int64_t block_vecs) {
  const int64_t per_pool = (int64_t)n * block_vecs;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < 2 * per_pool;
       idx += (int64_t)gridDim.x * kThreads) {
    const bool is_v = idx >= per_pool;
    const int64_t rem = is_v ? idx - per_pool : idx;
    const int i = (int)(rem / block_vecs);
    const int64_t piece = rem - (int64_t)i * block_vecs;
    const int b = blocks[i];
    const bool ok = b >= 0 && b < num_blocks;
    uint4 *pool = is_v ? v_pool : k_pool;
    if constexpr (kToStaging) {
      staging[idx] = ok ? pool[(int64_t)b * block_vecs + piece] : uint4{0u, 0u, 0u, 0u};
    } else {
      if (ok) pool[(int64_t)b * block_vecs + piece] = staging[idx];
    }
  }
}

namespace {

pkv_status check_swap(const void *k_pool, const void *v_pool, const int32_t *blocks,
                      int32_t n, const void *staging, const void *host, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      pkv_dtype dtype) {
  if ((dtype != PKV_F32 && dtype != PKV_BF16) || block_size != kBlock ||
      (head_dim != 64 && head_dim != 128))
    return PKV_ERR_UNSUPPORTED;
  if (n < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!k_pool || !v_pool || !blocks || !staging || !host))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

int grid_for(int64_t total) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  const int64_t want = (total + kThreads - 1) / kThreads;
  return (int)(want < (int64_t)cus * 8 ? want : (int64_t)cus * 8);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

size_t paged_kv_swap_bytes(int32_t n, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pkv_dtype dtype) {
  if (n <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size != kBlock ||
      (dtype != PKV_F32 && dtype != PKV_BF16))
    return 0;
  return (size_t)2 * n * num_kv_heads * kBlock * head_dim * (dtype == PKV_F32 ? 4 : 2);
}

pkv_status paged_kv_swap_out(const void *k_pool, const void *v_pool, const int32_t *blocks,
                             int32_t n, void *staging, void *host, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             pkv_dtype dtype, void *stream) {
  const pkv_status c = check_swap(k_pool, v_pool, blocks, n, staging, host, num_blocks,
                                  num_kv_heads, head_dim, block_size, dtype);
  if (c != PKV_OK || n == 0) return c;
  const size_t bytes = paged_kv_swap_bytes(n, num_kv_heads, head_dim, block_size, dtype);
  const int64_t block_vecs = (int64_t)bytes / 2 / n / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  swap_kernel<true><<<dim3(grid_for(2 * n * block_vecs)), dim3(kThreads), 0, st>>>(
      static_cast<uint4 *>(const_cast<void *>(k_pool)),
      static_cast<uint4 *>(const_cast<void *>(v_pool)), static_cast<uint4 *>(staging),
      blocks, n, num_blocks, block_vecs);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  if (hipMemcpyAsync(host, staging, bytes, hipMemcpyDeviceToHost, st) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

pkv_status paged_kv_swap_in(void *k_pool, void *v_pool, const int32_t *blocks, int32_t n,
                            void *staging, const void *host, int32_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            pkv_dtype dtype, void *stream) {
  const pkv_status c = check_swap(k_pool, v_pool, blocks, n, staging, host, num_blocks,
                                  num_kv_heads, head_dim, block_size, dtype);
  if (c != PKV_OK || n == 0) return c;
  const size_t bytes = paged_kv_swap_bytes(n, num_kv_heads, head_dim, block_size, dtype);
  const int64_t block_vecs = (int64_t)bytes / 2 / n / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(staging, host, bytes, hipMemcpyHostToDevice, st) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
  }
  swap_kernel<false><<<dim3(grid_for(2 * n * block_vecs)), dim3(kThreads), 0, st>>>(
      static_cast<uint4 *>(k_pool), static_cast<uint4 *>(v_pool),
      static_cast<uint4 *>(staging), blocks, n, num_blocks, block_vecs);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
