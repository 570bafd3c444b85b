// Cache write for chunked prefill: the keys and values of new tokens go into
// the paged pool before the chunk's attention reads them (VPP technical
// review, English edition, §2.3: every later chunk attends to the cache of
// all earlier chunks).  A bitwise copy into the pool layout the attention
// kernels read:
//   K pool [block, kv_head, D/X, 64, X]   (16-byte feature runs, token-interleaved)
//   V pool [block, kv_head, 64/X, DV, X]  (16-byte token runs, feature-interleaved)
// K moves in 16-byte chunks; V is transposed element by element, so a partly
// filled 16-byte run keeps the tokens already written around it.
#include "device_common.h"
#include "launch.h"

namespace chunkattn {

template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                       int64_t start_pos, int64_t n_tokens, int kv_heads,
                                                       int D, int DV, const int32_t* __restrict__ block_table,
                                                       int num_blocks, E* __restrict__ k_pool,
                                                       E* __restrict__ v_pool) {
  constexpr int X = Elem<E>::X;
  const int64_t nk = n_tokens * kv_heads * (D / X);
  const int64_t nv = n_tokens * kv_heads * DV;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nk + nv; idx += stride) {
    if (idx < nk) {
      const int dc = (int)(idx % (D / X));
      const int64_t tg = idx / (D / X);
      const int g = (int)(tg % kv_heads);
      const int64_t tok = start_pos + tg / kv_heads;
      const int64_t phys = clamp_block(block_table[tok / kBlock], num_blocks);
      const int slot = (int)(tok % kBlock);
      const u32x4_t v = *(const u32x4_t*)(k_new + tg * D + dc * X);
      *(u32x4_t*)(k_pool + (((phys * kv_heads + g) * (D / X) + dc) * kBlock + slot) * X) = v;
    } else {
      const int64_t e = idx - nk;
      const int dv = (int)(e % DV);
      const int64_t tg = e / DV;
      const int g = (int)(tg % kv_heads);
      const int64_t tok = start_pos + tg / kv_heads;
      const int64_t phys = clamp_block(block_table[tok / kBlock], num_blocks);
      const int slot = (int)(tok % kBlock);
      v_pool[(((phys * kv_heads + g) * (kBlock / X) + slot / X) * DV + dv) * X + slot % X] = v_new[tg * DV + dv];
    }
  }
}

// Identity block table t[i] = i: lets a contiguous cache, re-laid into a
// scratch pool block by block, be read by the paged kernels.
__global__ __launch_bounds__(256) void block_iota_kernel(int32_t* __restrict__ t, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) t[i] = i;
}

hipError_t launch_block_iota(int32_t* table, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_iota_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, table, n);
  return hipGetLastError();
}

hipError_t launch_kv_append(DType dt, int D, int DV, const void* k_new, const void* v_new,
                            int64_t start_pos, int64_t n_tokens, int kv_heads,
                            const int32_t* block_table, int num_blocks, void* k_pool, void* v_pool,
                            hipStream_t stream) {
  const int64_t work = n_tokens * kv_heads * (int64_t)(D + DV);
  const int64_t want = (work + 255) / 256;
  const int grid = (int)(want < 65536 ? (want < 1 ? 1 : want) : 65536);
  if (dt == DType::BF16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, start_pos, n_tokens, kv_heads, D, DV, block_table, num_blocks,
                       (uint16_t*)k_pool, (uint16_t*)v_pool);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(grid), dim3(256), 0, stream, (const float*)k_new,
                       (const float*)v_new, start_pos, n_tokens, kv_heads, D, DV, block_table, num_blocks,
                       (float*)k_pool, (float*)v_pool);
  return hipGetLastError();
}

}  // namespace chunkattn
