// Cache write for chunked prefill: the keys and values of new tokens go into
// the paged pool before the chunk's attention reads them (VPP technical
// review, English edition, §2.3: every later chunk attends to the cache of
// all earlier chunks).  A bitwise copy into the pool layout the attention
// kernels read:
//   K pool [block, kv_head, D/X, 64, X]   (16-byte feature runs, token-interleaved)
//   V pool [block, kv_head, 64/X, DV, X]  (16-byte token runs, feature-interleaved)
// K moves in 16-byte chunks.  V is transposed: in bf16, a work item takes one
// 8-token run of one KV head and two adjacent values, reads 8 x 4 bytes (a
// wave covers 256 contiguous bytes of each token row) and writes two whole
// 16-byte runs; a run only partly inside the appended range, and fp32 V,
// are written element by element, which keeps the tokens around them.
#include "device_common.h"
#include "launch.h"

namespace chunkattn {

template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                       int64_t k_tok, int64_t k_head, int64_t v_tok, int64_t v_head,
                                                       int64_t start_pos, int64_t n_tokens, int kv_heads,
                                                       int D, int DV, const int32_t* __restrict__ block_table,
                                                       int num_blocks, E* __restrict__ k_pool,
                                                       E* __restrict__ v_pool, bool with_v) {
  constexpr int X = Elem<E>::X;
  const int64_t nk = n_tokens * kv_heads * (D / X);
  const int64_t nv = with_v ? n_tokens * kv_heads * DV : 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nk + nv; idx += stride) {
    if (idx < nk) {
      const int dc = (int)(idx % (D / X));
      const int64_t tg = idx / (D / X);
      const int g = (int)(tg % kv_heads);
      const int64_t tok = start_pos + tg / kv_heads;
      const int64_t phys = clamp_block(block_table[tok / kBlock], num_blocks);
      const int slot = (int)(tok % kBlock);
      const u32x4_t v = *(const u32x4_t*)(k_new + (tg / kv_heads) * k_tok + g * k_head + dc * X);
      *(u32x4_t*)(k_pool + (((phys * kv_heads + g) * (D / X) + dc) * kBlock + slot) * X) = v;
    } else {
      const int64_t e = idx - nk;
      const int dv = (int)(e % DV);
      const int64_t tg = e / DV;
      const int g = (int)(tg % kv_heads);
      const int64_t tok = start_pos + tg / kv_heads;
      const int64_t phys = clamp_block(block_table[tok / kBlock], num_blocks);
      const int slot = (int)(tok % kBlock);
      v_pool[(((phys * kv_heads + g) * (kBlock / X) + slot / X) * DV + dv) * X + slot % X] =
          v_new[(tg / kv_heads) * v_tok + g * v_head + dv];
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

// bf16 V by 8-token runs (see the header comment).  Work item: (run, head,
// value pair), value pair fastest.
__global__ __launch_bounds__(256) void kv_append_v_bf16_kernel(const uint16_t* __restrict__ v_new, int64_t v_tok,
                                                               int64_t v_head, int64_t start_pos,
                                                               int64_t n_tokens, int kv_heads, int DV,
                                                               const int32_t* __restrict__ block_table,
                                                               int num_blocks, uint16_t* __restrict__ v_pool) {
  constexpr int X = 8;
  const int64_t run0 = start_pos / X, run1 = (start_pos + n_tokens - 1) / X;
  const int pairs = DV / 2;
  const int64_t items = (run1 - run0 + 1) * kv_heads * pairs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < items; idx += stride) {
    const int dp = (int)(idx % pairs);
    const int64_t rg = idx / pairs;
    const int g = (int)(rg % kv_heads);
    const int64_t run = run0 + rg / kv_heads;
    const int64_t tok0 = run * X;                             // runs never straddle a block
    const int64_t phys = clamp_block(block_table[tok0 / kBlock], num_blocks);
    uint16_t* dst = v_pool + (((phys * kv_heads + g) * (kBlock / X) + (tok0 % kBlock) / X) * DV + 2 * dp) * X;
    if (tok0 >= start_pos && tok0 + X <= start_pos + n_tokens) {
      const uint32_t* src = (const uint32_t*)(v_new + (tok0 - start_pos) * v_tok + g * v_head + 2 * dp);
      uint32_t w[X];
#pragma unroll
      for (int t = 0; t < X; ++t) w[t] = src[t * (v_tok / 2)];
      u32x4_t lo, hi;                                         // value 2dp, value 2dp + 1 of tokens 0..7
#pragma unroll
      for (int t = 0; t < X / 2; ++t) {
        lo[t] = (w[2 * t] & 0xffffu) | (w[2 * t + 1] << 16);
        hi[t] = (w[2 * t] >> 16) | (w[2 * t + 1] & 0xffff0000u);
      }
      *(u32x4_t*)dst = lo;
      *(u32x4_t*)(dst + X) = hi;
    } else {
      for (int t = 0; t < X; ++t) {
        const int64_t tok = tok0 + t;
        if (tok < start_pos || tok >= start_pos + n_tokens) continue;
        const uint16_t* src = v_new + (tok - start_pos) * v_tok + g * v_head + 2 * dp;
        dst[t] = src[0];
        dst[X + t] = src[1];
      }
    }
  }
}

hipError_t launch_kv_append(DType dt, int D, int DV, const void* k_new, const void* v_new,
                            int64_t k_tok, int64_t k_head, int64_t v_tok, int64_t v_head,
                            int64_t start_pos, int64_t n_tokens, int kv_heads,
                            const int32_t* block_table, int num_blocks, void* k_pool, void* v_pool,
                            hipStream_t stream) {
  auto grid_for = [](int64_t work) {
    const int64_t want = (work + 255) / 256;
    return (int)(want < 65536 ? (want < 1 ? 1 : want) : 65536);
  };
  if (dt == DType::BF16) {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(grid_for(n_tokens * kv_heads * (int64_t)(D / 8))), dim3(256), 0,
                       stream, (const uint16_t*)k_new, (const uint16_t*)v_new, k_tok, k_head, v_tok, v_head, start_pos,
                       n_tokens, kv_heads, D, DV, block_table, num_blocks, (uint16_t*)k_pool, (uint16_t*)v_pool, false);
    const int64_t runs = (start_pos + n_tokens - 1) / 8 - start_pos / 8 + 1;
    hipLaunchKernelGGL(kv_append_v_bf16_kernel, dim3(grid_for(runs * kv_heads * (DV / 2))), dim3(256), 0, stream,
                       (const uint16_t*)v_new, v_tok, v_head, start_pos, n_tokens, kv_heads, DV, block_table,
                       num_blocks, (uint16_t*)v_pool);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(grid_for(n_tokens * kv_heads * (int64_t)(D + DV))), dim3(256), 0,
                       stream, (const float*)k_new, (const float*)v_new, k_tok, k_head, v_tok, v_head, start_pos,
                       n_tokens, kv_heads, D, DV, block_table, num_blocks, (float*)k_pool, (float*)v_pool, true);
  }
  return hipGetLastError();
}

}  // namespace chunkattn
