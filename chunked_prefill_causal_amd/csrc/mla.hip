// MLA latent (absorbed) decode over a paged latent cache, gfx950.
//
// "02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16" deployment notes §1, §4:
// an MLA layer caches one latent record per token, shared by every query head
// (replicated, not split, across tensor-parallel ranks), of 1152 B in bf16 or
// 656 B in the fp8 latent format.  Read here as 512 latent + 64 rotary values;
// in fp8 the latent is 512 OCP e4m3 codes with one fp32 scale per 128 values
// and the rotary part stays bf16 (512 + 16 + 128 = 656 B).  Decode of a query
// head q (576 values) is attention with keys = records and values = their
// 512-value latents; the output stays in latent space.
//
// Kernel shape (one wave per (sequence, 16-head block, key split)):
//  * 32 keys per step, double-buffered in LDS by direct-to-LDS loads.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: two 16-key row blocks x 18
//    feature steps; a lane holds keys 4g..4g+3 and 16+4g..16+4g+3 (g = lane/16)
//    of head lane%16 — exactly the B operand P^T of the PV product over those
//    8 keys, so P needs no shuffle.
//  * O^T = V^T P^T on the same MFMA, 32 blocks of 16 latent values.  The V^T
//    operand (8 keys of one feature per lane) comes from the token-major tile
//    through transposing LDS reads: two ds_read_b64_tr_b16 (bf16) or one
//    ds_read_b64_tr_b8 (fp8 codes).
//  * fp8: codes are widened exactly (unit scale) by v_cvt_scalef32_pk_bf16_fp8,
//    one instruction per pair.  Scores are accumulated per 128-value group and
//    each key's fp32 group scale is applied to its partial score; for PV each
//    key's scale is folded into P, group by group.
//  * Unnormalised partials (O, max, sum) per split; mla_merge_kernel combines
//    them in split order.
#include "device_common.h"
#include "launch.h"

namespace chunkattn {

namespace {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) v2i32_t lds_v2i32;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_wave_base), "v"(g) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Eight e4m3 codes (two dwords) to eight bf16 values times `scale`.
__device__ __forceinline__ u32x4_t widen8(uint32_t lo, uint32_t hi, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true));
  return r;
}

template <bool FP8>
struct MlaCfg {
  // LDS bytes of one 32-key step: bf16 [72 runs][32][16 B]; fp8 codes [32 runs][32][16 B],
  // scales [32][16 B] (+512 B the second half-wave of the scale load writes), rotary [8 runs][32][16 B].
  static constexpr int kCodes = 0;
  static constexpr int kScales = 32 * 32 * 16;
  static constexpr int kRope = FP8 ? kScales + 1024 : 64 * 32 * 16;
  static constexpr int kStage = FP8 ? kRope + 8 * 32 * 16 : 72 * 32 * 16;
  static constexpr int kLoads = FP8 ? 16 + 1 + 4 : 36;     // direct loads per step
  static constexpr int64_t kBlock = FP8 ? kMlaFp8Block : kMlaBf16Block;
  static constexpr int64_t kBlkScales = 32 * 64 * 16;       // fp8 block: scales, then rotary
  static constexpr int64_t kBlkRope = FP8 ? kBlkScales + 64 * 16 : 64 * 64 * 16;
};

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(64) void mla_decode_kernel(const MlaArgs a) {
  using C = MlaCfg<FP8>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::kStage];
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int split = blockIdx.x, hb = blockIdx.y, s = blockIdx.z;
  const int kv_len = a.kv_lens[s];
  const int key_lo = split * a.split_tokens;
  if (kv_len <= 0 || key_lo >= kv_len) return;
  const int key_hi = min(kv_len, key_lo + a.split_tokens);
  const int n_steps = (key_hi - key_lo + kMlaStepKeys - 1) / kMlaStepKeys;
  const int head = hb * 16 + c;
  const float cs = a.scale_log2;

  // Q^T as B operands: 18 feature steps of 8 values (features 32i + 8g ..).
  u32x4_t qb[18];
  {
    const uint16_t* qrow = a.q + ((int64_t)s * a.heads + head) * kMlaRecord;
#pragma unroll
    for (int i = 0; i < 18; ++i) qb[i] = *(const u32x4_t*)(qrow + 32 * i + 8 * g);
  }

  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const uint32_t smem_base = lds_addr(smem);
  // step t covers keys key_lo + 32t .. +31: half (key / 32) & 1 of block key / 64
  auto issue = [&](int t, int st) {
    const int key0 = key_lo + kMlaStepKeys * t;
    const int blk = clamp_block(bt[key0 >> 6], a.num_blocks);
    const unsigned char* b = a.pool + (int64_t)blk * C::kBlock + ((key0 >> 5) & 1) * 32 * 16;
    const uint32_t lds = smem_base + st * C::kStage;
    const int run = lane >> 5, tok = lane & 31;
    if constexpr (FP8) {
#pragma unroll
      for (int n = 0; n < 16; ++n) dma16(b + (2 * n + run) * 1024 + tok * 16, lds + C::kCodes + n * 1024);
      dma16(b + C::kBlkScales + tok * 16, lds + C::kScales);
#pragma unroll
      for (int n = 0; n < 4; ++n) dma16(b + C::kBlkRope + (2 * n + run) * 1024 + tok * 16, lds + C::kRope + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < 36; ++n) dma16(b + (2 * n + run) * 1024 + tok * 16, lds + n * 1024);
    }
  };

  f32x4_t o[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  issue(0, 0);
  for (int t = 0; t < n_steps; ++t) {
    const int st = t & 1;
    if (t + 1 < n_steps) {
      issue(t + 1, st ^ 1);
      wait_vmem<C::kLoads>();
    } else {
      wait_vmem<0>();
    }
    unsigned char* stage = smem + st * C::kStage;
    const int key0 = key_lo + kMlaStepKeys * t;
    const int valid = key_hi - key0;                 // keys of this step that count (1..32)
    if (valid < kMlaStepKeys) {
      // Keys past the split's end (past the sequence) may hold anything: give
      // them zero values (and unit scales) so 0 * junk cannot reach O.
      if constexpr (FP8) {
        for (int e = lane; e < 32 * 32; e += 64) {
          const int run = e >> 5, tok = e & 31;
          if (tok >= valid) *(u32x4_t*)(stage + C::kCodes + run * 512 + tok * 16) = u32x4_t{0u, 0u, 0u, 0u};
        }
        if (lane < 32 && lane >= valid)
          *(f32x4_t*)(stage + C::kScales + lane * 16) = f32x4_t{1.f, 1.f, 1.f, 1.f};
      } else {
        for (int e = lane; e < 64 * 32; e += 64) {
          const int run = e >> 5, tok = e & 31;
          if (tok >= valid) *(u32x4_t*)(stage + run * 512 + tok * 16) = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }

    // ---- S^T = K Q^T: row blocks of keys 0-15 and 16-31 ----
    // A lane's S^T rows are keys 4g+r (s0) and 16+4g+r (s1), r = 0..3: kappa(g, j) below.
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    float vs[8][4];                                  // fp8: scale of key kappa(g, j), 128-value group q
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
        const f32x4_t sc = *(const f32x4_t*)(stage + C::kScales + key * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) vs[j][q] = sc[q];
      }
      // rotary part (bf16), then each latent group's codes widened exactly (scale 1)
      // with the group's partial scores scaled per key in fp32
#pragma unroll
      for (int i = 16; i < 18; ++i) {
        const int off = C::kRope + (4 * (i - 16) + g) * 512;
        s0 = mfma16(*(const u32x4_t*)(stage + off + c * 16), qb[i], s0);
        s1 = mfma16(*(const u32x4_t*)(stage + off + (16 + c) * 16), qb[i], s1);
      }
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        f32x4_t t0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, t1 = t0;
#pragma unroll
        for (int i = 4 * gr; i < 4 * gr + 4; ++i) {
          const int off = C::kCodes + (2 * i + (g >> 1)) * 512 + (g & 1) * 8;
          const u32x2_t c0 = *(const u32x2_t*)(stage + off + c * 16);
          const u32x2_t c1 = *(const u32x2_t*)(stage + off + (16 + c) * 16);
          t0 = mfma16(widen8(c0[0], c0[1], 1.0f), qb[i], t0);
          t1 = mfma16(widen8(c1[0], c1[1], 1.0f), qb[i], t1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s0[r] = __builtin_fmaf(t0[r], vs[r][gr], s0[r]);
          s1[r] = __builtin_fmaf(t1[r], vs[4 + r][gr], s1[r]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const int off = (4 * i + g) * 512;
        s0 = mfma16(*(const u32x4_t*)(stage + off + c * 16), qb[i], s0);
        s1 = mfma16(*(const u32x4_t*)(stage + off + (16 + c) * 16), qb[i], s1);
      }
    }

    // ---- online softmax over this step's keys (head c; keys 4g+r and 16+4g+r) ----
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * g + r >= valid) s0[r] = -INFINITY;
      if (16 + 4 * g + r >= valid) s1[r] = -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool grow = mx * cs > m_run * cs + kLazyRescale;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2((m_run - m_new) * cs) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < 32; ++b) o[b] *= alpha;
      m_run = m_new;
    }
    const float mb = m_run == -INFINITY ? 0.f : m_run * cs;
    float p[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(__builtin_fmaf(s0[r], cs, -mb));
      p[4 + r] = fast_exp2(__builtin_fmaf(s1[r], cs, -mb));
    }
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));

    // ---- O^T += V^T P^T over the 8 keys this lane's P covers ----
    if constexpr (FP8) {
      // each key's scale for 128-value group gr is folded into P
      // transposing read: this lane (as a source) points at key kappa(g, c/2), features 8(c%2)..
      const int src_r = c >> 1;
      const int src_key = src_r < 4 ? 4 * g + src_r : 16 + 4 * g + (src_r - 4);
      const int tr_off = C::kCodes + src_key * 16 + (c & 1) * 8;
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        u32x4_t pb;
#pragma unroll
        for (int q = 0; q < 4; ++q) pb[q] = pack_bf16(p[2 * q] * vs[2 * q][gr], p[2 * q + 1] * vs[2 * q + 1][gr]);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          const int b = 8 * gr + bb;                  // latent values 16b .. 16b+15 live in code run b
          const v2i32_t codes = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(stage + tr_off + b * 512));
          const u32x4_t va = widen8((uint32_t)codes[0], (uint32_t)codes[1], 1.0f);
          o[b] = mfma16(va, pb, o[b]);
        }
      }
    } else {
      u32x4_t pb;
#pragma unroll
      for (int q = 0; q < 4; ++q) pb[q] = pack_bf16(p[2 * q], p[2 * q + 1]);
      // two transposing reads: keys 4g + (c/4) and 16 + 4g + (c/4); features 4(c%4)..
      const int tr0 = (4 * g + (c >> 2)) * 16 + (c & 1) * 8 + ((c & 3) >> 1) * 512;
      const int tr1 = tr0 + 16 * 16;
#pragma unroll
      for (int b = 0; b < 32; ++b) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(stage + tr0 + 2 * b * 512));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(stage + tr1 + 2 * b * 512));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        o[b] = mfma16(u32x4_t{l2[0], l2[1], h2[0], h2[1]}, pb, o[b]);
      }
    }
  }

  // ---- partial of this split ----
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t slot = ((int64_t)s * a.heads + head) * a.max_splits + split;
  float* wo = a.ws_o + slot * kMlaLatent;
#pragma unroll
  for (int b = 0; b < 32; ++b) *(f32x4_t*)(wo + 16 * b + 4 * g) = o[b];
  if (g == 0) *(float2*)(a.ws_ml + slot * 2) = make_float2(m_run == -INFINITY ? -INFINITY : m_run * cs, l_tot);
}

// One workgroup per (sequence, head): combine the splits in order, normalise, store bf16 and the LSE.
__global__ __launch_bounds__(128) void mla_merge_kernel(const MlaArgs a) {
  const int s = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
  const int kv_len = a.kv_lens[s];
  const int nsplit = min(a.max_splits, (kv_len + a.split_tokens - 1) / a.split_tokens);
  const int64_t slot0 = ((int64_t)s * a.heads + h) * a.max_splits;
  float M, L;
  merge_weights(a.ws_ml + slot0 * 2, nsplit, 1, M, L);
  const int t = threadIdx.x;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nsplit; ++sp) {
    const float m = a.ws_ml[(slot0 + sp) * 2];
    if (m == -INFINITY) continue;
    acc += *(const f32x4_t*)(a.ws_o + (slot0 + sp) * kMlaLatent + 4 * t) * fast_exp2(m - M);
  }
  acc *= 1.f / L;
  uint16_t* orow = a.out + ((int64_t)s * a.heads + h) * kMlaLatent + 4 * t;
  *(u32x2_t*)orow = u32x2_t{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  if (a.lse && t == 0) a.lse[(int64_t)h * a.num_seqs + s] = (M + __log2f(L)) * kLn2;
}

// One wave per token: writes its record into the block's runs; fp8 quantises
// each 128-value group of the latent with scale amax / 448.
template <bool FP8>
__global__ __launch_bounds__(64) void mla_append_kernel(const MlaAppendArgs a) {
  const int64_t i = blockIdx.x;
  if (i >= a.n_tokens) return;
  const int lane = threadIdx.x;
  const int64_t pos = a.start_pos + i;
  const int blk = clamp_block(a.block_table[pos >> 6], a.num_blocks);
  const int tok = (int)(pos & 63);
  const int64_t block_bytes = FP8 ? kMlaFp8Block : kMlaBf16Block;
  unsigned char* b = a.pool + (int64_t)blk * block_bytes;
  const u32x4_t lat = *(const u32x4_t*)(a.latent + i * kMlaLatent + 8 * lane);   // latent 8l .. 8l+7
  if constexpr (!FP8) {
    *(u32x4_t*)(b + lane * 1024 + tok * 16) = lat;
    if (lane < 8) *(u32x4_t*)(b + (64 + lane) * 1024 + tok * 16) = *(const u32x4_t*)(a.rope + i * kMlaRope + 8 * lane);
  } else {
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(lat[q] << 16);
      v[2 * q + 1] = __uint_as_float(lat[q] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));   // the 16 lanes of a group
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = fminf(fmaxf(v[4 * q + e] / scale, -448.0f), 448.0f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pk, true);
      w[q] = (uint32_t)pk;
    }
    *(u32x2_t*)(b + (lane >> 1) * 1024 + tok * 16 + (lane & 1) * 8) = u32x2_t{w[0], w[1]};
    if ((lane & 15) == 0) *(float*)(b + 32 * 64 * 16 + tok * 16 + (lane >> 4) * 4) = scale;
    if (lane < 8)
      *(u32x4_t*)(b + 32 * 64 * 16 + 64 * 16 + lane * 1024 + tok * 16) =
          *(const u32x4_t*)(a.rope + i * kMlaRope + 8 * lane);
  }
}

hipError_t launch_mla_decode(bool fp8, const MlaArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.heads / 16, a.num_seqs);
  if (fp8) hipLaunchKernelGGL(mla_decode_kernel<true>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(mla_decode_kernel<false>, grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(a.num_seqs * a.heads), dim3(128), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mla_append(bool fp8, const MlaAppendArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 0) return hipSuccess;
  if (fp8) hipLaunchKernelGGL(mla_append_kernel<true>, dim3(a.n_tokens), dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(mla_append_kernel<false>, dim3(a.n_tokens), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace chunkattn
