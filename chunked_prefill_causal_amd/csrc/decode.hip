// Split-KV decode attention for the mixed prefill + decode batch, gfx950.
//
// A decode request contributes one query token (or a few) that must read its
// whole cached prefix; the work is bound by HBM bandwidth, not by the matrix
// cores (VPP technical review, English edition, §2.1; mixed batches: notes on
// "Revisiting Pipeline Parallelism for LLM Serving", preliminaries).
//
// Design:
//  * One wave per (sequence, KV head, key split).  The split's 64-key tiles
//    stream straight from HBM into matrix-core operand registers: with the
//    paged layout, each 32-lane half of the wave reads 512 contiguous bytes
//    per operand load, so no LDS staging is needed and no barrier exists.
//  * All query rows that share the KV head (the GQA group times the request's
//    query tokens, at most 32) ride in the 32 columns of one
//    v_mfma_f32_32x32x16_bf16, so K and V are read once per group.  The
//    matrix cores are mostly idle; they only spare the vector ALUs.
//  * Each wave writes an unnormalised partial (O, m, l) for its key range;
//    a merge kernel combines the partials of a row with log-sum-exp weights
//    in a fixed split order (deterministic).
//  * Partial slots are packed per sequence; a one-workgroup plan kernel
//    computes each sequence's first slot (and each prefill-path sequence's
//    first workgroup) from the device copies of the sequence lengths, so the
//    host never uploads a plan.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace chunkattn {

__device__ __forceinline__ int dec_key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ int dec_key_of_reg(int kb2, int r, int hl) { return 32 * kb2 + 16 * (r >> 3) + 8 * hl + (r & 7); }

__device__ __forceinline__ bool is_decode_seq(int q_len, int group) { return q_len >= 1 && q_len * group <= 32; }

// ---- plan: per-sequence offsets, computed from the device copies of the lengths ----
// ws_off[s]: first decode partial slot of sequence s (decode path);
// wg_off[s]: first prefill workgroup of sequence s (prefill path), with
// wg_off[num_seqs] = the total.  One workgroup scans both counts.
__device__ __forceinline__ void plan_counts(const DecodeArgs& a, int s, int64_t& dec, int64_t& pre) {
  const int q_len = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
  dec = pre = 0;
  if (is_decode_seq(q_len, a.group)) {
    const int nsplit = (a.kv_lens[s] + a.split_tokens - 1) / a.split_tokens;
    dec = (int64_t)q_len * a.heads * nsplit;
  } else if (q_len > 0) {
    pre = (int64_t)((q_len + a.tok_wg - 1) / a.tok_wg) * a.n_head_groups;
  }
}

__global__ __launch_bounds__(1024) void plan_kernel(const DecodeArgs a) {
  __shared__ int64_t part_dec[1024];
  __shared__ int64_t part_pre[1024];
  const int tid = threadIdx.x;
  const int per = (a.num_seqs + 1023) / 1024;
  const int s0 = tid * per, s1 = min(a.num_seqs, s0 + per);
  int64_t ld = 0, lp = 0;
  for (int s = s0; s < s1; ++s) {
    int64_t d, p;
    plan_counts(a, s, d, p);
    ld += d;
    lp += p;
  }
  part_dec[tid] = ld;
  part_pre[tid] = lp;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // inclusive scans
    const int64_t vd = tid >= off ? part_dec[tid - off] : 0;
    const int64_t vp = tid >= off ? part_pre[tid - off] : 0;
    __syncthreads();
    part_dec[tid] += vd;
    part_pre[tid] += vp;
    __syncthreads();
  }
  int64_t rd = part_dec[tid] - ld, rp = part_pre[tid] - lp;   // exclusive prefixes
  for (int s = s0; s < s1; ++s) {
    a.ws_off[s] = rd;
    a.wg_off[s] = rp;
    int64_t d, p;
    plan_counts(a, s, d, p);
    rd += d;
    rp += p;
  }
  if (tid == 1023) a.wg_off[a.num_seqs] = part_pre[1023];
}

// ---- partial attention of one key split -------------------------------------------
template <int D, int DV>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
  constexpr int NQ = D / 16, NB = DV / 32;
  const int sp = blockIdx.x, g = blockIdx.y, s = a.seq_begin + (int)blockIdx.z;
  const int lane = threadIdx.x, hl = lane >> 5, col = lane & 31;
  if (s >= a.num_seqs) return;
  const int q0 = a.cu_seqlens_q[s];
  const int q_len = a.cu_seqlens_q[s + 1] - q0;
  const int G = a.group;
  if (!is_decode_seq(q_len, G)) return;
  const int kvl = a.kv_lens[s];
  if (kvl < q_len || kvl > a.max_blocks * kBlock) return;   // inconsistent lengths never reach memory
  const int nsplit = (kvl + a.split_tokens - 1) / a.split_tokens;
  if (sp >= nsplit) return;
  const int key_lo = sp * a.split_tokens;
  const int key_hi = min(kvl, key_lo + a.split_tokens);

  const bool col_valid = col < q_len * G;
  const int i = col_valid ? col / G : 0;
  const int h = g * G + (col_valid ? col % G : 0);
  const int pos = kvl - q_len + i;             // causal limit of this row
  const int first_pos = kvl - q_len;           // smallest row position in the wave
  const float cs = a.scale_log2;

  u32x4_t qreg[NQ];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)(q0 + i) * a.heads + h) * D;
#pragma unroll
    for (int k = 0; k < NQ; ++k)
      qreg[k] = col_valid ? *(const u32x4_t*)(qrow + 16 * k + 8 * hl) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;

  f32x16_t o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // K and V of a tile each have one register set.  K of tile j+1 is requested as
  // soon as QK of tile j has consumed K, V of tile j+1 as soon as PV of tile j
  // has consumed V, so a tile's worth of loads is in flight while the wave
  // computes (one wave per SIMD fits these registers).
  u32x4_t ka[2][NQ];
  u32x4_t va[4][NB];
  auto load_k = [&](int j) {
    const int64_t tile = (int64_t)clamp_block(bt[j], a.num_blocks) * a.kv_heads + g;
    const uint16_t* kt = (const uint16_t*)a.k + tile * (D * kBlock);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int krow = 32 * kb2 + dec_key_of_row(col);
#pragma unroll
      for (int k = 0; k < NQ; ++k) ka[kb2][k] = *(const u32x4_t*)(kt + ((2 * k + hl) * kBlock + krow) * 8);
    }
  };
  auto load_v = [&](int j) {
    const int64_t tile = (int64_t)clamp_block(bt[j], a.num_blocks) * a.kv_heads + g;
    const uint16_t* vt = (const uint16_t*)a.v + tile * (DV * kBlock);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int b = 0; b < NB; ++b) va[st][b] = *(const u32x4_t*)(vt + ((2 * st + hl) * DV + 32 * b + col) * 8);
  };
  const int j_first = key_lo / kBlock, j_end = (key_hi + kBlock - 1) / kBlock;
  load_k(j_first);
  load_v(j_first);
  for (int j = j_first; j < j_end; ++j) {
    f32x16_t sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sc[kb2] = f32x16_t{};
#pragma unroll
      for (int k = 0; k < NQ; ++k) sc[kb2] = mfma_bf16(ka[kb2][k], qreg[k], sc[kb2]);
    }
    if (j + 1 < j_end) load_k(j + 1);
    const int key0 = j * kBlock;
    if (key0 + kBlock - 1 > first_pos) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + dec_key_of_reg(kb2, r, hl) > pos) sc[kb2][r] = -INFINITY;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb2][r]);
    mx = half_max(mx);
    const bool grow = mx * cs > m_run * cs + kLazyRescale;   // lazy maximum (see kLazyRescale)
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2((m_run - m_new) * cs) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
      m_run = m_new;
    }
    const float mb = (m_run == -INFINITY) ? 0.f : m_run * cs;
    uint32_t pk[16];
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float p0 = fast_exp2(__builtin_fmaf(sc[kb2][2 * rr], cs, -mb));
        const float p1 = fast_exp2(__builtin_fmaf(sc[kb2][2 * rr + 1], cs, -mb));
        psum += p0 + p1;
        pk[kb2 * 8 + rr] = pack_bf16(p0, p1);
      }
    l_run += psum;
    if (key0 + kBlock > kvl) {   // values past the sequence end are zeroed (0 * NaN guard)
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + 16 * st + 8 * hl + e >= kvl)
#pragma unroll
            for (int b = 0; b < NB; ++b) va[st][b][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int base = (st >> 1) * 8 + 4 * (st & 1);
      const u32x4_t pb = u32x4_t{pk[base], pk[base + 1], pk[base + 2], pk[base + 3]};
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = mfma_bf16(va[st][b], pb, o[b]);
    }
    if (j + 1 < j_end) load_v(j + 1);
  }

  const float l_tot = half_sum(l_run);
  if (!col_valid) return;
  const int64_t slot = a.ws_off[s] + ((int64_t)(i * a.heads + h) * nsplit + sp);
  if (slot < 0 || slot >= a.total_slots) return;   // host and device lengths disagree: drop, never overrun
  float* wo = a.ws_o + slot * DV;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *(f32x4_t*)(wo + 32 * b + 8 * rq + 4 * hl) =
          f32x4_t{o[b][4 * rq], o[b][4 * rq + 1], o[b][4 * rq + 2], o[b][4 * rq + 3]};
  if (hl == 0) *(float2*)(a.ws_ml + slot * 2) = make_float2(m_run == -INFINITY ? -INFINITY : m_run * cs, l_tot);
}

// ---- merge: workgroup (sequence, block of 256 / (DV/4) rows), DV/4 threads per row ----
// A long context has hundreds of splits per row; spreading rows over workgroups
// and loading four splits at a time keeps the merge from becoming a serial
// chain of loads when the batch has few sequences.
template <int DV>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs a) {
  const int s = blockIdx.x;
  const int q0 = a.cu_seqlens_q[s];
  const int q_len = a.cu_seqlens_q[s + 1] - q0;
  if (!is_decode_seq(q_len, a.group)) return;
  const int nsplit = (a.kv_lens[s] + a.split_tokens - 1) / a.split_tokens;
  constexpr int TPR = DV / 4, RPW = 256 / TPR;
  const int rows = q_len * a.heads;
  const int q4 = threadIdx.x % TPR;
  for (int row = blockIdx.y * RPW + threadIdx.x / TPR; row < rows; row += gridDim.y * RPW) {
    const int i = row / a.heads, h = row % a.heads;
    const int64_t slot0 = a.ws_off[s] + (int64_t)row * nsplit;
    if (slot0 < 0 || slot0 + nsplit > a.total_slots) continue;
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      float m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) m[j] = s0 + j < nsplit ? a.ws_ml[(slot0 + s0 + j) * 2] : -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) M = fmaxf(M, m[j]);
    }
    float L = 0.f;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      float m[4], l[4];
      f32x4_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t sl = slot0 + min(s0 + j, nsplit - 1);
        m[j] = s0 + j < nsplit ? a.ws_ml[sl * 2] : -INFINITY;
        l[j] = a.ws_ml[sl * 2 + 1];
        v[j] = *(const f32x4_t*)(a.ws_o + sl * DV + 4 * q4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (m[j] == -INFINITY) continue;             // no visible key: no weight, O never written
        const float wgt = fast_exp2(m[j] - M);
        L += l[j] * wgt;
        acc += v[j] * wgt;
      }
    }
    acc *= 1.f / L;
    const int64_t o_off = ((int64_t)(q0 + i) * a.heads + h) * DV + 4 * q4;
    if (a.out_f32) *(f32x4_t*)((float*)a.out + o_off) = acc;
    else *(u32x2_t*)((uint16_t*)a.out + o_off) = u32x2_t{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    if (a.lse && q4 == 0) a.lse[(int64_t)h * a.total_q + q0 + i] = (M + __log2f(L)) * kLn2;
  }
}

// ---- host launchers -------------------------------------------------------------------

bool decode_supported(int D, int DV) {
  return (D == 64 && DV == 64) || (D == 128 && DV == 128) || (D == 192 && DV == 128);
}

hipError_t launch_batch_plan(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(int D, int DV, const DecodeArgs& args, int max_splits, int seq_begin, int seq_end,
                         hipStream_t stream) {
  if (seq_end <= seq_begin) return hipSuccess;
  DecodeArgs a = args;
  a.seq_begin = seq_begin;
  const dim3 grid(max_splits, a.kv_heads, seq_end - seq_begin);
  if (D == 64 && DV == 64) hipLaunchKernelGGL((decode_kernel<64, 64>), grid, dim3(64), 0, stream, a);
  else if (D == 128 && DV == 128) hipLaunchKernelGGL((decode_kernel<128, 128>), grid, dim3(64), 0, stream, a);
  else if (D == 192 && DV == 128) hipLaunchKernelGGL((decode_kernel<192, 128>), grid, dim3(64), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(int DV, const DecodeArgs& a, hipStream_t stream) {
  // a decode-path sequence has q_len * group <= 32, so at most 32 * kv_heads rows; larger counts loop
  const int max_rows = 32 * a.kv_heads;
  const int rpw = DV == 64 ? 16 : 8;
  const dim3 grid(a.num_seqs, std::min((max_rows + rpw - 1) / rpw, 4096));
  if (DV == 64) hipLaunchKernelGGL((decode_merge_kernel<64>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((decode_merge_kernel<128>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace chunkattn
