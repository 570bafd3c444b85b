// Chunked-prefill causal attention on gfx950 matrix cores.
//
// What it computes: for each query token i of a chunk starting at absolute
// position past_len and each query head h, softmax over keys j <= past_len+i
// of scale * q.k_j, applied to v_j (VPP technical review, English edition,
// §2.2 Eq. (1) and its causal rule; §2.3 for the chunk's offset into a cache
// that already holds every earlier chunk).
//
// How (flash-style, one pass over the keys with an online softmax):
//  * A workgroup is 4 waves.  Each wave owns 32 query rows of one head.  The
//    4 waves share one KV head: either 4 heads of a GQA group on the same 32
//    tokens, 2 heads x 64 tokens, or 1 head x 128 tokens.  One 64-key K/V
//    tile in LDS therefore feeds 128 query rows.
//  * Key tiles are 64 tokens = one paged block.  A tile is brought from HBM
//    into registers one iteration ahead and written into the other half of a
//    double-buffered LDS stage, so one barrier per tile suffices.
//  * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16 (or the
//    fp32 32x32x2 form).  Keeping keys on the accumulator rows puts each
//    query row in a single lane pair (l, l^32): the row max needs one
//    permlane32 swap, the row sum none until the end, and the rescale of O by
//    exp(m_old - m_new) is a per-lane scalar.  The rescale is skipped when no
//    row of the wave raised its maximum.
//  * The accumulator's key rows are permuted (middle quads of every 16 swapped)
//    so that the bf16 P fragment a lane holds is exactly the B operand of the
//    P.V contraction over 8 consecutive keys, read with one 16-byte LDS load.
//  * exp is exp2 with log2(e) folded into the scale; P is rounded to bf16
//    (round to nearest even) for the matrix core, the running sum uses the
//    fp32 values.  The causal mask is applied only on tiles that cross a
//    row's position; tiles past the workgroup's last row are never loaded.
//  * Optional split-KV: the tiles of a workgroup are cut into num_splits
//    contiguous ranges, each writes an unnormalised partial (O, m, l), and a
//    merge kernel combines them with log-sum-exp weights.
#include "device_common.h"
#include "launch.h"

namespace chunkattn {

template <typename E, int D, int DV>
struct PrefillCfg {
  static constexpr bool kBf16 = sizeof(E) == 2;
  static constexpr int X = Elem<E>::X;
  static constexpr int kThreads = 256;
  static constexpr int KBytes = D * kBlock * (int)sizeof(E);
  static constexpr int VBytes = DV * kBlock * (int)sizeof(E);
  static constexpr int Stage = KBytes + VBytes;
  static constexpr int KPT = KBytes / 16 / kThreads;   // 16-byte chunks per thread
  static constexpr int VPT = VBytes / 16 / kThreads;
  static constexpr int NQ = kBf16 ? D / 16 : D / 8;    // 16-byte Q operand chunks per lane
  static constexpr int NB = DV / 32;                   // 32-row output blocks
  static_assert(KBytes % (16 * kThreads) == 0 && VBytes % (16 * kThreads) == 0, "tile split");
};

// Accumulator row m of a 32-key half stands for key kappa(m): for bf16 the
// quads 4..7 and 8..11 of every 16 are swapped (see file comment).
template <bool kBf16>
__device__ __forceinline__ int key_of_row(int m) {
  if constexpr (kBf16) return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
  else return m;
}
// Key offset (within the 64-key tile) of accumulator register r of half kb2.
template <bool kBf16>
__device__ __forceinline__ int key_of_reg(int kb2, int r, int hl) {
  if constexpr (kBf16) return 32 * kb2 + 16 * (r >> 3) + 8 * hl + (r & 7);
  else return 32 * kb2 + 8 * (r >> 2) + 4 * hl + (r & 3);
}

template <typename E, typename EO, int D, int DV, bool kPaged>
__global__ __launch_bounds__(256, sizeof(E) == 2 ? 2 : 1) void prefill_kernel(const PrefillArgs a) {
  using C = PrefillCfg<E, D, DV>;
  constexpr bool kBf16 = C::kBf16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::Stage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int hpw = a.hpw;
  const int tok_wg = 128 / hpw;

  // ---- which (sequence, token block, head group, split) this workgroup owns --
  const E* qbase = (const E*)a.q;
  EO* obase = (EO*)a.out;
  float* lse = a.lse;
  const int32_t* btab = a.block_table;
  int64_t c = a.chunk_len, P = a.past_len, kv_len = a.kv_len;
  int n_tb = a.n_tok_blocks;
  const int S = a.num_splits;
  int split, w;
  split = blockIdx.x % S;
  w = blockIdx.x / S;
  int tb, hg;
  if (a.xcd_remap) {
    // Consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD
    // a fixed slice of head groups (hence of KV heads) so its L2 serves the
    // same K/V to every workgroup it runs, heaviest token blocks first.
    const int xcd = w & 7, slot = w >> 3, hpx = a.n_head_groups >> 3;
    hg = xcd * hpx + slot % hpx;
    tb = n_tb - 1 - slot / hpx;
  } else {
    hg = w % a.n_head_groups;
    tb = n_tb - 1 - w / a.n_head_groups;
  }
  const int h = hg * hpw + (wave % hpw);
  const int g = h / a.group;
  const int64_t t_wg0 = (int64_t)tb * tok_wg;
  const int64_t t0 = t_wg0 + (int64_t)(wave / hpw) * 32;
  const int64_t t_wg_last = min(t_wg0 + tok_wg, c) - 1;
  const int n_tiles = (int)((P + t_wg_last) / kBlock) + 1;
  const int tps = (n_tiles + S - 1) / S;
  const int j_lo = split * tps;
  const int j_hi = min(n_tiles, j_lo + tps);

  const int64_t t = t0 + col;
  const bool row_valid = t < c;
  const int64_t t_c = row_valid ? t : c - 1;       // rows past the chunk mirror its last row
  const int64_t pos = P + t_c;
  const bool wave_active = t0 < c;
  const int wave_last_tile = wave_active ? (int)((P + min(t0 + 31, c - 1)) / kBlock) : -1;
  const int64_t wave_first_pos = P + t0;
  const float cs = a.scale_log2;

  if (j_lo >= j_hi) {   // an empty split: no key for any row
    if (row_valid && hl == 0) {
      const int64_t row = t * a.heads + h;
      *(float2*)(a.ws_ml + ((int64_t)split * c * a.heads + row) * 2) = make_float2(-INFINITY, 0.f);
    }
    return;
  }

  // ---- this lane's query row as B operands (kept for the whole loop) -------
  u32x4_t qreg[C::NQ];
  {
    const E* qrow = qbase + (t_c * a.heads + h) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      const int off = kBf16 ? (16 * i + 8 * hl) : (4 * (2 * i + hl));
      qreg[i] = *(const u32x4_t*)(qrow + off);
    }
  }

  // ---- K/V tile staging ------------------------------------------------------
  u32x4_t kst[C::KPT], vst[C::VPT];
  auto load_tile = [&](int j) {
    const int64_t key0 = (int64_t)j * kBlock;
    if constexpr (kPaged) {
      const int phys = clamp_block(btab[j], a.num_blocks);
      const int64_t tile = (int64_t)phys * a.kv_heads + g;
      const unsigned char* kb = (const unsigned char*)a.k + tile * C::KBytes;
      const unsigned char* vb = (const unsigned char*)a.v + tile * C::VBytes;
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) kst[i] = *(const u32x4_t*)(kb + (tid + C::kThreads * i) * 16);
#pragma unroll
      for (int i = 0; i < C::VPT; ++i) vst[i] = *(const u32x4_t*)(vb + (tid + C::kThreads * i) * 16);
      if (key0 + kBlock > kv_len) {
        // Values of keys past the sequence end are zeroed: a masked key has
        // probability 0, but 0 * NaN would still poison the sum.
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
          const int cidx = tid + C::kThreads * i;
          const int64_t kfirst = key0 + (cidx / DV) * C::X;
#pragma unroll
          for (int e = 0; e < C::X; ++e) {
            if (kfirst + e >= kv_len) {
              if constexpr (kBf16) vst[i][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
              else vst[i][e] = 0u;
            }
          }
        }
      }
    } else {
      const E* kbase = (const E*)a.k;
      const E* vbase = (const E*)a.v;
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        const int cidx = tid + C::kThreads * i;
        const int tok = cidx / (D / C::X), dc = cidx % (D / C::X);
        const int64_t key = key0 + tok;
        kst[i] = key < kv_len
                     ? *(const u32x4_t*)(kbase + key * a.k_stride_tok + g * a.k_stride_head + dc * C::X)
                     : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < C::VPT; ++i) {
        const int cidx = tid + C::kThreads * i;
        const int tok = cidx / (DV / C::X), dvc = cidx % (DV / C::X);
        const int64_t key = key0 + tok;
        vst[i] = key < kv_len
                     ? *(const u32x4_t*)(vbase + key * a.v_stride_tok + g * a.v_stride_head + dvc * C::X)
                     : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* ks = smem + stage * C::Stage;
    unsigned char* vs = ks + C::KBytes;
    if constexpr (kPaged) {
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) *(u32x4_t*)(ks + (tid + C::kThreads * i) * 16) = kst[i];
#pragma unroll
      for (int i = 0; i < C::VPT; ++i) *(u32x4_t*)(vs + (tid + C::kThreads * i) * 16) = vst[i];
    } else {
      // Token-major cache: K chunks go to their interleaved slot, V elements
      // are transposed one by one into the feature-major tile.
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        const int cidx = tid + C::kThreads * i;
        const int tok = cidx / (D / C::X), dc = cidx % (D / C::X);
        *(u32x4_t*)(ks + (dc * kBlock + tok) * 16) = kst[i];
      }
#pragma unroll
      for (int i = 0; i < C::VPT; ++i) {
        const int cidx = tid + C::kThreads * i;
        const int tok = cidx / (DV / C::X), dvc = cidx % (DV / C::X);
        E* vt = (E*)vs + (tok / C::X) * DV * C::X + (tok % C::X);
        const E* src = (const E*)&vst[i];
#pragma unroll
        for (int e = 0; e < C::X; ++e) vt[(dvc * C::X + e) * C::X] = src[e];
      }
    }
  };

  // ---- running state -----------------------------------------------------------
  f32x16_t o[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) o[b] = f32x16_t{};
  float m_run = -INFINITY;   // raw-logit maximum
  float l_run = 0.f;         // this lane's half of the row sum

  auto compute_tile = [&](int j, int stage) {
    const unsigned char* ks = smem + stage * C::Stage;
    const unsigned char* vs = ks + C::KBytes;
    f32x16_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x16_t{};
      const int krow = 32 * kb2 + key_of_row<kBf16>(col);
#pragma unroll
      for (int i = 0; i < C::NQ; ++i) {
        const unsigned char* p = ks + ((2 * i + hl) * kBlock + krow) * 16;
        if constexpr (kBf16) {
          s[kb2] = mfma_bf16(*(const u32x4_t*)p, qreg[i], s[kb2]);
        } else {
          const f32x4_t a4 = *(const f32x4_t*)p;
          const f32x4_t q4 = __builtin_bit_cast(f32x4_t, qreg[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb2] = mfma_f32(a4[e], q4[e], s[kb2]);
        }
      }
    }
    const int64_t key0 = (int64_t)j * kBlock;
    if (key0 + kBlock - 1 > wave_first_pos) {   // tile crosses some row's diagonal
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + key_of_reg<kBf16>(kb2, r, hl) > pos) s[kb2][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
    mx = half_max(mx);
    // The running maximum is raised lazily (see kLazyRescale).
    const bool grow = mx * cs > m_run * cs + kLazyRescale;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2((m_run - m_new) * cs) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
      m_run = m_new;
    }
    const float mb = (m_run == -INFINITY) ? 0.f : m_run * cs;
    float psum = 0.f;
    if constexpr (kBf16) {
      // Same arithmetic, in the same order, as the paged kernel, so both give
      // identical bits.
      uint32_t pk[16];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float p0 = fast_exp2(__builtin_fmaf(s[0][2 * rr], cs, -mb));
        const float p1 = fast_exp2(__builtin_fmaf(s[0][2 * rr + 1], cs, -mb));
        const float p2 = fast_exp2(__builtin_fmaf(s[1][2 * rr], cs, -mb));
        const float p3 = fast_exp2(__builtin_fmaf(s[1][2 * rr + 1], cs, -mb));
        psum += (p0 + p1) + (p2 + p3);
        pk[rr] = pack_bf16(p0, p1);
        pk[8 + rr] = pack_bf16(p2, p3);
      }
      l_run += psum;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int base = (st >> 1) * 8 + 4 * (st & 1);
        const u32x4_t pb = u32x4_t{pk[base], pk[base + 1], pk[base + 2], pk[base + 3]};
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
          const u32x4_t va = *(const u32x4_t*)(vs + ((2 * st + hl) * DV + 32 * b + col) * 16);
          o[b] = mfma_bf16(va, pb, o[b]);
        }
      }
    } else {
      float p[2][16];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb2][r] = fast_exp2(__builtin_fmaf(s[kb2][r], cs, -mb));
          psum += p[kb2][r];
        }
      l_run += psum;
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x4_t va = *(const f32x4_t*)(vs + ((8 * kb2 + 2 * jq + hl) * DV + 32 * b + col) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[b] = mfma_f32(va[e], p[kb2][4 * jq + e], o[b]);
          }
    }
  };

  // ---- main loop: one barrier per tile, next tile in flight ----------------
  load_tile(j_lo);
  store_tile(0);
  __syncthreads();
  for (int j = j_lo; j < j_hi; ++j) {
    const int stage = (j - j_lo) & 1;
    const bool more = j + 1 < j_hi;
    if (more) load_tile(j + 1);
    if (j <= wave_last_tile) compute_tile(j, stage);
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------
  const float l_tot = half_sum(l_run);
  if (!row_valid) return;
  if (S == 1) {
    const float inv = 1.f / l_tot;
    EO* orow = obase + (t * a.heads + h) * (int64_t)DV;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dv0 = 32 * b + 8 * rq + 4 * hl;
        const float v0 = o[b][4 * rq] * inv, v1 = o[b][4 * rq + 1] * inv;
        const float v2 = o[b][4 * rq + 2] * inv, v3 = o[b][4 * rq + 3] * inv;
        if constexpr (sizeof(EO) == 2) {
          *(u32x2_t*)(orow + dv0) = u32x2_t{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        } else {
          *(f32x4_t*)(orow + dv0) = f32x4_t{v0, v1, v2, v3};
        }
      }
    if (lse && hl == 0) lse[(int64_t)h * a.lse_stride + t] = (m_run * cs + __log2f(l_tot)) * kLn2;
  } else {
    const int64_t R = c * a.heads;
    const int64_t row = t * a.heads + h;
    float* wo = a.ws_o + ((int64_t)split * R + row) * DV;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dv0 = 32 * b + 8 * rq + 4 * hl;
        *(f32x4_t*)(wo + dv0) = f32x4_t{o[b][4 * rq], o[b][4 * rq + 1], o[b][4 * rq + 2], o[b][4 * rq + 3]};
      }
    if (hl == 0)
      *(float2*)(a.ws_ml + ((int64_t)split * R + row) * 2) =
          make_float2(m_run == -INFINITY ? -INFINITY : m_run * cs, l_tot);
  }
}

// Merge of prefill split partials: 32 threads per row, 4 features each.
template <typename EO, int DV>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a) {
  const int64_t R = a.chunk_len * a.heads;
  constexpr int TPR = DV / 4;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  if (row >= R) return;
  const int S = a.num_splits;
  float M, L;
  merge_weights(a.ws_ml + row * 2, S, R, M, L);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // four splits' partials are loaded before any is used, so each thread keeps 64 B in flight; a partial
  // with m = -inf (no visible key) is selected away, its O (never written) is not used
  for (int s0 = 0; s0 < S; s0 += 4) {
    float m[4];
    f32x4_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(s0 + i, S - 1);
      m[i] = s0 + i < S ? a.ws_ml[((int64_t)s * R + row) * 2] : -INFINITY;
      v[i] = *(const f32x4_t*)(a.ws_o + ((int64_t)s * R + row) * DV + 4 * q4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wgt = fast_exp2(m[i] - M);
      if (m[i] != -INFINITY) acc += v[i] * wgt;
    }
  }
  const float inv = 1.f / L;
  acc *= inv;
  EO* orow = (EO*)a.out + row * DV + 4 * q4;
  if constexpr (sizeof(EO) == 2) *(u32x2_t*)orow = u32x2_t{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  else *(f32x4_t*)orow = acc;
  if (a.lse && q4 == 0) {
    const int64_t t = row / a.heads;
    const int h = (int)(row % a.heads);
    a.lse[(int64_t)h * a.lse_stride + t] = (M + __log2f(L)) * kLn2;
  }
}

// ---- host launchers --------------------------------------------------------------

template <typename E, typename EO, int D, int DV>
static hipError_t launch_one(bool paged, const PrefillArgs& a, int grid, hipStream_t stream) {
  if (paged)
    hipLaunchKernelGGL((prefill_kernel<E, EO, D, DV, true>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<E, EO, D, DV, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename E, typename EO>
static hipError_t launch_dims(int D, int DV, bool paged, const PrefillArgs& a, int grid, hipStream_t s) {
  if (D == 64 && DV == 64) return launch_one<E, EO, 64, 64>(paged, a, grid, s);
  if (D == 128 && DV == 128) return launch_one<E, EO, 128, 128>(paged, a, grid, s);
  if (D == 192 && DV == 128) return launch_one<E, EO, 192, 128>(paged, a, grid, s);
  return hipErrorInvalidValue;
}

bool prefill_supported(DType in, DType out, int D, int DV) {
  const bool dims = (D == 64 && DV == 64) || (D == 128 && DV == 128) || (D == 192 && DV == 128);
  const bool types = (in == DType::BF16) || (in == DType::F32 && out == DType::F32);
  return dims && types;
}

hipError_t launch_prefill(DType in, DType out, int D, int DV, bool paged, const PrefillArgs& a,
                          int grid, hipStream_t stream) {
  if (in == DType::BF16 && out == DType::BF16) return launch_dims<uint16_t, uint16_t>(D, DV, paged, a, grid, stream);
  if (in == DType::BF16 && out == DType::F32) return launch_dims<uint16_t, float>(D, DV, paged, a, grid, stream);
  if (in == DType::F32 && out == DType::F32) return launch_dims<float, float>(D, DV, paged, a, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_merge(DType out, int DV, const PrefillArgs& a, hipStream_t stream) {
  const int64_t R = a.chunk_len * a.heads;
  const int rows_per_wg = 256 / (DV / 4);
  const int grid = (int)((R + rows_per_wg - 1) / rows_per_wg);
  if (out == DType::BF16) {
    if (DV == 64) hipLaunchKernelGGL((prefill_merge_kernel<uint16_t, 64>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((prefill_merge_kernel<uint16_t, 128>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (DV == 64) hipLaunchKernelGGL((prefill_merge_kernel<float, 64>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((prefill_merge_kernel<float, 128>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace chunkattn
