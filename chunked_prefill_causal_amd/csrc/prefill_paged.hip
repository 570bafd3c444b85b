// Chunked-prefill causal attention over the paged bf16 KV pool, gfx950.
//
// Same result as prefill_kernel (VPP technical review, English edition, §2.2
// Eq. (1) with its causal rule, §2.3 for the chunk offset); this is the
// kernel the paged bf16 path runs, built around the costs measured on MI355X:
//  * A workgroup is 8 waves x 32 query rows = 256 rows sharing one KV head
//    (the whole GQA group of 8 heads over 32 tokens, 4 heads x 64 tokens,
//    2 x 128 or 1 x 256), so each 64-key K/V tile crosses the L2 once per 256
//    rows instead of once per 128.
//  * Tiles move HBM/L2 -> LDS by direct-to-LDS loads (global_load_lds_dwordx4):
//    no staging registers, no LDS write instructions.  Four LDS stages (three
//    at d = 192) give each load two tile-times to land; one barrier per tile.
//    Only the four leading waves issue them, one load after every fourth MFMA
//    of their matrix phase.  Measured on MI355X, the direct-to-LDS path drains
//    ~40 B/clk per CU, so a tile issued as a burst holds the issuing wave at
//    issue for several hundred cycles; that delayed the leading waves' matrix
//    phase into the trailing waves' and the trailing waves, younger, lost the
//    matrix cores to them.  Spread out, the loads never stall issue.  The
//    first interval of a workgroup, which has no matrix phase before its
//    barrier, still issues its tile as a burst.  The vector-memory
//    counter is managed by hand: inside the key loop the only vector-memory
//    operations are these loads (block-table entries come through the scalar
//    unit, one tile ahead), so "s_waitcnt vmcnt(N)" with N = loads of the
//    newer tile is exact (the trailing waves have none outstanding and pass).
//  * The per-wave matrix work is the same as prefill_kernel's: S^T = K Q^T
//    and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, one query row per lane
//    pair, rescale skipped when no row's maximum grew.  The two waves that
//    share a SIMD run the same tiles half an interval apart (ping-pong), so
//    one feeds the matrix cores while the other computes its softmax.
//  * Values of keys past the sequence end are zeroed in LDS once the tile
//    holding the sequence end has landed, logits past a row's position are
//    masked with a select, so NaN in unused pool slots never reaches an output.
#include "device_common.h"
#include "launch.h"

namespace chunkattn {

template <int D, int DV>
struct PagedCfg {
  static constexpr int kThreads = 512;
  static constexpr int kStages = (D + DV) * kBlock * 2 * 4 <= 131072 ? 4 : 3;   // LDS stages (160 KB per CU)
  static constexpr int KBytes = D * kBlock * 2;
  static constexpr int VBytes = DV * kBlock * 2;
  static constexpr int Stage = KBytes + VBytes;
  static constexpr int kLoaders = 256;                 // the four leading waves move the tiles
  static constexpr int KPT = KBytes / 16 / kLoaders;   // direct loads per loading thread per tile
  static constexpr int VPT = VBytes / 16 / kLoaders;
  static constexpr int LPT = KPT + VPT;
  static constexpr int NQ = D / 16;
  static constexpr int NB = DV / 32;
  static_assert(KBytes % (16 * kLoaders) == 0 && VBytes % (16 * kLoaders) == 0, "tile split");
};

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
__device__ __forceinline__ void load_to_lds16(const void* g, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_wave_base), "v"(g) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename EO, int D, int DV, bool kVarlen>
__global__ __launch_bounds__(512, 1) void prefill_paged_kernel(const PrefillArgs a) {
  using C = PagedCfg<D, DV>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kStages * C::Stage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int hpw = a.hpw;                 // heads per workgroup: 8, 4, 2 or 1
  const int tok_wg = 256 / hpw;

  // ---- which (sequence, token block, head group, split) this workgroup owns --
  const uint16_t* qbase = (const uint16_t*)a.q;
  EO* obase = (EO*)a.out;
  float* lse = a.lse;
  const int32_t* btab = a.block_table;
  int64_t c = a.chunk_len, P = a.past_len, kv_len = a.kv_len;
  int n_tb = a.n_tok_blocks;
  const int S = a.num_splits;
  int split, w;
  if constexpr (kVarlen) {
    const int64_t bid = blockIdx.x;
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.wg_off[mid] <= bid) lo = mid;
      else hi = mid;
    }
    const int q0 = a.cu_seqlens_q[lo];
    c = a.cu_seqlens_q[lo + 1] - q0;
    kv_len = a.kv_lens[lo];
    P = kv_len - c;
    n_tb = (int)((c + tok_wg - 1) / tok_wg);
    qbase += (int64_t)q0 * a.heads * D;
    obase += (int64_t)q0 * a.heads * DV;
    if (lse) lse += q0;
    btab += (int64_t)lo * a.max_blocks;
    split = 0;
    w = (int)(bid - a.wg_off[lo]);
    if (c <= 0 || P < 0 || kv_len > (int64_t)a.max_blocks * kBlock || w >= n_tb * a.n_head_groups) return;
  } else {
    split = blockIdx.x % S;
    w = blockIdx.x / S;
  }
  int tb, hg;
  if (a.xcd_remap) {
    const int xcd = w & 7, slot = w >> 3, hpx = a.n_head_groups >> 3;
    hg = xcd * hpx + slot % hpx;
    tb = n_tb - 1 - slot / hpx;
  } else {
    hg = w % a.n_head_groups;
    tb = n_tb - 1 - w / a.n_head_groups;
  }
  const int h = hg * hpw + (wave % hpw);
  const int g = (hg * hpw) / a.group;
  const int64_t t_wg0 = (int64_t)tb * tok_wg;
  const int64_t t0 = t_wg0 + (int64_t)(wave / hpw) * 32;
  const int64_t t_wg_last = min(t_wg0 + tok_wg, c) - 1;
  const int n_tiles = (int)((P + t_wg_last) / kBlock) + 1;
  const int tps = (n_tiles + S - 1) / S;
  const int j_lo = split * tps;
  const int j_hi = min(n_tiles, j_lo + tps);

  const int64_t t = t0 + col;
  const bool row_valid = t < c;
  const int64_t t_c = row_valid ? t : c - 1;
  const int64_t pos = P + t_c;
  const int64_t wave_first_pos = P + min(t0, c - 1);
  const float cs = a.scale_log2;

  if (j_lo >= j_hi) {
    if (row_valid && hl == 0) {
      const int64_t row = t * a.heads + h;
      *(float2*)(a.ws_ml + ((int64_t)split * c * a.heads + row) * 2) = make_float2(-INFINITY, 0.f);
    }
    return;
  }

  // Query row of this lane as B operands, held for the whole key loop.
  u32x4_t qreg[C::NQ];
  {
    const uint16_t* qrow = qbase + (t_c * a.heads + h) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) qreg[i] = *(const u32x4_t*)(qrow + 16 * i + 8 * hl);
  }

  // ---- tile transfer: block table through the scalar unit, data straight into LDS ----
  const __attribute__((address_space(4))) int32_t* bt4 = (const __attribute__((address_space(4))) int32_t*)btab;
  const unsigned char* kpool = (const unsigned char*)a.k;
  const unsigned char* vpool = (const unsigned char*)a.v;
  const uint32_t smem_base = lds_address(smem);
  auto issue = [&](int32_t block_id, int st) {
    if (wave >= 4) return;
    const int phys = clamp_block(block_id, a.num_blocks);
    const int64_t tile = (int64_t)phys * a.kv_heads + g;
    const unsigned char* kb = kpool + tile * C::KBytes;
    const unsigned char* vb = vpool + tile * C::VBytes;
    const uint32_t ks = smem_base + st * C::Stage;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int chunk = wave * 64 + i * C::kLoaders;
      load_to_lds16(kb + (chunk + lane) * 16, __builtin_amdgcn_readfirstlane(ks + chunk * 16));
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int chunk = wave * 64 + i * C::kLoaders;
      load_to_lds16(vb + (chunk + lane) * 16, __builtin_amdgcn_readfirstlane(ks + C::KBytes + chunk * 16));
    }
  };
  // The same transfer spread over the leading waves' matrix phase: prep() fixes
  // the tile and stage, dma_one(j) moves this thread's j-th 16-byte chunk
  // (K chunks first, then V).  Issued in a burst, the loads would hold the wave
  // for as long as the direct-to-LDS path needs to drain a tile; one load per
  // four MFMAs stays under that rate, so the wave never waits at issue.
  const unsigned char* pend_k = kpool;
  const unsigned char* pend_v = vpool;
  uint32_t pend_lds = 0;
  auto prep = [&](int32_t block_id, int st) {
    const int phys = clamp_block(block_id, a.num_blocks);
    const int64_t tile = (int64_t)phys * a.kv_heads + g;
    pend_k = kpool + tile * C::KBytes + (wave * 64 + lane) * 16;
    pend_v = vpool + tile * C::VBytes + (wave * 64 + lane) * 16;
    pend_lds = smem_base + st * C::Stage + wave * 64 * 16;
  };
  auto dma_one = [&](int j) {
    if (j < C::KPT)
      load_to_lds16(pend_k + j * C::kLoaders * 16, __builtin_amdgcn_readfirstlane(pend_lds + j * C::kLoaders * 16));
    else
      load_to_lds16(pend_v + (j - C::KPT) * C::kLoaders * 16,
                    __builtin_amdgcn_readfirstlane(pend_lds + C::KBytes + (j - C::KPT) * C::kLoaders * 16));
  };

  f32x16_t o[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) o[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};   // S^T of the tile between QK and softmax
  u32x4_t pkv[4];                               // bf16 P of the tile between softmax and PV,
#pragma unroll                                    // one MFMA B operand per 16-key step
  for (int i = 0; i < 4; ++i) pkv[i] = u32x4_t{0u, 0u, 0u, 0u};

  auto stage_ptr = [&](int st) { return smem + st * C::Stage; };

  // S^T = K Q^T for one 64-key tile (two 32-key halves).
  const int k_lane = (hl * kBlock + bf16_key_of_row(col)) * 16;   // this lane's K operand offset
  const int v_lane = C::KBytes + (hl * DV + col) * 16;             // this lane's V operand offset
  auto qk = [&](int st) {
    const unsigned char* kb = stage_ptr(st) + k_lane;
    s0 = f32x16_t{};
    s1 = f32x16_t{};
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      const u32x4_t k0 = *(const u32x4_t*)(kb + 2 * i * kBlock * 16);
      const u32x4_t k1 = *(const u32x4_t*)(kb + (2 * i * kBlock + 32) * 16);
      s0 = mfma_bf16(k0, qreg[i], s0);
      s1 = mfma_bf16(k1, qreg[i], s1);
    }
  };

  // Online softmax of tile j: mask, running max (raised lazily), rescale,
  // P in bf16, running sum of the fp32 P.
  auto softmax = [&](int j) {
    const int64_t key0 = (int64_t)j * kBlock;
    if (key0 + kBlock - 1 > wave_first_pos) {
      const int lim = (int)(pos - key0);          // keys past lim are invisible to this row
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (bf16_key_of_reg(0, r, hl) > lim) s0[r] = -INFINITY;
        if (bf16_key_of_reg(1, r, hl) > lim) s1[r] = -INFINITY;
      }
    }
    float mx = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = half_max(mx);
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
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[2 * rr], cs, -mb));
      const float p1 = fast_exp2(__builtin_fmaf(s0[2 * rr + 1], cs, -mb));
      const float p2 = fast_exp2(__builtin_fmaf(s1[2 * rr], cs, -mb));
      const float p3 = fast_exp2(__builtin_fmaf(s1[2 * rr + 1], cs, -mb));
      psum += (p0 + p1) + (p2 + p3);
      pkv[rr >> 2][rr & 3] = pack_bf16(p0, p1);
      pkv[2 + (rr >> 2)][rr & 3] = pack_bf16(p2, p3);
    }
    l_run += psum;
  };

  // O^T += V^T P^T for tile j.
  auto pv = [&](int st) {
    const unsigned char* vb = stage_ptr(st) + v_lane;
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
        const u32x4_t va = *(const u32x4_t*)(vb + (2 * stp * DV + 32 * b) * 16);
        o[b] = mfma_bf16(va, pkv[stp], o[b]);
      }
    }
  };

  // PV of tile jp and QK of the next tile, issued alternately: six independent
  // accumulator chains (four O blocks, two S halves), so no matrix-core
  // instruction waits on the one just before it.
  auto pv_qk = [&](int st_prev, int st_cur) {
    const unsigned char* vb = stage_ptr(st_prev) + v_lane;
    const unsigned char* kb = stage_ptr(st_cur) + k_lane;
    f32x16_t n0 = f32x16_t{}, n1 = f32x16_t{};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      {   // PV step (stp, b) = (u / NB, u % NB), covering all 16 for NB = 4
        constexpr int kPv = 4 * C::NB;
        if (u < kPv) {
          const int stp = u / C::NB, b = u % C::NB;
          const u32x4_t va = *(const u32x4_t*)(vb + (2 * stp * DV + 32 * b) * 16);
          o[b] = mfma_bf16(va, pkv[stp], o[b]);
        }
      }
      {   // QK step (i, half) = (u / 2, u % 2)
        const int i = u >> 1;
        if (i < C::NQ) {
          const u32x4_t kk = *(const u32x4_t*)(kb + (2 * i * kBlock + 32 * (u & 1)) * 16);
          if (u & 1) n1 = mfma_bf16(kk, qreg[i], n1);
          else n0 = mfma_bf16(kk, qreg[i], n0);
        }
      }
    }
#pragma unroll
    for (int u = 16; u < 2 * C::NQ; ++u) {   // remaining QK steps when d > 128
      const int i = u >> 1;
      const u32x4_t kk = *(const u32x4_t*)(kb + (2 * i * kBlock + 32 * (u & 1)) * 16);
      if (u & 1) n1 = mfma_bf16(kk, qreg[i], n1);
      else n0 = mfma_bf16(kk, qreg[i], n0);
    }
    s0 = n0;
    s1 = n1;
    // Issue order: kLead LDS operand reads ahead, then one matrix op per read,
    // so about kLead reads are in flight while the matrix cores run.
    constexpr int kReads = 4 * C::NB + 2 * C::NQ, kLead = 6;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
    for (int r = 0; r < kReads - kLead; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
  };

  // pv_qk for the leading waves with the pending tile's loads interleaved: the
  // operand reads are software-pipelined by hand (kAhead in flight) and one
  // load goes out after every fourth MFMA, fenced so the order stays as written.
  auto pv_qk_dma = [&](int st_prev, int st_cur, bool with_dma) {
    const unsigned char* vb = stage_ptr(st_prev) + v_lane;
    const unsigned char* kb = stage_ptr(st_cur) + k_lane;
    constexpr int kPv = 4 * C::NB, kQk = 2 * C::NQ, kOps = kPv + kQk, kAhead = 6;
    // op k: PV and QK alternate while both remain, then the rest of QK
    auto is_pv = [&](int k) { return k < 2 * kPv ? (k & 1) == 0 : false; };
    auto op_ptr = [&](int k) -> const u32x4_t* {
      if (is_pv(k)) {
        const int u = k >> 1, stp = u / C::NB, b = u % C::NB;
        return (const u32x4_t*)(vb + (2 * stp * DV + 32 * b) * 16);
      }
      const int q = k < 2 * kPv ? (k >> 1) : k - kPv;      // QK step index
      return (const u32x4_t*)(kb + (2 * (q >> 1) * kBlock + 32 * (q & 1)) * 16);
    };
    f32x16_t n0 = f32x16_t{}, n1 = f32x16_t{};
    u32x4_t rd[kOps];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) rd[k] = *op_ptr(k);
#pragma unroll
    for (int k = 0; k < kOps; ++k) {
      if (is_pv(k)) {
        const int u = k >> 1, stp = u / C::NB, b = u % C::NB;
        o[b] = mfma_bf16(rd[k], pkv[stp], o[b]);
      } else {
        const int q = k < 2 * kPv ? (k >> 1) : k - kPv;
        if (q & 1) n1 = mfma_bf16(rd[k], qreg[q >> 1], n1);
        else n0 = mfma_bf16(rd[k], qreg[q >> 1], n0);
      }
      if (k + kAhead < kOps) rd[k + kAhead] = *op_ptr(k + kAhead);
      if ((k & 3) == 3 && (k >> 2) < C::LPT) {
        __builtin_amdgcn_sched_barrier(0);
        if (with_dma) dma_one(k >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    static_assert(kOps >= 4 * C::LPT, "one load per four MFMAs must fit in the matrix phase");
    s0 = n0;
    s1 = n1;
  };

  // ---- key loop -------------------------------------------------------------------
  // Interval i (between two barriers) does, for every wave, PV of tile i-1,
  // QK of tile i and the softmax of the tile in between.  Waves 0-3 run
  // "PV(i-1), QK(i), softmax(i)"; waves 4-7 run "softmax(i-1), PV(i-1), QK(i)".
  // Waves w and w+4 share a SIMD, so while one streams matrix-core work the
  // other runs its softmax on the vector ALUs, and they swap halfway.
  // Tile t is read in intervals t and t+1; its stage is refilled with tile
  // t + kStages, issued in interval t + 2, which leaves kStages - 2 intervals
  // for the load to land.
  constexpr int NS = C::kStages;
  const int n = j_hi - j_lo;
#pragma unroll
  for (int p = 0; p < NS - 2; ++p)
    if (p < n) issue(bt4[j_lo + p], p);
  int32_t block_ahead = (NS - 2 < n) ? bt4[j_lo + NS - 2] : 0;
  // Start of interval i: tile i must have landed (tiles i+1 .. i+NS-3 may
  // still be in flight); after the barrier the stage of tile i-2 is free and
  // receives tile i+NS-2.
  bool pending = false;
  auto interval_start = [&](int i) {
    if (i < n) {
      if (min(NS - 3, n - 1 - i) >= 1) wait_vmem<C::LPT>();
      else wait_vmem<0>();
    }
    workgroup_barrier();
    pending = i + NS - 2 < n;
    if (pending) {
      if (i == 0) issue(block_ahead, NS - 2);          // no matrix phase to hide it in
      else prep(block_ahead, (i + NS - 2) % NS);       // issued inside pv_qk_dma
    }
    block_ahead = (i + NS - 1 < n) ? bt4[j_lo + i + NS - 1] : 0;
    const int64_t key0 = (int64_t)(j_lo + i) * kBlock;
    if (i < n && key0 + kBlock > kv_len) {
      // The tile holding the sequence end: zero its values of keys >= kv_len
      // in LDS (a masked key has probability 0, but 0 * NaN would poison the
      // sum).  Nobody reads this V before the next barrier.
      uint16_t* vt = (uint16_t*)(stage_ptr(i % NS) + C::KBytes);
      const int first = (int)(kv_len - key0);          // 1..63 keys stay
      const int count = (kBlock - first) * DV;
      for (int e = tid; e < count; e += C::kThreads) {
        const int key = first + e / DV, dv = e % DV;
        vt[((key >> 3) * DV + dv) * 8 + (key & 7)] = 0;
      }
    }
  };
  // Each group has its own copy of the loop, so only P (leading waves) or
  // only S (trailing waves) stays live across the barrier.  Every wave runs
  // every tile of the workgroup's range: a tile past a wave's rows is fully
  // masked (probability 0 against finite values), which leaves its output
  // unchanged and keeps one straight-line loop body.  Scheduling fences keep
  // the matrix and vector phases in one piece each, so the two waves of a
  // SIMD stay interleaved as written.
  if (wave < 4) {
    interval_start(0);
    qk(0);
    __builtin_amdgcn_sched_barrier(0);
    softmax(j_lo);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 1; i < n; ++i) {
      interval_start(i);
      pv_qk_dma((i - 1) % NS, i % NS, pending);
      __builtin_amdgcn_sched_barrier(0);
      softmax(j_lo + i);
      __builtin_amdgcn_sched_barrier(0);
    }
    interval_start(n);
    pv((n - 1) % NS);
  } else {
    interval_start(0);
    qk(0);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 1; i < n; ++i) {
      interval_start(i);
      softmax(j_lo + i - 1);
      __builtin_amdgcn_sched_barrier(0);
      pv_qk((i - 1) % NS, i % NS);
      __builtin_amdgcn_sched_barrier(0);
    }
    interval_start(n);
    softmax(j_lo + n - 1);
    __builtin_amdgcn_sched_barrier(0);
    pv((n - 1) % NS);
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
        if constexpr (sizeof(EO) == 2) *(u32x2_t*)(orow + dv0) = u32x2_t{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        else *(f32x4_t*)(orow + dv0) = f32x4_t{v0, v1, v2, v3};
      }
    if (lse && hl == 0) lse[(int64_t)h * a.lse_stride + t] = (m_run * cs + __log2f(l_tot)) * kLn2;
  } else {
    const int64_t R = c * a.heads;
    const int64_t row = t * a.heads + h;
    float* wo = a.ws_o + ((int64_t)split * R + row) * DV;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(f32x4_t*)(wo + 32 * b + 8 * rq + 4 * hl) =
            f32x4_t{o[b][4 * rq], o[b][4 * rq + 1], o[b][4 * rq + 2], o[b][4 * rq + 3]};
    if (hl == 0)
      *(float2*)(a.ws_ml + ((int64_t)split * R + row) * 2) =
          make_float2(m_run == -INFINITY ? -INFINITY : m_run * cs, l_tot);
  }
}

// ---- host launchers -----------------------------------------------------------------

bool prefill_paged_supported(int D, int DV) {
  return (D == 64 && DV == 64) || (D == 128 && DV == 128) || (D == 192 && DV == 128);
}

template <typename EO, bool kVarlen>
static hipError_t launch_paged_dims(int D, int DV, const PrefillArgs& a, int grid, hipStream_t s) {
  if (D == 64 && DV == 64)
    hipLaunchKernelGGL((prefill_paged_kernel<EO, 64, 64, kVarlen>), dim3(grid), dim3(512), 0, s, a);
  else if (D == 128 && DV == 128)
    hipLaunchKernelGGL((prefill_paged_kernel<EO, 128, 128, kVarlen>), dim3(grid), dim3(512), 0, s, a);
  else if (D == 192 && DV == 128)
    hipLaunchKernelGGL((prefill_paged_kernel<EO, 192, 128, kVarlen>), dim3(grid), dim3(512), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill_paged(DType out, int D, int DV, const PrefillArgs& a, int grid, hipStream_t stream) {
  if (out == DType::BF16) return launch_paged_dims<uint16_t, false>(D, DV, a, grid, stream);
  return launch_paged_dims<float, false>(D, DV, a, grid, stream);
}

hipError_t launch_prefill_paged_varlen(int D, int DV, const PrefillArgs& a, int grid, hipStream_t stream) {
  return launch_paged_dims<uint16_t, true>(D, DV, a, grid, stream);
}

}  // namespace chunkattn
