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
//    Only the four leading waves issue them, one load after every eighth MFMA
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
//  * Per wave, S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16:
//    the wave's 32 query rows are two 16-row blocks, and every 1 KiB K or V
//    operand read from LDS feeds one MFMA per block, so LDS bytes per flop
//    are those of v_mfma_f32_32x32x16_bf16.  On random bf16 data the chip is
//    power-bound; measured on MI355X, this loop holds a ~17% higher shader
//    clock with the 16x16x32 shape than with 32x32x16 but needs more issue
//    cycles (twice the MFMA instructions, 4-lane row reductions).  With the
//    softmax kept to the minimum of vector ops it comes out 2-3% faster.
//    A lane holds query 16*blk + lane%16 and, in lane group g = lane/16, keys
//    8g..8g+7 of every 32-key step: the K tile's LDS slots are ordered by the
//    loads themselves (key_of_slot) so that the accumulator registers of two
//    QK blocks are exactly the bf16 P^T operand of the PV step over those 8
//    keys, which one 16-byte read of the V tile matches.  Row maxima and sums
//    combine the 4 lanes of a query with v_permlane16/32_swap.
//  * Per row the softmax keeps the running offset m (the exact maximum of the
//    workgroup's first tile, raised lazily after that), the exp offset
//    -m*scale and the threshold a new maximum must pass; a tile costs one fma
//    + exp per logit, the fp32 row sum and the pack to bf16.  The row maxima
//    are reduced over the lanes of a row only on the first tile and when a
//    lane's row sum shows that some logit may have passed the threshold.
//    Measured on MI355X, dropping the per-tile maximum this way is 3% faster
//    on the 128K chunks and on the 512K MLA-shaped chunks.
//  * The two waves that share a SIMD run the same tiles half an interval
//    apart (ping-pong), so one feeds the matrix cores while the other
//    computes its softmax; the rescale is skipped when no row's maximum grew.
//  * Values of keys past the sequence end are zeroed in LDS once the tile
//    holding the sequence end has landed, logits past a row's position are
//    masked with a select, so NaN in unused pool slots never reaches an output.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace chunkattn {

// Bound on a lane's sum of its 16 exps of one row while no logit exceeds the
// row's offset by more than kLazyRescale: 16 x 2^kLazyRescale.
constexpr float kPsumCap = 16.f * (1 << (int)kLazyRescale);

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
  static constexpr int QS = D / 32;                    // 32-feature steps of QK
  static constexpr int NDB = DV / 16;                  // 16-value blocks of O
  static constexpr int KF = 4 * QS;                    // K operands per tile: 4 key blocks x QS
  static constexpr int VF = 2 * NDB;                   // V operands per tile: 2 key steps x NDB
  static_assert(KBytes % (16 * kLoaders) == 0 && VBytes % (16 * kLoaders) == 0, "tile split");
  static_assert(VF <= KF, "PV operands interleave with QK operands");
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from global memory (uniform base + this lane's 32-bit
// offset) straight into LDS at m0 + 16 * lane.
__device__ __forceinline__ void load_to_lds16(const void* base, uint32_t lane_off, uint32_t lds_wave_base) {
  // one wait state between the M0 write and the load that reads it (a GFX9 hazard)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_wave_base), "v"(lane_off), "s"(base)
               : "memory", "m0");
}

// The same load split in two for the matrix phase: set_m0 writes the LDS
// destination, and load_at_m0, issued two MFMAs later, reads it.  The MFMAs
// between them are the wait state the M0 hazard needs, so neither carries an
// s_nop.  Sound only because nothing the compiler emits in this kernel writes
// m0: every m0 write is one of these asm statements.
__device__ __forceinline__ void set_m0(uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0" ::"s"(lds_wave_base) : "m0");
}
__device__ __forceinline__ void load_at_m0(const void* base, uint32_t lane_off) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Combine x over the four lanes l, l^16, l^32, l^48 that hold one query row.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Row maxima of both query blocks at once: x0, x1 are this lane's partial
// maxima of blocks 0 and 1.  permlane16_swap(x0, x1) hands lane group g the
// pair (x0 of group g&~1, x1 of group g&~1) or its odd partners, so one max
// leaves group 0 / 2 with block 0 over groups {0,1} / {2,3} and group 1 / 3
// with block 1; permlane32_swap folds the two halves, and a last
// permlane16_swap gives every lane both totals.
__device__ __forceinline__ void quad_max2(float& x0, float& x1) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float c = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  const float d = max_raw(__uint_as_float(u[0]), __uint_as_float(u[1]));
  const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(d), __float_as_uint(d), false, false);
  x0 = __uint_as_float(v[0]);
  x1 = __uint_as_float(v[1]);
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return half_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// LDS slot s of a 64-key K chunk holds key key_of_slot(s).  Slot 16b + m is
// row m of QK key block b, which stands for key 32(b>>1) + 8(m>>2) + 4(b&1) + (m&3):
// lane group g then finds keys 8g..8g+3 of a 32-key step in block 2*step and
// keys 8g+4..8g+7 in block 2*step+1.
__device__ __forceinline__ int key_of_slot(int s) {
  const int b = s >> 4, m = s & 15;
  return 32 * (b >> 1) + 8 * (m >> 2) + 4 * (b & 1) + (m & 3);
}
// Key offset (before the lane group's 8g) of register r of QK block b.
__host__ __device__ constexpr int key_of_reg(int b, int r) { return 32 * (b >> 1) + 4 * (b & 1) + r; }

template <typename EO, int D, int DV, bool kVarlen, bool kContig = false>
__global__ __launch_bounds__(512, 1) void prefill_paged_kernel(const PrefillArgs a) {
  using C = PagedCfg<D, DV>;
  static_assert(!kContig || (D == 128 && DV == 128 && !kVarlen), "token-major tiles are laid out for d = 128");
  // Raw tile stages, and the intervals a tile's stage is read in: two on the
  // paged pool (K by QK(t), V by PV(t) one interval later); one on a
  // contiguous cache, whose V tile is transposed into one of two V^T buffers
  // in its own interval and read by PV from there.
  constexpr int NS = kContig ? 3 : C::kStages;
  constexpr int kReads = kContig ? 1 : 2;
  constexpr int NA = NS - kReads;                // tiles in flight ahead of the current one
  static_assert(NA == 1 || NA == 2, "at most one tile in flight past the one awaited");
  constexpr int kSmem = NS * C::Stage + (kContig ? 2 * C::VBytes : 0);
  static_assert(kSmem <= 131072, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lc = lane & 15;   // lane group (8-key run / 8-feature run), query column
  const int hpw = a.hpw;                      // heads per workgroup: 8, 4, 2 or 1
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

  // This lane's two query rows, one per 16-row block.
  int64_t t[2], pos[2];
  bool row_valid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    t[qb] = t0 + 16 * qb + lc;
    row_valid[qb] = t[qb] < c;
    pos[qb] = P + (row_valid[qb] ? t[qb] : c - 1);
  }
  const int64_t wave_first_pos = P + min(t0, c - 1);
  const int wave_first_pos32 = __builtin_amdgcn_readfirstlane((int)wave_first_pos);
  const int kv_len32 = __builtin_amdgcn_readfirstlane((int)kv_len);
  const float cs = a.scale_log2;

  if (j_lo >= j_hi) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      if (row_valid[qb] && lg == 0) {
        const int64_t row = t[qb] * a.heads + h;
        *(float2*)(a.ws_ml + ((int64_t)split * c * a.heads + row) * 2) = make_float2(-INFINITY, 0.f);
      }
    return;
  }

  // Query rows of this lane as B operands (features 32i + 8lg .. +7), held for the whole key loop.
  u32x4_t qreg[2][C::QS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t* qrow = qbase + ((pos[qb] - P) * a.heads + h) * (int64_t)D + 8 * lg;
#pragma unroll
    for (int i = 0; i < C::QS; ++i) qreg[qb][i] = *(const u32x4_t*)(qrow + 32 * i);
  }

  // ---- tile transfer: block table through the scalar unit, data straight into LDS ----
  // A K load instruction covers one 8-feature chunk of all 64 keys; lane s
  // fetches key key_of_slot(s) into slot s.  V keeps the pool's order.
  // Loop-local bases (this split's first block-table entry, this KV head's
  // first tile), so the key loop holds none of the argument block.
  const __attribute__((address_space(4))) int32_t* bt4 =
      kContig ? nullptr : (const __attribute__((address_space(4))) int32_t*)(btab + j_lo);
  // Tile handle: the block id of tile j_lo + idx (paged) or its index (contiguous cache).
  auto tile_id = [&](int idx) -> int32_t {
    if constexpr (kContig) return j_lo + idx;
    else return bt4[idx];
  };
  const unsigned char* kpool = (const unsigned char*)a.k + (int64_t)g * C::KBytes;
  const unsigned char* vpool = (const unsigned char*)a.v + (int64_t)g * C::VBytes;
  const int64_t kstride = (int64_t)a.kv_heads * C::KBytes, vstride = (int64_t)a.kv_heads * C::VBytes;
  const uint32_t smem_base = lds_address(smem);
  // Pool tiles: load i of leading wave w moves the 1 KB unit 4 i + w of K (one
  // 8-feature run of all 64 keys, lane s fetching key key_of_slot(s) into slot
  // s) or of V, so the four waves' i-th loads cover 4 contiguous KB.  The
  // per-load lane offsets are set up once (a block-relative address per load,
  // 6 more registers than one shared offset), so a load adds nothing to the
  // block base: 0.6 % on the 128K loop against a 64-bit scalar add per load.
  // Giving each wave a contiguous run instead, so that the loads could share
  // one offset through the instruction's immediate, was 0.7 % slower: the
  // waves' concurrent loads then sit 4 KB apart rather than side by side.
  constexpr int kUnits = C::kLoaders / 64;       // 1 KB units per load of the four waves
  uint32_t k_off_lane[C::KPT], v_off_lane[C::VPT];
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) k_off_lane[i] = (kUnits * i + wave) * 1024 + key_of_slot(lane) * 16;
#pragma unroll
  for (int i = 0; i < C::VPT; ++i) v_off_lane[i] = (kUnits * i + wave) * 1024 + lane * 16;
  auto pool_m0 = [&](uint32_t lds_part, int i) {
    return __builtin_amdgcn_readfirstlane(lds_part + (kUnits * i + wave) * 1024);
  };
  auto pool_load = [&](const unsigned char* blk, uint32_t lane_off, uint32_t lds_part, int i) {
    load_to_lds16(blk, lane_off, pool_m0(lds_part, i));
  };
  // Contiguous cache ([tokens][kv_heads][128], token-major): the tiles are laid
  // out token-major in LDS, one 256-byte row per key, its 16-byte units
  // permuted per row so that operand reads meet no bank conflict.
  //  * K: LDS row s holds key key_of_slot(s) (the order the S^T registers need);
  //    unit u of row s holds feature run u ^ (s & 15).
  //  * V: row = key; unit u of row key holds value run u ^ fv(key),
  //    fv(key) = 2 (key & 3) + 8 ((key >> 3) & 1).
  // Each direct load then moves whole 256-byte rows of four keys; a lane's
  // load i of a tile reads K key kc_lane + kio(i), V key vkey_lane + 16 i, at
  // fixed units.  Keys past the sequence end read its last row (finite,
  // masked), so no slot past the cache is touched and nothing needs zeroing.
  const unsigned char* kcont = (const unsigned char*)a.k + (int64_t)g * a.k_stride_head * 2;
  const unsigned char* vcont = (const unsigned char*)a.v + (int64_t)g * a.v_stride_head * 2;
  const uint32_t ktok = (uint32_t)(a.k_stride_tok * 2), vtok = (uint32_t)(a.v_stride_tok * 2);
  const int mslot = 4 * (wave & 3) + (lane >> 4);
  const int kc_lane = 8 * (mslot >> 2) + (mslot & 3);
  const uint32_t krun_off = (uint32_t)(((lane & 15) ^ mslot) * 16);
  const int vkey_lane = mslot;
  const uint32_t vunit_off = (uint32_t)(((lane & 15) ^ (2 * ((lane >> 4) & 3) + 8 * ((vkey_lane >> 3) & 1))) * 16);
  auto kio = [](int i) { return 32 * (i >> 1) + 4 * (i & 1); };
  auto k_cont_off = [&](int i, int lim) { return (uint32_t)min(kc_lane + kio(i), lim) * ktok + krun_off; };
  auto v_cont_off = [&](int i, int lim) { return (uint32_t)min(vkey_lane + 16 * i, lim) * vtok + vunit_off; };
  auto issue = [&](int32_t block_id, int st) {
    if (wave >= 4) return;
    if constexpr (kContig) {
      const int key0 = block_id * kBlock;
      const int lim = min(kBlock - 1, kv_len32 - 1 - key0);
      const unsigned char* kb = kcont + (int64_t)key0 * ktok;
      const unsigned char* vb = vcont + (int64_t)key0 * vtok;
      const uint32_t ks = smem_base + st * C::Stage;
#pragma unroll
      for (int i = 0; i < C::KPT; ++i)
        load_to_lds16(kb, k_cont_off(i, lim), __builtin_amdgcn_readfirstlane(ks + (wave * 64 + i * C::kLoaders) * 16));
#pragma unroll
      for (int i = 0; i < C::VPT; ++i)
        load_to_lds16(vb, v_cont_off(i, lim),
                      __builtin_amdgcn_readfirstlane(ks + C::KBytes + (wave * 64 + i * C::kLoaders) * 16));
      return;
    }
    const int phys = clamp_block(block_id, a.num_blocks);
    const unsigned char* kb = kpool + phys * kstride;
    const unsigned char* vb = vpool + phys * vstride;
    const uint32_t ks = smem_base + st * C::Stage;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) pool_load(kb, k_off_lane[i], ks, i);
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) pool_load(vb, v_off_lane[i], ks + C::KBytes, i);
  };
  // The same transfer spread over the leading waves' matrix phase: prep() fixes
  // the tile and stage, and load j moves this thread's j-th 16-byte chunk (K
  // chunks first, then V).  Issued in a burst, the loads would hold the wave
  // for as long as the direct-to-LDS path needs to drain a tile; one load per
  // eight MFMAs stays under that rate, so the wave never waits at issue.
  const unsigned char* pend_k = kpool;
  const unsigned char* pend_v = vpool;
  uint32_t pend_lds = 0;                         // the stage (pool) or this wave's first unit in it (contiguous)
  int pend_lim = 0;                              // contiguous cache: last key of the pending tile
  auto prep = [&](int32_t block_id, int st) {
    if constexpr (kContig) {
      const int key0 = block_id * kBlock;
      pend_lim = min(kBlock - 1, kv_len32 - 1 - key0);
      pend_k = kcont + (int64_t)key0 * ktok;
      pend_v = vcont + (int64_t)key0 * vtok;
    } else {
      const int phys = clamp_block(block_id, a.num_blocks);
      pend_k = kpool + phys * kstride;
      pend_v = vpool + phys * vstride;
    }
    pend_lds = smem_base + st * C::Stage + (kContig ? wave * 64 * 16 : 0);
  };
  // Pool tiles: dma_m0(j) then dma_load(j), the LDS destination and the load
  // of chunk j.  The contiguous cache keeps the single-statement load: its
  // registers are nearly all in use, and the extra scheduling fences of the
  // split form cost it ~5 %.
  auto dma_m0 = [&](int j) {
    if (j < C::KPT) set_m0(pool_m0(pend_lds, j));
    else set_m0(pool_m0(pend_lds + C::KBytes, j - C::KPT));
  };
  auto dma_load = [&](int j) {
    if (j < C::KPT) load_at_m0(pend_k, k_off_lane[j]);
    else load_at_m0(pend_v, v_off_lane[j - C::KPT]);
  };
  auto dma_one_contig = [&](int j) {
    if (j < C::KPT)
      load_to_lds16(pend_k, k_cont_off(j, pend_lim), __builtin_amdgcn_readfirstlane(pend_lds + j * C::kLoaders * 16));
    else
      load_to_lds16(pend_v, v_cont_off(j - C::KPT, pend_lim),
                    __builtin_amdgcn_readfirstlane(pend_lds + C::KBytes + (j - C::KPT) * C::kLoaders * 16));
  };

  f32x4_t o[C::NDB][2];
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  // Per row, kept in step with m_run: the exp offset -m_run*cs (0 while no key
  // was visible) and the threshold m_run + kLazyRescale/cs that a new maximum
  // must pass to be taken (cs > 0: the boundary rejects other scales).
  float neg_mb[2] = {0.f, 0.f}, thr[2] = {-INFINITY, -INFINITY};
  const float lazy_unscaled = kLazyRescale / cs;
  f32x4_t s[4][2];                              // S^T of the tile between QK and softmax
#pragma unroll
  for (int b = 0; b < 4; ++b) s[b][0] = s[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t pkv[2][2];                            // bf16 P^T of the tile between softmax and PV,
#pragma unroll                                    // one B operand per (query block, 32-key step)
  for (int qb = 0; qb < 2; ++qb) pkv[qb][0] = pkv[qb][1] = u32x4_t{0u, 0u, 0u, 0u};

  auto stage_ptr = [&](int st) { return smem + st * C::Stage; };
  // Where PV reads the V operands of tile i: the stage's V part (paged pool)
  // or V^T buffer i & 1 (contiguous cache); both hold the pool's V block order.
  auto v_base = [&](int i) -> const unsigned char* {
    if constexpr (kContig) return smem + NS * C::Stage + (i & 1) * C::VBytes;
    else return stage_ptr(i % NS) + C::KBytes;
  };

  // Operand offsets: K operand (key block b, feature step i) at k_lane + (256 i + 16 b) * 16,
  // V operand (key step ks, value block db) at v_lane + (4 ks DV + 16 db) * 16.
  const int k_lane = (lg * kBlock + lc) * 16;
  const int v_lane = (lg * DV + lc) * 16;
  auto k_off = [](int q) { return (256 * (q >> 2) + 16 * (q & 3)) * 16; };            // QK operand q = 4 i + b
  auto v_off = [](int u) { return (4 * (u / C::NDB) * DV + 16 * (u % C::NDB)) * 16; };   // PV operand u = NDB ks + db
  // Contiguous-cache tiles (token-major rows, see above): K operand (step i, block b)
  // at row 16 b + lc, unit (4 i + lg) ^ lc; the V^T operand (step ks, block db) of
  // the raw V tile is two transposing reads: lane c of group lg at row
  // 32 ks + 8 lg + c / 4 (then 4 rows on), value run 2 db + (c % 4) / 2
  // (permuted), half c % 2.
  // This wave transposes V^T operands u = 2 wave and 2 wave + 1 (step u / 8, block u % 8).
  int kq[4], vq[2];
  if constexpr (kContig) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kq[i] = lc * 256 + ((4 * i + lg) ^ lc) * 16;
    const int fv = 2 * (lc >> 2) + 8 * (lg & 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int u = 2 * wave + e, ks = u / C::NDB, db = u % C::NDB;
      vq[e] = (32 * ks + 8 * lg + (lc >> 2)) * 256 + ((2 * db + ((lc & 3) >> 1)) ^ fv) * 16 + (lc & 1) * 8;
    }
  }
  auto k_read = [&](const unsigned char* stage, int q) -> u32x4_t {
    if constexpr (kContig) return *(const u32x4_t*)(stage + kq[q >> 2] + 4096 * (q & 3));
    else return *(const u32x4_t*)(stage + k_lane + k_off(q));
  };
  auto v_read = [&](const unsigned char* vb, int u) -> u32x4_t {
    return *(const u32x4_t*)(vb + v_lane + v_off(u));
  };
  // Contiguous cache: this wave's two V^T operands (u = 2 wave, 2 wave + 1) of
  // tile i, read from the raw token-major tile and written to V^T buffer i & 1
  // at the place PV reads them, so the eight waves transpose the tile once.
  // All four transposing reads go out before the first write waits on them.
  auto vt_fill = [&](int i) {
    if constexpr (kContig) {
      const unsigned char* raw = stage_ptr(i % NS) + C::KBytes;
      unsigned char* dst = smem + NS * C::Stage + (i & 1) * C::VBytes + v_lane;
      v4i16_t lo[2], hi[2];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const unsigned char* pp = raw + vq[e];
        lo[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)pp);
        hi[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pp + 4 * 256));
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo[e]), h2 = __builtin_bit_cast(u32x2_t, hi[e]);
        *(u32x4_t*)(dst + v_off(2 * wave + e)) = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // the four LDS reads, then
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);   // the two LDS writes
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  static_assert(!kContig || 2 * 8 == C::VF, "two V^T operands per wave cover the tile");
  auto qk_mfma = [&](int q, u32x4_t kf, f32x4_t (&n)[4][2]) {
    n[q & 3][0] = mfma16(kf, qreg[0][q >> 2], n[q & 3][0]);
    n[q & 3][1] = mfma16(kf, qreg[1][q >> 2], n[q & 3][1]);
  };
  auto pv_mfma = [&](int u, u32x4_t vf) {
    const int ks = u / C::NDB, db = u % C::NDB;
    o[db][0] = mfma16(vf, pkv[0][ks], o[db][0]);
    o[db][1] = mfma16(vf, pkv[1][ks], o[db][1]);
  };

  // S^T = K Q^T for one 64-key tile.
  auto qk = [&](int st) {
    const unsigned char* stg = stage_ptr(st);
    f32x4_t n[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) n[b][0] = n[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < C::KF; ++q) qk_mfma(q, k_read(stg, q), n);
#pragma unroll
    for (int b = 0; b < 4; ++b) s[b][0] = n[b][0], s[b][1] = n[b][1];
  };

  // Online softmax of tile j: mask, exps with the running offset, running sum
  // of the fp32 P, P in bf16.  The offset (running max m) is set exactly on a
  // workgroup's first tile and afterwards raised only when needed: while no
  // logit exceeds m by more than kLazyRescale (log2 units after the scale),
  // every exp is at most 2^kLazyRescale, so a lane's 16 exps of one row sum to
  // at most kPsumCap.  A larger (or infinite) sum is therefore the only case
  // that may need a new offset; only then are the row maxima reduced over the
  // 4 lanes of a row, and a row whose maximum passed the threshold is rescaled
  // and its exps redone.  Otherwise each exp stays below kPsumCap, which keeps
  // the fp32 sums far from overflow, so the result is the same softmax.
  auto softmax = [&](int j, bool first, auto maskable_tag) {
    const int key0 = j * kBlock;                 // positions stay below 2^30 (the boundary checks it)
    if (decltype(maskable_tag)::value && key0 + kBlock - 1 > wave_first_pos32) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int lim = (int)(pos[qb] - key0) - 8 * lg;   // register offsets past lim are invisible
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key_of_reg(b, r) > lim) s[b][qb][r] = -INFINITY;
      }
    }
    float p[2][4][4];
    auto exps = [&]() {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[qb][b][r] = fast_exp2(__builtin_fmaf(s[b][qb][r], cs, neg_mb[qb]));
    };
    float psum[2];
    auto row_sums = [&]() {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float (&pq)[4][4] = p[qb];
        float acc = (pq[0][0] + pq[0][1]) + (pq[0][2] + pq[0][3]);
#pragma unroll
        for (int b = 1; b < 4; ++b) acc += (pq[b][0] + pq[b][1]) + (pq[b][2] + pq[b][3]);
        psum[qb] = acc;
      }
    };
    exps();
    row_sums();
    if (first || (__builtin_amdgcn_ballot_w64(!(psum[0] <= kPsumCap)) |
                  __builtin_amdgcn_ballot_w64(!(psum[1] <= kPsumCap))) != 0) {
      float mx[2];
      bool grow[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m = max3_raw(s[0][qb][0], s[0][qb][1], s[0][qb][2]);
        m = max3_raw(m, s[0][qb][3], s[1][qb][0]);
        m = max3_raw(m, s[1][qb][1], s[1][qb][2]);
        m = max3_raw(m, s[1][qb][3], s[2][qb][0]);
        m = max3_raw(m, s[2][qb][1], s[2][qb][2]);
        m = max3_raw(m, s[2][qb][3], s[3][qb][0]);
        m = max3_raw(m, s[3][qb][1], s[3][qb][2]);
        mx[qb] = max_raw(m, s[3][qb][3]);
      }
      quad_max2(mx[0], mx[1]);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) grow[qb] = mx[qb] > thr[qb];
      if (__any(grow[0] || grow[1])) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = grow[qb] ? mx[qb] : m_run[qb];
          const float alpha = grow[qb] ? fast_exp2((m_run[qb] - m_new) * cs) : 1.f;
          l_run[qb] *= alpha;
#pragma unroll
          for (int b = 0; b < C::NDB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[b][qb][r] *= alpha;
          m_run[qb] = m_new;
          if (grow[qb]) {
            neg_mb[qb] = -(m_new * cs);
            thr[qb] = m_new + lazy_unscaled;
          }
        }
        exps();
        row_sums();
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float (&pq)[4][4] = p[qb];
      l_run[qb] += psum[qb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pkv[qb][ks] = u32x4_t{pack_bf16(pq[2 * ks][0], pq[2 * ks][1]), pack_bf16(pq[2 * ks][2], pq[2 * ks][3]),
                              pack_bf16(pq[2 * ks + 1][0], pq[2 * ks + 1][1]),
                              pack_bf16(pq[2 * ks + 1][2], pq[2 * ks + 1][3])};
    }
  };

  // O^T += V^T P^T for one tile.
  auto pv = [&](int i) {
    const unsigned char* vb = v_base(i);
#pragma unroll
    for (int u = 0; u < C::VF; ++u) pv_mfma(u, v_read(vb, u));
  };

  // Operand order of the combined matrix phase: PV and QK operands alternate
  // while both remain, then the rest of QK.  Every operand feeds two MFMAs on
  // independent accumulators, so no matrix-core instruction waits on the one
  // just before it.
  constexpr int kOps = C::VF + C::KF;
  auto is_pv = [](int k) { return k < 2 * C::VF ? (k & 1) == 0 : false; };
  auto qk_index = [](int k) { return k < 2 * C::VF ? (k >> 1) : k - C::VF; };

  // PV of the previous tile and QK of the current one (trailing waves).
  auto pv_qk = [&](int i) {
    const unsigned char* vs = v_base(i - 1);
    const unsigned char* kst = stage_ptr(i % NS);
    f32x4_t n[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) n[b][0] = n[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kOps; ++k) {
      if (is_pv(k)) pv_mfma(k >> 1, v_read(vs, k >> 1));
      else qk_mfma(qk_index(k), k_read(kst, qk_index(k)), n);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) s[b][0] = n[b][0], s[b][1] = n[b][1];
    // Issue order: kLead LDS operand reads ahead, then two matrix ops per read,
    // so about kLead reads are in flight while the matrix cores run.
    constexpr int kLead = 8;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
    for (int r = 0; r < kOps - kLead; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kLead, 0);
  };

  // pv_qk for the leading waves with the pending tile's loads interleaved: the
  // operand reads are software-pipelined by hand (kAhead in flight) and one
  // load goes out after every fourth operand (eighth MFMA), its m0 written
  // two operands before (pool tiles), fenced so the order stays as written.  Whether the interval moves a tile is a
  // compile-time tag: a runtime test at each load point put branches into the
  // matrix phase and cost ~3.5 % of the loop.
  auto pv_qk_dma = [&](int i, auto with_dma_tag) {
    constexpr bool with_dma = decltype(with_dma_tag)::value;
    const unsigned char* vs = v_base(i - 1);
    const unsigned char* kst = stage_ptr(i % NS);
    constexpr int kAhead = 8;
    auto op_read = [&](int k) -> u32x4_t {
      if (is_pv(k)) return v_read(vs, k >> 1);
      return k_read(kst, qk_index(k));
    };
    f32x4_t n[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) n[b][0] = n[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t rd[kOps];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) rd[k] = op_read(k);
#pragma unroll
    for (int k = 0; k < kOps; ++k) {
      if (is_pv(k)) pv_mfma(k >> 1, rd[k]);
      else qk_mfma(qk_index(k), rd[k], n);
      if (k + kAhead < kOps) rd[k + kAhead] = op_read(k + kAhead);
      if constexpr (with_dma && !kContig) {
        if ((k & 3) == 1 && (k >> 2) < C::LPT) {
          __builtin_amdgcn_sched_barrier(0);
          dma_m0(k >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if ((k & 3) == 3 && (k >> 2) < C::LPT) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (with_dma) {
          if constexpr (kContig) dma_one_contig(k >> 2);
          else dma_load(k >> 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    static_assert(kOps >= 4 * C::LPT, "one load per four operands must fit in the matrix phase");
#pragma unroll
    for (int b = 0; b < 4; ++b) s[b][0] = n[b][0], s[b][1] = n[b][1];
  };

  // ---- key loop -------------------------------------------------------------------
  // Interval i (between two barriers) does, for every wave, PV of tile i-1,
  // QK of tile i and the softmax of the tile in between.  Waves 0-3 run
  // "PV(i-1), QK(i), softmax(i)"; waves 4-7 run "softmax(i-1), PV(i-1), QK(i)".
  // Waves w and w+4 share a SIMD, so while one streams matrix-core work the
  // other runs its softmax on the vector ALUs, and they swap halfway.
  // Tile t's stage is read in intervals t .. t + kReads - 1 and refilled with
  // tile t + NS, issued in interval t + kReads, which leaves NA = NS - kReads
  // intervals for the load to land.  On a contiguous cache every wave also
  // transposes its share of V(t) in interval t (vt_fill), before its phases.
  const int n = j_hi - j_lo;
#pragma unroll
  for (int p = 0; p < NA; ++p)
    if (p < n) issue(tile_id(p), p);
  int32_t block_ahead = (NA < n) ? tile_id(NA) : 0;
  // Start of interval i: tile i must have landed (tile i+1 may still be in
  // flight); after the barrier the stage of tile i-kReads is free and
  // receives tile i+NA.
  bool pending = false;
  auto interval_start = [&](int i) {
    if (i < n) {
      if (min(NA - 1, n - 1 - i) >= 1) wait_vmem<C::LPT>();
      else wait_vmem<0>();
    }
    workgroup_barrier();
    pending = i + NA < n;
    if (pending) {
      if (i == 0) issue(block_ahead, NA % NS);         // no matrix phase to hide it in
      else if (wave < 4) prep(block_ahead, (i + NA) % NS);   // issued inside pv_qk_dma
    }
    block_ahead = (i + NA + 1 < n) ? tile_id(i + NA + 1) : 0;
    const int key0 = (j_lo + i) * kBlock;
    if (!kContig && i < n && key0 + kBlock > kv_len32) {
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
    if (i < n) vt_fill(i);
  };
  // Each group has its own copy of the loop, so only P (leading waves) or
  // only S (trailing waves) stays live across the barrier.  Every wave runs
  // every tile of the workgroup's range: a tile past a wave's rows is fully
  // masked (probability 0 against finite values), which leaves its output
  // unchanged and keeps one straight-line loop body.  Scheduling fences keep
  // the matrix and vector phases in one piece each, so the two waves of a
  // SIMD stay interleaved as written.
  // Tiles from j_mask on hold keys past this wave's first row and need the
  // causal mask; the tiles before them never do.  Both splits below are
  // compile-time tags of the loop bodies (wave-uniform bounds; every wave still
  // runs n + 1 intervals).  The contiguous-cache kernel keeps the mask test in
  // every body (measured faster there: its registers are nearly all in use).
  const int i_mask = kContig ? 0 : max(0, (wave_first_pos32 + 1) / kBlock - j_lo);
  if (wave < 4) {
    interval_start(0);
    qk(0);
    __builtin_amdgcn_sched_barrier(0);
    softmax(j_lo, true, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    // intervals 1 .. n-NA-1 each move a tile (i + NA < n); the last NA do not
    int i = 1;
    for (const int i_a = min(n - NA, i_mask); i < i_a; ++i) {
      interval_start(i);
      pv_qk_dma(i, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      softmax(j_lo + i, false, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; i < n - NA; ++i) {
      interval_start(i);
      pv_qk_dma(i, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      softmax(j_lo + i, false, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; i < n; ++i) {
      interval_start(i);
      pv_qk_dma(i, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      softmax(j_lo + i, false, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    interval_start(n);
    pv(n - 1);
  } else {
    interval_start(0);
    qk(0);
    __builtin_amdgcn_sched_barrier(0);
    int i = 1;
    for (const int i_t = min(n, i_mask + 1); i < i_t; ++i) {   // softmax of tile i - 1 < j_mask
      interval_start(i);
      softmax(j_lo + i - 1, i == 1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      pv_qk(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; i < n; ++i) {
      interval_start(i);
      softmax(j_lo + i - 1, i == 1, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      pv_qk(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    interval_start(n);
    softmax(j_lo + n - 1, n == 1, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    pv(n - 1);
  }

  // ---- epilogue ------------------------------------------------------------------
  // Lane (lg, lc) holds values 16 db + 4 lg .. +3 of query row t[qb].
  float l_tot[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) l_tot[qb] = quad_sum(l_run[qb]);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!row_valid[qb]) continue;
    const int64_t row = t[qb] * a.heads + h;
    if (S == 1) {
      const float inv = 1.f / l_tot[qb];
      EO* orow = obase + row * (int64_t)DV + 4 * lg;
#pragma unroll
      for (int b = 0; b < C::NDB; ++b) {
        const float v0 = o[b][qb][0] * inv, v1 = o[b][qb][1] * inv;
        const float v2 = o[b][qb][2] * inv, v3 = o[b][qb][3] * inv;
        if constexpr (sizeof(EO) == 2) *(u32x2_t*)(orow + 16 * b) = u32x2_t{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        else *(f32x4_t*)(orow + 16 * b) = f32x4_t{v0, v1, v2, v3};
      }
      if (lse && lg == 0) lse[(int64_t)h * a.lse_stride + t[qb]] = (m_run[qb] * cs + __log2f(l_tot[qb])) * kLn2;
    } else {
      const int64_t R = c * a.heads;
      float* wo = a.ws_o + ((int64_t)split * R + row) * DV + 4 * lg;
#pragma unroll
      for (int b = 0; b < C::NDB; ++b) *(f32x4_t*)(wo + 16 * b) = o[b][qb];
      if (lg == 0)
        *(float2*)(a.ws_ml + ((int64_t)split * R + row) * 2) =
            make_float2(m_run[qb] == -INFINITY ? -INFINITY : m_run[qb] * cs, l_tot[qb]);
    }
  }
}

// ---- host launchers -----------------------------------------------------------------

bool prefill_paged_supported(int D, int DV) {
  return (D == 64 && DV == 64) || (D == 128 && DV == 128) || (D == 192 && DV == 128);
}

int prefill_paged_rows(int, int) { return 256; }

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

bool prefill_contig_supported(DType in, int D, int DV) { return in == DType::BF16 && D == 128 && DV == 128; }

hipError_t launch_prefill_contig(DType out, const PrefillArgs& a, int grid, hipStream_t stream) {
  if (out == DType::BF16)
    hipLaunchKernelGGL((prefill_paged_kernel<uint16_t, 128, 128, false, true>), dim3(grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_paged_kernel<float, 128, 128, false, true>), dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_paged_varlen(DType out, int D, int DV, const PrefillArgs& a, int grid, hipStream_t stream) {
  if (out == DType::BF16) return launch_paged_dims<uint16_t, true>(D, DV, a, grid, stream);
  return launch_paged_dims<float, true>(D, DV, a, grid, stream);
}

}  // namespace chunkattn
