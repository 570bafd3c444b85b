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
// Kernel shape (two waves per (work unit, 16-head block)):
//  * 32 keys per step, double-buffered in LDS by direct-to-LDS loads.  Wave w
//    owns latent values 256w.. and rotary values 32w..: it loads only those
//    runs, so neither wave waits for the other's loads.
//  * Partial S^T = K Q^T over the wave's 288 values on
//    v_mfma_f32_16x16x32_bf16: two 16-key row blocks x 9 feature steps.  A lane
//    holds keys 4g..4g+3 and 16+4g..16+4g+3 (g = lane/16) of head lane%16 —
//    exactly the B operand P^T of the PV product over those 8 keys, so P needs
//    no shuffle.  The waves swap their 2 KiB of partial scores through LDS and
//    both run the same online softmax.
//  * O^T = V^T P^T on the same MFMA, 16 blocks of 16 latent values per wave.
//    The V^T operand (8 keys of one value per lane) comes from the token-major
//    tile through transposing LDS reads: two ds_read_b64_tr_b16 (bf16) or one
//    ds_read_b64_tr_b8 (fp8 codes).  LDS reads run several MFMAs ahead.
//  * fp8: codes are widened exactly (unit scale) by v_cvt_scalef32_pk_bf16_fp8,
//    one instruction per pair.  Scores are accumulated per 128-value group and
//    each key's fp32 group scale is applied to its partial score; for PV each
//    key's scale is folded into P, group by group.
//  * Work plan: the 32-key steps of all sequences, end to end, are cut into
//    equal units (mla_plan_kernel finds where each starts), so every
//    workgroup streams the same number of bytes whatever the length mix.
//    Each segment (a unit's piece of one sequence) leaves an unnormalised
//    partial (O, max, sum); mla_merge_kernel combines them in unit order.
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
  // one wait state between the M0 write and the load that reads it (a GFX9 hazard)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_wave_base), "v"(g) : "memory", "m0");
}

// N loads of 16 bytes per lane, 1 KiB apart: global uniform base + this lane's
// 32-bit offset + 1024 i (the instruction offset, which moves the LDS address
// alike) into LDS at m0 + 1024 i + 16 * lane.  One m0 write, one wait state.
template <int N>
__device__ __forceinline__ void dma16_run(const void* base, uint32_t lane_off, uint32_t lds_wave_base) {
  static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 KiB (the offset field reaches 4095)");
  if constexpr (N == 1)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_wave_base), "v"(lane_off),
                 "s"(base)
                 : "memory", "m0");
  else if constexpr (N == 2)
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\tglobal_load_lds_dwordx4 %1, %2 offset:1024" ::"s"(
            lds_wave_base),
        "v"(lane_off), "s"(base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\tglobal_load_lds_dwordx4 %1, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:2048\n\tglobal_load_lds_dwordx4 %1, %2 offset:3072" ::"s"(lds_wave_base),
        "v"(lane_off), "s"(base)
        : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` (<= K) steps of L loads each are still in flight.
template <int K, int L>
__device__ __forceinline__ void wait_steps(int ahead) {
  static_assert(K * L <= 63, "vmcnt holds 6 bits");
  if constexpr (K == 0) {
    wait_vmem<0>();
  } else {
    if (ahead >= K) wait_vmem<K * L>();
    else wait_steps<K - 1, L>(ahead);
  }
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

// Waits for this wave's LDS operations and meets the other wave; loads in
// flight keep flying.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Max / sum of x over lanes l and l^16 (then l^32) on the vector ALU:
// v_permlane16_swap / v_permlane32_swap hand each lane its partner's value.
// Both lanes of a pair add in the same order, so they hold identical sums.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool FP8>
struct MlaCfg {
  // LDS bytes of one 32-key step.  bf16: [72 runs][32 tokens][16 B].  fp8: codes
  // [32 runs][32][16 B]; per wave a copy of the 32 keys' scales [32][16 B] plus the
  // 512 B the upper half-wave of that load writes; rotary [8 runs][32][16 B].
  static constexpr int kCodes = 0;
  static constexpr int kScales = 32 * 32 * 16;
  static constexpr int kRope = FP8 ? kScales + 2 * 1024 : 64 * 32 * 16;
  static constexpr int kStage = FP8 ? kRope + 8 * 32 * 16 : 72 * 32 * 16;
  // ring depth: kStages - 1 steps in flight per wave while one is consumed.
  // fp8 steps are small, so three of them (two workgroups per CU) keep more
  // bytes in flight than two (three workgroups per CU) would.
  static constexpr int kStages = FP8 ? kMlaStagesFp8 : kMlaStagesBf16;
  static constexpr int kLoads = FP8 ? 8 + 1 + 2 : 16 + 2;     // direct loads per wave per step
  // partial scores: [kXSlots][2 waves][64 lanes][8 fp32].  With two slots (by
  // step parity) one barrier per step suffices.  bf16 keeps one slot and a
  // second barrier: its loads bound it, and two slots measured no faster.
  static constexpr int kXSlots = FP8 ? 2 : 1;
  static constexpr int kXchg = kStages * kStage;
  static constexpr int kLds = kXchg + kXSlots * 2 * 64 * 32;
  static_assert((FP8 ? kMlaWgPerCuFp8 : kMlaWgPerCuBf16) * kLds <= 160 * 1024,
                "the plan's workgroups per CU fit the CU's LDS");
  static constexpr int64_t kBlock = FP8 ? kMlaFp8Block : kMlaBf16Block;
};

}  // namespace

// Two waves per (work unit, 16-head block).  Wave w owns latent
// values 256w .. 256w+255 and rotary values 32w .. 32w+31: it loads only those
// runs, forms the partial scores over them, and after the two waves swap
// partials through LDS (both then hold identical scores and run the same
// softmax) it accumulates its half of the output.
template <bool FP8>
__global__ __launch_bounds__(128) void mla_decode_kernel(const MlaArgs a) {
  using C = MlaCfg<FP8>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kLds];
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup -> (unit, head block).  Workgroups go round-robin to the 8 XCDs;
  // with a unit count divisible by 8 the head blocks of one unit land on one
  // XCD back to back and share its L2 copy of the unit's cache blocks.
  const int nhb = a.heads / 16;
  int unit, hb;
  if ((a.units & 7) == 0) {
    const int id = blockIdx.x;
    unit = (id / (8 * nhb)) * 8 + (id & 7);
    hb = (id >> 3) % nhb;
  } else {
    unit = blockIdx.x % a.units;
    hb = blockIdx.x / a.units;
  }
  const int head = hb * 16 + c;
  const float cs = a.scale_log2;
  const int64_t total = a.seq_steps[a.num_seqs];
  const int64_t u_hi = (int64_t)(unit + 1) * total / a.units;
  int64_t x = (int64_t)unit * total / a.units;
  int s = a.unit_seq[unit];
  const uint32_t smem_base = lds_addr(smem);
  // fp8: this lane's offsets inside a half-block for the wave's code, scale and rotary loads
  const uint32_t off_codes = lane * 16 + 8 * w * 1024, off_codes4 = off_codes + 4096;
  const uint32_t off_scales = lane * 16 + (uint32_t)kMlaFp8HalfScales;
  const uint32_t off_rope = lane * 16 + (uint32_t)kMlaFp8HalfRope + 2 * w * 1024;

  // one segment per sequence the unit touches
  for (; x < u_hi; ++s) {
    const int64_t p0 = a.seq_steps[s];
    const int64_t seg_end = min(u_hi, a.seq_steps[s + 1]);
    const int kv_len = a.kv_lens[s];
    const int key_lo = (int)(x - p0) * kMlaStepKeys;
    const int key_hi = min(kv_len, (int)(seg_end - p0) * kMlaStepKeys);
    x = seg_end;
    const int n_steps = (key_hi - key_lo + kMlaStepKeys - 1) / kMlaStepKeys;

    // Q^T as B operands of this wave's 9 feature steps (32 values each): latent
    // steps 8w .. 8w+7, then rotary step 16 + w; lane group g holds values 8g ..
    u32x4_t qb[9];
    {
      const uint16_t* qrow = a.q + ((int64_t)s * a.heads + head) * kMlaRecord + 8 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[j] = *(const u32x4_t*)(qrow + 32 * (8 * w + j));
      qb[8] = *(const u32x4_t*)(qrow + 32 * (16 + w));
    }
    // The segment's block ids, lane l of register r holding the (64r + l + 1)-th
    // (a segment spans at most 64 * kMlaBtRegs blocks): the step loop then makes
    // no load the compiler tracks, so none of its waits can stall on the direct
    // loads in flight.
    const int blk0 = key_lo >> 6;
    const int n_blk = ((key_hi - 1) >> 6) - blk0 + 1;
    int bt_lane[kMlaBtRegs];
#pragma unroll
    for (int r = 0; r < kMlaBtRegs; ++r)
      bt_lane[r] = 64 * r + lane < n_blk ? a.block_tables[(int64_t)s * a.max_blocks + blk0 + 64 * r + lane] : 0;
#pragma unroll
    for (int j = 0; j < 9; ++j) asm volatile("" ::"v"(qb[j]));
#pragma unroll
    for (int r = 0; r < kMlaBtRegs; ++r) asm volatile("" ::"v"(bt_lane[r]));
    // id of the segment's idx-th block (idx wave-uniform)
    auto block_of = [&](int idx) -> int {
      int id = __builtin_amdgcn_readlane(bt_lane[0], idx & 63);
#pragma unroll
      for (int r = 1; r < kMlaBtRegs; ++r)
        if ((idx >> 6) == r) id = __builtin_amdgcn_readlane(bt_lane[r], idx & 63);
      return id;
    };

    // step t covers keys key_lo + 32t .. +31: half (key / 32) & 1 of block key / 64.
    // Load n moves runs 2n and 2n+1 (32 tokens each); the wave issues only its own.
    auto issue = [&](int t, int st) {
      const int key0 = key_lo + kMlaStepKeys * t;
      const int blk = clamp_block(block_of((key0 >> 6) - blk0), a.num_blocks);
      const uint32_t lds = smem_base + st * C::kStage;
      if constexpr (FP8) {
        // The step is one contiguous half-block, addressed from a scalar base: the wave's 8 KiB of code
        // runs, then the 32 keys' scales (the upper half-wave brings the first 512 B of the rotary runs
        // into the unused half of the slot), then its 2 KiB of rotary runs, 1 KiB per load.
        const unsigned char* h = a.pool + (int64_t)blk * C::kBlock + ((key0 >> 5) & 1) * kMlaFp8Half;
        dma16_run<4>(h, off_codes, lds + C::kCodes + 8 * w * 1024);
        dma16_run<4>(h, off_codes4, lds + C::kCodes + 8 * w * 1024 + 4096);
        dma16_run<1>(h, off_scales, lds + C::kScales + w * 1024);
        dma16_run<2>(h, off_rope, lds + C::kRope + 2 * w * 1024);
      } else {
        const unsigned char* b = a.pool + (int64_t)blk * C::kBlock + ((key0 >> 5) & 1) * 32 * 16 +
                                 (lane >> 5) * 1024 + (lane & 31) * 16;
#pragma unroll
        for (int n = 16 * w; n < 16 * w + 16; ++n) dma16(b + 2 * n * 1024, lds + n * 1024);
#pragma unroll
        for (int n = 32 + 2 * w; n < 34 + 2 * w; ++n) dma16(b + 2 * n * 1024, lds + n * 1024);
      }
    };

    f32x4_t o[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // this lane's keys as a score row: kappa(g, j) = 4g + j (j < 4), 16 + 4g + (j - 4)
    auto kappa = [&](int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); };

#pragma unroll
    for (int i = 0; i < C::kStages - 1; ++i)
      if (i < n_steps) issue(i, i);
    int st = 0;                                        // stage of step t: t % kStages
    for (int t = 0; t < n_steps; ++t) {
      // refill the stage step t-1 used, then wait for step t's loads only
      const int t_next = t + C::kStages - 1;
      if (t_next < n_steps) issue(t_next, st == 0 ? C::kStages - 1 : st - 1);
      const int ahead = min(C::kStages - 1, n_steps - 1 - t);   // steps issued after t
      wait_steps<C::kStages - 1, C::kLoads>(ahead);
      unsigned char* stage = smem + st * C::kStage;
      const int key0 = key_lo + kMlaStepKeys * t;
      const int valid = key_hi - key0;                 // keys of this step that count (1..32)
      if (valid < kMlaStepKeys) {
        // Keys past the sequence's end may hold anything: give this wave's latent
        // runs zeros (and its scales ones) there, so 0 * junk cannot reach O.
        if constexpr (FP8) {
          for (int e = lane; e < 16 * 32; e += 64) {
            const int run = 16 * w + (e >> 5), tok = e & 31;
            if (tok >= valid) *(u32x4_t*)(stage + C::kCodes + run * 512 + tok * 16) = u32x4_t{0u, 0u, 0u, 0u};
          }
          if (lane < 32 && lane >= valid)
            *(f32x4_t*)(stage + C::kScales + w * 1024 + lane * 16) = f32x4_t{1.f, 1.f, 1.f, 1.f};
        } else {
          for (int e = lane; e < 32 * 32; e += 64) {
            const int run = 32 * w + (e >> 5), tok = e & 31;
            if (tok >= valid) *(u32x4_t*)(stage + run * 512 + tok * 16) = u32x4_t{0u, 0u, 0u, 0u};
          }
        }
      }

      // ---- partial S^T = K Q^T over this wave's values; row blocks keys 0-15 and 16-31 ----
      // fp8: scale of key kappa(j) for latent group 2w + q
      float vs[8][2];
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2_t sc = *(const u32x2_t*)(stage + C::kScales + w * 1024 + kappa(j) * 16 + 8 * w);
          vs[j][0] = __uint_as_float(sc[0]);
          vs[j][1] = __uint_as_float(sc[1]);
        }
      }
      // op k: k = 0, 1 rotary (row block k); k >= 2 latent step (k - 2) / 2, row block k & 1
      const unsigned char* kr = stage + C::kRope + (4 * w + g) * 512 + c * 16;
      const unsigned char* kl = FP8 ? stage + C::kCodes + (16 * w + (g >> 1)) * 512 + (g & 1) * 8 + c * 16
                                    : stage + (32 * w + g) * 512 + c * 16;
      constexpr int kQ = 18, kAq = 8;
      auto qk_read = [&](int k) -> u32x4_t {
        if (k < 2) return *(const u32x4_t*)(kr + k * 256);
        const int j = (k - 2) >> 1, row = k & 1;
        if constexpr (FP8) {
          const u32x2_t v = *(const u32x2_t*)(kl + j * 1024 + row * 256);
          return u32x4_t{v[0], v[1], 0u, 0u};
        } else {
          return *(const u32x4_t*)(kl + j * 2048 + row * 256);
        }
      };
      u32x4_t rd[kQ];
#pragma unroll
      for (int k = 0; k < kAq; ++k) rd[k] = qk_read(k);
      f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      // fp8: per 128-value group q and row block, the partial scores of unit-scale codes; each operand is
      // widened one MFMA ahead into the other of two register sets, so the conversions run beside the
      // previous MFMA
      f32x4_t tq[2][2];
      u32x4_t kvw[2];
      if constexpr (FP8) tq[0][0] = tq[0][1] = tq[1][0] = tq[1][1] = s0;
#pragma unroll
      for (int k = 0; k < kQ; ++k) {
        const int row = k & 1;
        if constexpr (FP8)
          if (k + 1 >= 2 && k + 1 < kQ) kvw[(k + 1) & 1] = widen8(rd[k + 1][0], rd[k + 1][1], 1.0f);
        if (k < 2) {
          if (row) s1 = mfma16(rd[k], qb[8], s1);
          else s0 = mfma16(rd[k], qb[8], s0);
        } else {
          const int j = (k - 2) >> 1;
          if constexpr (FP8) tq[j >> 2][row] = mfma16(kvw[k & 1], qb[j], tq[j >> 2][row]);
          else if (row) s1 = mfma16(rd[k], qb[j], s1);
          else s0 = mfma16(rd[k], qb[j], s0);
        }
        if (k + kAq < kQ) rd[k + kAq] = qk_read(k + kAq);
        __builtin_amdgcn_sched_barrier(0);            // keep the reads kAq operations ahead
      }
      if constexpr (FP8) {
        // each group's partial gets its keys' scales in fp32, group 0 first
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s0[r] = __builtin_fmaf(tq[q][0][r], vs[r][q], s0[r]);
            s1[r] = __builtin_fmaf(tq[q][1][r], vs[4 + r][q], s1[r]);
          }
      }

      // ---- swap partial scores with the other wave (same lane = same keys and head) ----
      const int xs = C::kXSlots == 2 ? (t & 1) * 4096 : 0;
      float* x_own = (float*)(smem + C::kXchg + xs + w * 2048 + lane * 32);
      const float* x_other = (const float*)(smem + C::kXchg + xs + (1 - w) * 2048 + lane * 32);
      // one slot: the other wave must have read the previous partials
      if (C::kXSlots == 1) lds_barrier();
      *(f32x4_t*)x_own = s0;
      *(f32x4_t*)(x_own + 4) = s1;
      lds_barrier();
      s0 += *(const f32x4_t*)x_other;                  // fp32 addition commutes: both waves get the same sums
      s1 += *(const f32x4_t*)(x_other + 4);

      // ---- online softmax over this step's keys (head c; keys kappa(0..7)) ----
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= valid) s0[r] = -INFINITY;
        if (16 + 4 * g + r >= valid) s1[r] = -INFINITY;
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      mx = xor32_max(xor16_max(mx));
      const bool grow = mx * cs > m_run * cs + kLazyRescale;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? fast_exp2((m_run - m_new) * cs) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < 16; ++b) o[b] *= alpha;
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

      // ---- O^T += V^T P^T over the 8 keys this lane's P covers; this wave's 16 value blocks ----
      constexpr int kP = 16, kAp = 6;
      if constexpr (FP8) {
        // transposing read: this lane (as a source) points at key kappa(c / 2), codes 8(c % 2) ..
        const int src_r = c >> 1;
        const int src_key = src_r < 4 ? 4 * g + src_r : 16 + 4 * g + (src_r - 4);
        const unsigned char* vb = stage + C::kCodes + (16 * w) * 512 + src_key * 16 + (c & 1) * 8;
        auto pv_read = [&](int bb) -> v2i32_t {
          return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(vb + bb * 512));
        };
        v2i32_t rv[kP];
#pragma unroll
        for (int k = 0; k < kAp; ++k) rv[k] = pv_read(k);
        u32x4_t pb[2];                                 // P with each key's group scale folded in
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) pb[q][i] = pack_bf16(p[2 * i] * vs[2 * i][q], p[2 * i + 1] * vs[2 * i + 1][q]);
        // V^T operands widened one MFMA ahead into alternating register sets
        u32x4_t va[2];
        va[0] = widen8((uint32_t)rv[0][0], (uint32_t)rv[0][1], 1.0f);
#pragma unroll
        for (int bb = 0; bb < kP; ++bb) {
          if (bb + 1 < kP) va[(bb + 1) & 1] = widen8((uint32_t)rv[bb + 1][0], (uint32_t)rv[bb + 1][1], 1.0f);
          o[bb] = mfma16(va[bb & 1], pb[bb >> 3], o[bb]);
          if (bb + kAp < kP) rv[bb + kAp] = pv_read(bb + kAp);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // two transposing reads: keys 4g + (c/4) and 16 + 4g + (c/4); values 4(c%4) ..
        const unsigned char* vb = stage + (32 * w) * 512 + (4 * g + (c >> 2)) * 16 + (c & 1) * 8 + ((c & 3) >> 1) * 512;
        auto pv_read = [&](int bb) -> u32x4_t {
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + bb * 1024));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + bb * 1024 + 256));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
          return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        };
        u32x4_t rv[kP];
#pragma unroll
        for (int k = 0; k < kAp; ++k) rv[k] = pv_read(k);
        u32x4_t pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
#pragma unroll
        for (int bb = 0; bb < kP; ++bb) {
          o[bb] = mfma16(rv[bb], pb, o[bb]);
          if (bb + kAp < kP) rv[bb + kAp] = pv_read(bb + kAp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      st = st + 1 == C::kStages ? 0 : st + 1;
    }

    // ---- partial of this segment: wave w writes latent values 256w .. 256w+255 ----
    const float l_tot = xor32_sum(xor16_sum(l_run));
    const int64_t slot = (int64_t)head * a.slots + s + unit;
    float* wo = a.ws_o + slot * kMlaLatent + 256 * w;
#pragma unroll
    for (int b = 0; b < 16; ++b) *(f32x4_t*)(wo + 16 * b + 4 * g) = o[b];
    if (w == 0 && g == 0)
      *(float2*)(a.ws_ml + slot * 2) = make_float2(m_run == -INFINITY ? -INFINITY : m_run * cs, l_tot);
  }
}

// One workgroup of 1024 threads: steps per sequence (ceil(kv / 32)), their
// exclusive prefix sums, and the sequence where each unit's step range starts.
__global__ __launch_bounds__(1024) void mla_plan_kernel(const MlaArgs a) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int per = (a.num_seqs + 1023) / 1024;
  const int s0 = min(a.num_seqs, t * per), s1 = min(a.num_seqs, s0 + per);
  int64_t sum = 0;
  for (int s = s0; s < s1; ++s) sum += (a.kv_lens[s] + kMlaStepKeys - 1) / kMlaStepKeys;
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {     // inclusive scan
    const int64_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const int64_t total = part[1023];
  int64_t run = t > 0 ? part[t - 1] : 0;
  for (int s = s0; s < s1; ++s) {
    a.seq_steps[s] = run;
    const int64_t next = run + (a.kv_lens[s] + kMlaStepKeys - 1) / kMlaStepKeys;
    // units whose first step (unit * total / units) lies in [run, next)
    const int64_t g_lo = (run * a.units + total - 1) / total, g_hi = (next * a.units + total - 1) / total;
    for (int64_t u = g_lo; u < g_hi; ++u) a.unit_seq[u] = s;
    run = next;
  }
  if (t == 0) a.seq_steps[a.num_seqs] = total;
}

// One workgroup per (sequence, head): combine the sequence's segment partials
// in unit order, normalise, store bf16 (RNE) or fp32 and the LSE.
__global__ __launch_bounds__(128) void mla_merge_kernel(const MlaArgs a) {
  const int s = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
  const int64_t total = a.seq_steps[a.num_seqs];
  const int64_t p0 = a.seq_steps[s], p1 = a.seq_steps[s + 1];
  // unit holding step x: ((x + 1) * units - 1) / total
  const int u0 = (int)(((p0 + 1) * a.units - 1) / total), u1 = (int)((p1 * a.units - 1) / total);
  const int64_t slot0 = (int64_t)h * a.slots + s + u0;
  const int n = u1 - u0 + 1;
  float M, L;
  merge_weights(a.ws_ml + slot0 * 2, n, 1, M, L);
  const int t = threadIdx.x;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n; ++i) {
    const float m = a.ws_ml[(slot0 + i) * 2];
    if (m == -INFINITY) continue;
    acc += *(const f32x4_t*)(a.ws_o + (slot0 + i) * kMlaLatent + 4 * t) * fast_exp2(m - M);
  }
  acc *= 1.f / L;
  const int64_t o_off = ((int64_t)s * a.heads + h) * kMlaLatent + 4 * t;
  if (a.out_f32) *(f32x4_t*)((float*)a.out + o_off) = acc;
  else *(u32x2_t*)((uint16_t*)a.out + o_off) = u32x2_t{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
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
    unsigned char* h = b + (tok >> 5) * kMlaFp8Half;                // this token's half of the block
    const int u = tok & 31;
    *(u32x2_t*)(h + ((lane >> 1) * 32 + u) * 16 + (lane & 1) * 8) = u32x2_t{w[0], w[1]};
    if ((lane & 15) == 0) *(float*)(h + kMlaFp8HalfScales + u * 16 + (lane >> 4) * 4) = scale;
    if (lane < 8)
      *(u32x4_t*)(h + kMlaFp8HalfRope + (lane * 32 + u) * 16) = *(const u32x4_t*)(a.rope + i * kMlaRope + 8 * lane);
  }
}

hipError_t launch_mla_decode(bool fp8, const MlaArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.units * (a.heads / 16));
  if (fp8) hipLaunchKernelGGL(mla_decode_kernel<true>, grid, dim3(128), 0, stream, a);
  else hipLaunchKernelGGL(mla_decode_kernel<false>, grid, dim3(128), 0, stream, a);
  e = hipGetLastError();
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
