// MLA latent (absorbed) chunked prefill over a paged latent cache, gfx950.
//
// "02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16" deployment notes §1, §4:
// an MLA layer caches one latent record per token shared by every query head
// (512 latent + 64 rotary values, 1152 B in bf16).  A prompt chunk of c tokens
// at offset past_len (VPP technical review, English edition, §2.3) attends,
// head by head, causally to the records of every earlier position and of
// itself (§2.2, Eq. (1) and its causal rule): keys are the 576-value records,
// values their 512-value latents, and the output stays in latent space.  It is
// the decode path's absorbed attention with many query tokens instead of one.
//
// Kernel shape (one workgroup = 4 waves, one wave per SIMD):
//  * A wave holds 32 query rows: two 16-row blocks, each one token's 16
//    consecutive heads, so a block shares one causal limit.  Per 64-key tile
//    (one cache block), S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 over
//    4 key blocks x 18 feature steps, and every 1 KiB K operand read from LDS
//    feeds both row blocks.  The queries (144 VGPRs) stay in registers and the
//    512-wide output accumulators (256 registers) in AGPRs.
//  * With d_qk = 576 and d_v = 512 a row-key pair costs 2176 matrix flops
//    against the same handful of vector ops as a d = 128 head, so the
//    softmax is a small share of a tile (~1/5) and the wave runs it between
//    its own QK and PV phases; no second wave per SIMD (there would be no
//    registers for it).
//  * Tiles move into a two-stage LDS ring (144 KiB) by direct-to-LDS loads,
//    issued a whole tile ahead.  The V^T operand (8 keys of one latent value
//    per lane) comes from the same token-major tile through two transposing
//    reads (ds_read_b64_tr_b16), on exactly the keys a lane's QK accumulators
//    hold, so P needs no shuffle.
//  * Softmax: exps with the running offset, row sums, and the exact row
//    maxima (over the 4 lanes of a row) only on the first tile or when a
//    lane's row sum shows that a logit may have passed the lazy threshold.
//  * Latent values of keys past the sequence end are zeroed in LDS, logits
//    past a row's position are masked with a select: NaN in unused pool slots
//    never reaches an output.
//  * fp8 latent cache (the deployment notes' 656 B record: e4m3 codes, one
//    fp32 scale per 128 values): a memory-bound pass first widens the chunk's
//    visible prefix to bf16 blocks in logical order (code x scale, one
//    rounding), then this same kernel runs on them.  That pass moves about
//    1.8 KB per visible token, well under 1% of a chunk's matrix time, where
//    widening inside the kernel would put ~256 vector ops per lane and tile on
//    the only wave of each SIMD.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace chunkattn {

namespace {

constexpr int kRuns = 72;                       // runs of 8 values: 64 latent, 8 rotary
constexpr int kTileBytes = kRuns * 64 * 16;     // one 64-token bf16 cache block
constexpr int kThreads = 256;
constexpr int kLoads = kTileBytes / (kThreads * 16);   // direct loads per thread per tile
constexpr int kQS = kMlaRecord / 32;            // 32-value feature steps of QK
constexpr int kNDB = kMlaLatent / 16;           // 16-value output blocks
// A lane's 16 exps of one row sum to at most this while no logit passes the
// row's offset by more than kLazyRescale (log2 units).
constexpr float kRowSumCap = 16.f * (1 << (int)kLazyRescale);
static_assert(kTileBytes % (kThreads * 16) == 0, "tile split");

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// S^T += K Q^T with the accumulator pinned to VGPRs: the 32 x 512 output
// tile takes all 256 AGPRs, and the compiler would otherwise put S^T there too
// and spill.  The compiler cannot see hazards through the asm; the caller waits
// 18+ states before vector code reads S^T.  The first product's result is
// early-clobber: it must not take the registers of an operand that dies there.
__device__ __forceinline__ void mfma16_vgpr(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_vgpr_first(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from global memory (uniform base + this lane's offset)
// straight into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* base, uint32_t lane_off, uint32_t lds_wave_base) {
  // one wait state between the M0 write and the load that reads it (a GFX9 hazard)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_wave_base), "v"(lane_off), "s"(base)
               : "memory", "m0");
}
// The same load split in two for the QK phase: set_m0 writes the LDS
// destination, and load_at_m0, issued two K operands (four MFMAs) later,
// reads it.  The MFMAs between them are the wait state the M0 hazard needs,
// so neither carries an s_nop.  Sound only because nothing the compiler emits
// in this kernel writes m0: every m0 write is one of these asm statements.
__device__ __forceinline__ void set_m0(uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0" ::"s"(lds_wave_base) : "m0");
}
__device__ __forceinline__ void load_at_m0(const void* base, uint32_t lane_off) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base) : "memory");
}

__device__ __forceinline__ void wait_all_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Row maxima of both row blocks over the four lanes l, l^16, l^32, l^48 that
// hold a row: permlane16_swap(x0, x1) leaves lane groups 0 / 2 with block 0
// over groups {0,1} / {2,3} and groups 1 / 3 with block 1, permlane32_swap
// folds the halves, a last permlane16_swap gives every lane both totals.
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

}  // namespace

template <typename EO>
__global__ __launch_bounds__(256, 1) void mla_prefill_kernel(const MlaPrefillArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTileBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h16 = a.heads / 16;
  const int64_t c = a.chunk_len, P = a.past_len, kv_len = P + c;
  const int64_t n_rb = c * h16;                          // row blocks: (token, 16-head block)
  const int64_t wg = (int64_t)gridDim.x - 1 - blockIdx.x;   // latest tokens (most keys) first

  // This wave's two row blocks; lane column lc is a head of the block.
  int64_t tok[2], pos[2];
  int head[2];
  bool row_valid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t rb = wg * 8 + 2 * wave + qb;
    row_valid[qb] = rb < n_rb;
    const int64_t rbc = row_valid[qb] ? rb : n_rb - 1;
    tok[qb] = rbc / h16;
    head[qb] = (int)(rbc % h16) * 16 + lc;
    pos[qb] = P + tok[qb];
  }
  const int64_t last_tok = min(wg * 8 + 7, n_rb - 1) / h16;
  const int n_tiles = (int)((P + last_tok) / kBlock) + 1;
  const int wave_first_pos = __builtin_amdgcn_readfirstlane((int)pos[0]);
  const int kv_len32 = (int)kv_len;
  const float cs = a.scale_log2;

  // Query rows as B operands: features 32 i + 8 lg .. +7 of (tok, head).
  // Loaded again after a rescale of O: the rescale needs the registers, and
  // the opaque pointer keeps the compiler from reusing the first load.
  u32x4_t qreg[2][kQS];
  const uint16_t* qrow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) qrow[qb] = a.q + (tok[qb] * a.heads + head[qb]) * (int64_t)kMlaRecord + 8 * lg;
  auto load_q = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const uint16_t* p = qrow[qb];
      asm volatile("" : "+v"(p));
#pragma unroll
      for (int i = 0; i < kQS; ++i) qreg[qb][i] = *(const u32x4_t*)(p + 32 * i);
    }
  };
  load_q();

  // ---- tile transfer: block ids through the scalar unit, records straight into LDS ----
  const __attribute__((address_space(4))) int32_t* bt4 = (const __attribute__((address_space(4))) int32_t*)a.block_table;
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t lane_off = (uint32_t)(wave * 64 + lane) * 16;
  // The next tile's loads go out one after every eighth QK MFMA (18 of them over
  // the 144): issued as a burst they would hold the wave at issue while the
  // direct-to-LDS path drains them.  Only the first tile, with no matrix phase
  // before it, goes as a burst.
  const unsigned char* pend_b = a.pool;
  uint32_t pend_lds = 0;
  auto prep = [&](int j, int st) {
    const int phys = a.block_table ? clamp_block(bt4[j], a.num_blocks) : j;   // null table: logical order
    pend_b = a.pool + (int64_t)phys * kTileBytes;
    pend_lds = smem_base + st * kTileBytes + wave * 1024;
  };
  auto dma_one = [&](int n) {
    dma16(pend_b + n * kThreads * 16, lane_off, __builtin_amdgcn_readfirstlane(pend_lds + n * kThreads * 16));
  };
  auto dma_m0 = [&](int n) { set_m0(__builtin_amdgcn_readfirstlane(pend_lds + n * kThreads * 16)); };
  auto dma_load = [&](int n) { load_at_m0(pend_b + n * kThreads * 16, lane_off); };

  f32x4_t o[kNDB][2];
#pragma unroll
  for (int b = 0; b < kNDB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  float neg_mb[2] = {0.f, 0.f}, thr[2] = {-INFINITY, -INFINITY};
  const float lazy_unscaled = kLazyRescale / cs;

  // K operand (key block kb, feature step i): run 4 i + lg, token 16 kb + lc.
  const int k_lane = (lg * 64 + lc) * 16;
  // V^T operand (32-key step ks, value block bb): two transposing reads; lane lc of
  // group lg points at key 4 lg + lc / 4 (and 16 later), values 4 (lc % 4) .. +3 of
  // the block's 16, i.e. run 2 bb + (lc % 4) / 2, half lc % 2.
  const int v_lane = (4 * lg + (lc >> 2)) * 16 + (lc & 1) * 8 + ((lc & 3) >> 1) * 1024;

  auto tile = [&](int j, int st, bool first, auto with_dma_tag) {
    constexpr bool with_dma = decltype(with_dma_tag)::value;
    const unsigned char* stage = smem + st * kTileBytes;
    // ---- S^T = K Q^T ----
    f32x4_t s[4][2];
    {
      const unsigned char* kbase = stage + k_lane;
      constexpr int kOps = 4 * kQS, kAhead = 4;
      auto k_ptr = [&](int k) { return (const u32x4_t*)(kbase + (256 * (k >> 2) + 16 * (k & 3)) * 16); };
      u32x4_t rd[kOps];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) rd[k] = *k_ptr(k);
#pragma unroll
      for (int k = 0; k < kOps; ++k) {            // op k: feature step k / 4, key block k % 4
        if (k < 4) {
          mfma16_vgpr_first(s[k][0], rd[k], qreg[0][0]);
          mfma16_vgpr_first(s[k][1], rd[k], qreg[1][0]);
        } else {
          mfma16_vgpr(s[k & 3][0], rd[k], qreg[0][k >> 2]);
          mfma16_vgpr(s[k & 3][1], rd[k], qreg[1][k >> 2]);
        }
        if (k + kAhead < kOps) rd[k + kAhead] = *k_ptr(k + kAhead);
        if constexpr (with_dma) {
          if ((k & 3) == 1) {
            __builtin_amdgcn_sched_barrier(0);
            dma_m0(k >> 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if ((k & 3) == 3) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (with_dma) dma_load(k >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      static_assert(kOps / 4 == kLoads, "one load per four K operands");
    }
    // the asm MFMAs wrote S^T: 18+ wait states before vector code reads it
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]), "+v"(s[2][0]), "+v"(s[2][1]),
                   "+v"(s[3][0]), "+v"(s[3][1]));
    // ---- online softmax: register (kb, r) of lane group lg holds key 16 kb + 4 lg + r ----
    const int key0 = j * kBlock;
    if (key0 + kBlock - 1 > wave_first_pos) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int lim = (int)(pos[qb] - key0) - 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r > lim) s[kb][qb][r] = -INFINITY;
      }
    }
    float p[2][4][4], psum[2];
    auto exps = [&]() {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[qb][kb][r] = fast_exp2(__builtin_fmaf(s[kb][qb][r], cs, neg_mb[qb]));
    };
    auto row_sums = [&]() {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float acc = (p[qb][0][0] + p[qb][0][1]) + (p[qb][0][2] + p[qb][0][3]);
#pragma unroll
        for (int kb = 1; kb < 4; ++kb) acc += (p[qb][kb][0] + p[qb][kb][1]) + (p[qb][kb][2] + p[qb][kb][3]);
        psum[qb] = acc;
      }
    };
    exps();
    row_sums();
    if (first || (__builtin_amdgcn_ballot_w64(!(psum[0] <= kRowSumCap)) |
                  __builtin_amdgcn_ballot_w64(!(psum[1] <= kRowSumCap))) != 0) {
      float mx[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m = s[0][qb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = max_raw(m, s[i >> 2][qb][i & 3]);
        mx[qb] = m;
      }
      quad_max2(mx[0], mx[1]);
      const bool grow0 = mx[0] > thr[0], grow1 = mx[1] > thr[1];
      if ((__builtin_amdgcn_ballot_w64(grow0) | __builtin_amdgcn_ballot_w64(grow1)) != 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bool grow = qb ? grow1 : grow0;
          const float m_new = grow ? mx[qb] : m_run[qb];
          const float alpha = grow ? fast_exp2((m_run[qb] - m_new) * cs) : 1.f;
          l_run[qb] *= alpha;
#pragma unroll
          for (int b = 0; b < kNDB; ++b) {
            // through VGPRs and back, with the class fixed on both sides so that O stays in AGPRs
            f32x4_t t;
            asm volatile("" : "=v"(t) : "0"(o[b][qb]));
            t *= alpha;
            asm volatile("" : "=a"(o[b][qb]) : "0"(t));
          }
          m_run[qb] = m_new;
          if (grow) {
            neg_mb[qb] = -(m_new * cs);
            thr[qb] = m_new + lazy_unscaled;
          }
        }
        exps();
        row_sums();
      }
    }
    // P^T of each 32-key step ks: keys 32 ks + 4 lg .. +3 (block 2 ks) and 32 ks + 16 + 4 lg .. +3
    u32x4_t pkv[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      l_run[qb] += psum[qb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pkv[qb][ks] = u32x4_t{pack_bf16(p[qb][2 * ks][0], p[qb][2 * ks][1]), pack_bf16(p[qb][2 * ks][2], p[qb][2 * ks][3]),
                              pack_bf16(p[qb][2 * ks + 1][0], p[qb][2 * ks + 1][1]),
                              pack_bf16(p[qb][2 * ks + 1][2], p[qb][2 * ks + 1][3])};
    }
    // ---- O^T += V^T P^T ----
    {
      const unsigned char* vbase = stage + v_lane;
      constexpr int kOps = 2 * kNDB, kAhead = 4;
      auto v_read = [&](int k) -> u32x4_t {       // op k: 32-key step k / kNDB, value block k % kNDB
        const unsigned char* pp = vbase + (k / kNDB) * 32 * 16 + (k % kNDB) * 2048;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)pp);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pp + 256));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      };
      u32x4_t rv[kOps];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) rv[k] = v_read(k);
#pragma unroll
      for (int k = 0; k < kOps; ++k) {
        const int ks = k / kNDB, bb = k % kNDB;
        o[bb][0] = mfma16(rv[k], pkv[0][ks], o[bb][0]);
        o[bb][1] = mfma16(rv[k], pkv[1][ks], o[bb][1]);
        if (k + kAhead < kOps) rv[k + kAhead] = v_read(k + kAhead);
      }
    }
  };

  // ---- key loop: tile t in stage t % 2; tile t + 1 loads while tile t runs ----
  prep(0, 0);
#pragma unroll
  for (int n = 0; n < kLoads; ++n) dma_one(n);
  // Every tile but the last moves the next one; that is a compile-time tag of
  // the tile body, so no load point in the QK phase carries a branch.
  auto step = [&](int t, auto with_dma_tag) {
    wait_all_vmem();
    barrier();                                     // tile t landed everywhere; stage (t + 1) % 2 is free
    if constexpr (decltype(with_dma_tag)::value) prep(t + 1, (t + 1) & 1);
    const int key0 = t * kBlock;
    if (key0 + kBlock > kv_len32) {
      // keys past the sequence end: zero their latent values (0 * NaN would poison O)
      unsigned char* st = smem + (t & 1) * kTileBytes;
      const int first = kv_len32 - key0;          // 1..63 keys stay
      for (int e = tid; e < 64 * (kBlock - first); e += kThreads) {
        const int run = e / (kBlock - first), key = first + e % (kBlock - first);
        *(u32x4_t*)(st + run * 1024 + key * 16) = u32x4_t{0u, 0u, 0u, 0u};
      }
      barrier();
    }
    tile(t, t & 1, t == 0, with_dma_tag);
  };
  for (int t = 0; t < n_tiles - 1; ++t) step(t, std::true_type{});
  if (n_tiles > 0) step(n_tiles - 1, std::false_type{});

  // ---- epilogue: lane (lg, lc) holds latent values 16 bb + 4 lg .. +3 of its rows ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = quad_sum(l_run[qb]);
    if (!row_valid[qb]) continue;
    const float inv = 1.f / l_tot;
    EO* orow = (EO*)a.out + (tok[qb] * a.heads + head[qb]) * (int64_t)kMlaLatent + 4 * lg;
#pragma unroll
    for (int b = 0; b < kNDB; ++b) {
      const float v0 = o[b][qb][0] * inv, v1 = o[b][qb][1] * inv, v2 = o[b][qb][2] * inv, v3 = o[b][qb][3] * inv;
      if constexpr (sizeof(EO) == 2) *(u32x2_t*)(orow + 16 * b) = u32x2_t{pack_bf16(v0, v1), pack_bf16(v2, v3)};
      else *(f32x4_t*)(orow + 16 * b) = f32x4_t{v0, v1, v2, v3};
    }
    if (a.lse && lg == 0) a.lse[(int64_t)head[qb] * c + tok[qb]] = (m_run[qb] * cs + __log2f(l_tot)) * kLn2;
  }
}

// fp8 latent cache -> bf16 blocks in logical order: staging block j holds the
// records of logical block j, each value its e4m3 code times the token's fp32
// group scale, rounded once to bf16 (the rotary part is bf16 already).  One
// workgroup per block; the prefill kernel then reads the staging buffer.
__global__ __launch_bounds__(256) void mla_dequant_kernel(const unsigned char* pool, const int32_t* table,
                                                          int32_t num_blocks, unsigned char* staging) {
  const int j = blockIdx.x;
  const unsigned char* src = pool + (int64_t)clamp_block(table[j], num_blocks) * kMlaFp8Block;
  unsigned char* dst = staging + (int64_t)j * kTileBytes;
  for (int it = threadIdx.x; it < 32 * 64; it += kThreads) {   // code run r of token t: values 16 r .. +15
    const int r = it >> 6, t = it & 63;
    const unsigned char* h = src + (t >> 5) * kMlaFp8Half;       // the token's half of the block
    const u32x4_t c = *(const u32x4_t*)(h + (r * 32 + (t & 31)) * 16);
    const float sc = *(const float*)(h + kMlaFp8HalfScales + (t & 31) * 16 + (r >> 3) * 4);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {                  // exact widening (unit scale), then the fp32 group scale
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[k], 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[k], 1.0f, true);
      w[2 * k] = pack_bf16(lo[0] * sc, lo[1] * sc);
      w[2 * k + 1] = pack_bf16(hi[0] * sc, hi[1] * sc);
    }
    *(u32x4_t*)(dst + ((2 * r) * 64 + t) * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
    *(u32x4_t*)(dst + ((2 * r + 1) * 64 + t) * 16) = u32x4_t{w[4], w[5], w[6], w[7]};
  }
  for (int it = threadIdx.x; it < 8 * 64; it += kThreads) {        // rotary runs -> bf16 runs 64 .. 71
    const int r = it >> 6, t = it & 63;
    *(u32x4_t*)(dst + (64 * 64 + it) * 16) =
        *(const u32x4_t*)(src + (t >> 5) * kMlaFp8Half + kMlaFp8HalfRope + (r * 32 + (t & 31)) * 16);
  }
}

int64_t mla_prefill_staging_bytes(bool fp8, int64_t kv_len) {
  return fp8 ? (kv_len + kBlock - 1) / kBlock * (int64_t)kTileBytes : 0;
}

hipError_t launch_mla_prefill(bool fp8, const MlaPrefillArgs& a, void* staging, hipStream_t stream) {
  const int64_t n_rb = a.chunk_len * (a.heads / 16);
  const int64_t grid = (n_rb + 7) / 8;
  if (grid == 0) return hipSuccess;
  MlaPrefillArgs b = a;
  if (fp8) {
    const int64_t n_blocks = (a.past_len + a.chunk_len + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(mla_dequant_kernel, dim3((unsigned)n_blocks), dim3(kThreads), 0, stream, a.pool,
                       a.block_table, a.num_blocks, (unsigned char*)staging);
    b.pool = (const unsigned char*)staging;
    b.block_table = nullptr;
    b.num_blocks = (int32_t)n_blocks;
  }
  if (b.out_f32)
    hipLaunchKernelGGL((mla_prefill_kernel<float>), dim3((unsigned)grid), dim3(kThreads), 0, stream, b);
  else
    hipLaunchKernelGGL((mla_prefill_kernel<uint16_t>), dim3((unsigned)grid), dim3(kThreads), 0, stream, b);
  return hipGetLastError();
}

}  // namespace chunkattn
