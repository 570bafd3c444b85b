// Host-visible kernel argument blocks and launchers of libchunkattn.
// Internal to the library: the public ABI is include/chunkattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace chunkattn {

constexpr int kBlock = 64;                     // tokens per paged block == keys per KV tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum class DType : int { F32 = 0, BF16 = 1 };

// One chunk of causal prefill over one sequence's cache.
struct PrefillArgs {
  const void* q;             // [chunk_len, heads, D]
  const void* k;             // contiguous [cap, kv_heads, D] or paged pool
  const void* v;
  void* out;                 // [chunk_len, heads, DV]
  float* lse;                // optional [heads, lse_stride] (column = token)
  const int32_t* block_table;
  float* ws_o;               // split partials [S][chunk_len*heads][DV]
  float* ws_ml;              // split partials [S][chunk_len*heads][2]
  int64_t past_len;
  int64_t chunk_len;
  int64_t kv_len;            // past_len + chunk_len
  int64_t lse_stride;
  int64_t k_stride_tok, k_stride_head;   // contiguous cache, in elements (always set)
  int64_t v_stride_tok, v_stride_head;
  int32_t heads, kv_heads, group;
  int32_t num_blocks;
  int32_t hpw;               // query heads per workgroup (1/2/4; paged bf16 path 1/2/4/8)
  int32_t n_tok_blocks;
  int32_t n_head_groups;
  int32_t num_splits;
  int32_t xcd_remap;
  float scale_log2;          // scale * log2(e)
  // Varlen batch: one launch covers every prefill-path sequence.  Then q, out
  // and lse point at the whole batch, block_table at [num_seqs, max_blocks],
  // and each sequence's chunk_len / past_len come from the device arrays.
  const int32_t* cu_seqlens_q;   // [num_seqs + 1]
  const int32_t* kv_lens;        // [num_seqs]
  const int64_t* wg_off;         // [num_seqs + 1] first workgroup of each sequence
  int32_t num_seqs, max_blocks;
};

// Split-KV decode over a varlen batch (sequences with q_len * group <= 32).
struct DecodeArgs {
  const void* q;             // [total_q, heads, D]
  const void* k;             // paged pools
  const void* v;
  const int32_t* block_tables;   // [num_seqs, max_blocks]
  const int32_t* cu_seqlens_q;   // [num_seqs + 1]
  const int32_t* kv_lens;        // [num_seqs]
  int64_t* ws_off;               // [num_seqs] first partial slot of each sequence
  int64_t* wg_off;               // [num_seqs + 1] first prefill workgroup of each sequence
  float* ws_o;                   // [slots][DV]
  float* ws_ml;                  // [slots][2]
  void* out;                     // [total_q, heads, DV] (merge)
  float* lse;                    // optional [heads, total_q] (merge)
  int64_t total_q;
  int64_t total_slots;           // partial slots the workspace holds (bound on every access)
  int32_t num_seqs, max_blocks, num_blocks;
  int32_t seq_begin;             // first sequence of this decode launch (grid z counts from it)
  int32_t heads, kv_heads, group;
  int32_t split_tokens;          // keys per split (multiple of 64)
  int32_t tok_wg;                // query tokens per prefill workgroup
  int32_t n_head_groups;         // prefill workgroups per token block
  int32_t out_f32;               // 1: fp32 output, 0: bf16
  float scale_log2;
};

// Prefill launch: returns the HIP launch status.
hipError_t launch_prefill(DType in, DType out, int D, int DV, bool paged, const PrefillArgs& a,
                          int grid, hipStream_t stream);
hipError_t launch_prefill_merge(DType out, int DV, const PrefillArgs& a, hipStream_t stream);
// Paged bf16 path: 8-wave workgroups (256 query rows), direct-to-LDS tiles.
bool prefill_paged_supported(int D, int DV);
// The 8-wave kernel on a token-major contiguous bf16 cache (k/v strides in
// PrefillArgs), read in place: d = d_v = 128.
bool prefill_contig_supported(DType in, int D, int DV);
hipError_t launch_prefill_contig(DType out, const PrefillArgs& a, int grid, hipStream_t stream);
// Workgroups chunk_attn_varlen launches for one sequence's prefill-path rows
// (0 for a sequence that takes the decode path); defined with the host API.
int64_t varlen_prefill_workgroups(int q_len, int heads, int kv_heads);
// Query rows per workgroup of the paged bf16 kernel for these head dims.
int prefill_paged_rows(int D, int DV);
hipError_t launch_prefill_paged(DType out, int D, int DV, const PrefillArgs& a, int grid, hipStream_t stream);
hipError_t launch_prefill_paged_varlen(DType out, int D, int DV, const PrefillArgs& a, int grid, hipStream_t stream);
bool prefill_supported(DType in, DType out, int D, int DV);

hipError_t launch_batch_plan(const DecodeArgs& a, hipStream_t stream);
// Decode partials of sequences [seq_begin, seq_end) of the batch.
hipError_t launch_decode(int D, int DV, const DecodeArgs& a, int max_splits, int seq_begin, int seq_end,
                         hipStream_t stream);
hipError_t launch_decode_merge(int DV, const DecodeArgs& a, hipStream_t stream);
bool decode_supported(int D, int DV);

// MLA latent (absorbed) decode over a paged latent cache (one record of 512
// latent + 64 rotary values per token, shared by every query head).
constexpr int kMlaLatent = 512, kMlaRope = 64, kMlaRecord = 576, kMlaStepKeys = 32;
// A decode work unit holds at most this many steps, so a segment spans at most
// 64 * kMlaBtRegs cache blocks (the kernel keeps their ids one per lane in
// kMlaBtRegs registers): a segment of U steps starting on either half of a
// block covers at most (U + 1) / 2 blocks.
constexpr int kMlaBtRegs = 3;
// LDS ring depth (32-key steps) of the decode kernel and how many of its
// workgroups one CU holds with that ring; the plan sizes a round of units by it.
constexpr int kMlaStagesBf16 = 2, kMlaStagesFp8 = 3;
constexpr int kMlaWgPerCuBf16 = 2, kMlaWgPerCuFp8 = 2;
constexpr int kMlaMaxUnitSteps = 2 * 64 * kMlaBtRegs - 1;
// Block bytes (64 tokens): bf16 [72 runs][64][16 B].  fp8: two 32-token halves,
// each one contiguous region of codes [32 runs][32][16 B], scales [32][4 fp32]
// and rotary [8 runs][32][16 B], so a 32-key decode step is a single region.
constexpr int64_t kMlaBf16Block = 72 * 64 * 16;
constexpr int64_t kMlaFp8Half = 32 * 32 * 16 + 32 * 16 + 8 * 32 * 16;
constexpr int64_t kMlaFp8HalfScales = 32 * 32 * 16;                  // offsets inside a half
constexpr int64_t kMlaFp8HalfRope = kMlaFp8HalfScales + 32 * 16;
constexpr int64_t kMlaFp8Block = 2 * kMlaFp8Half;

// MLA decode work plan: the 32-key steps of all sequences, laid end to end,
// are cut into `units` equal ranges; a unit's piece of one sequence (a
// segment) writes one partial, into slot s + unit of each head.
struct MlaArgs {
  const uint16_t* q;             // [num_seqs, heads, 576] bf16
  const unsigned char* pool;     // [num_blocks][block bytes]
  const int32_t* block_tables;   // [num_seqs, max_blocks]
  const int32_t* kv_lens;        // [num_seqs]
  int64_t* seq_steps;            // [num_seqs + 1] steps before each sequence (plan kernel output)
  int32_t* unit_seq;             // [units] sequence holding each unit's first step (plan kernel output)
  float* ws_o;                   // [heads][slots][512] unnormalised partials
  float* ws_ml;                  // [heads][slots][2]: max (log2 units) and sum
  void* out;                     // [num_seqs, heads, 512] bf16 or fp32
  float* lse;                    // [heads, num_seqs] or null
  int32_t num_seqs, max_blocks, num_blocks, heads, units, slots;
  int32_t out_f32;               // 1: fp32 output, 0: bf16
  float scale_log2;
};

struct MlaAppendArgs {
  const uint16_t* latent;        // [n_tokens, 512] bf16
  const uint16_t* rope;          // [n_tokens, 64] bf16
  const int32_t* block_table;
  unsigned char* pool;
  int64_t start_pos, n_tokens;
  int32_t num_blocks;
};

// MLA latent prefill of one prompt chunk: tokens past_len .. past_len + chunk_len - 1
// of one sequence, every head attending causally to the records 0 .. its position.
struct MlaPrefillArgs {
  const uint16_t* q;             // [chunk_len, heads, 576] bf16
  const unsigned char* pool;     // [num_blocks][block bytes]
  const int32_t* block_table;    // [ceil((past_len + chunk_len) / 64)]; null: block j is logical block j
  void* out;                     // [chunk_len, heads, 512] bf16 or fp32
  float* lse;                    // [heads, chunk_len] or null
  int64_t past_len, chunk_len;
  int32_t num_blocks, heads;     // heads: a multiple of 16
  int32_t out_f32;
  float scale_log2;
};

hipError_t launch_mla_decode(bool fp8, const MlaArgs& a, hipStream_t stream);
// fp8: `staging` holds mla_prefill_staging_bytes(true, past_len + chunk_len) bytes.
hipError_t launch_mla_prefill(bool fp8, const MlaPrefillArgs& a, void* staging, hipStream_t stream);
int64_t mla_prefill_staging_bytes(bool fp8, int64_t kv_len);
hipError_t launch_mla_append(bool fp8, const MlaAppendArgs& a, hipStream_t stream);

hipError_t launch_block_iota(int32_t* table, int n, hipStream_t stream);
// k_new / v_new: element (t, g, e) at t * *_tok + g * *_head + e (dense: kv_heads * D, D).
hipError_t launch_kv_append(DType dt, int D, int DV, const void* k_new, const void* v_new,
                            int64_t k_tok, int64_t k_head, int64_t v_tok, int64_t v_head,
                            int64_t start_pos, int64_t n_tokens, int kv_heads,
                            const int32_t* block_table, int num_blocks, void* k_pool, void* v_pool,
                            hipStream_t stream);

}  // namespace chunkattn
