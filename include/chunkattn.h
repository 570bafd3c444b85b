/*
 * libchunkattn — chunked-prefill causal attention for AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operation.  A chunk of `chunk_len` query tokens whose first token sits
 * at absolute position `past_len` attends, under the causal mask, to the
 * cached keys and values of every earlier position and of itself:
 *
 *   out[i, h, :] = sum_{j <= past_len + i} softmax_j(scale * q[i,h,:] . k[j,g,:]) v[j,g,:]
 *   g = h / (heads / kv_heads)          (grouped-query heads, contiguous groups)
 *
 * Sources: "VPP: Virtual Pipeline Parallelism for Efficient Chunked Prefill in
 * Long-Context LLM Inference", technical review (English edition):
 *   §2.2 Eq. (1) (softmax(QK^T/sqrt(d))V) and the causal rule beside it;
 *   §2.3 (a later chunk attends to all preceding chunks' KV cache);
 *   §2.1 (prefill is compute-bound, decode reads the whole cache).
 * "Revisiting Pipeline Parallelism for LLM Serving" notes, preliminaries on
 * chunks: a batch can mix prefill tokens with one token per decode request.
 * "GLM5.3 CyberSec W4A16 — parallel strategy and PP split" notes, §1 and §7:
 * a paged KV pool of 64-token blocks, and attention that returns the LSE so
 * partial results can be merged.
 *
 * Conventions for every call:
 *  - Pointers named *_host are host memory; every other pointer is device
 *    memory owned by the caller.  The library makes no device allocation;
 *    scratch space is passed in as `workspace`.  Two things it keeps per
 *    device until the process ends: the static scratch array behind
 *    chunk_attn_varlen_noalloc (part of its code object), and the two
 *    CU-masked streams and three events chunk_attn_varlen creates on its
 *    first co-scheduled call on that device.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return without synchronising.
 *  - Arguments are validated before any HIP call.  A rejected call returns a
 *    negative ca_status, enqueues nothing and leaves a message for
 *    chunkattn_last_error() (thread-local).  A failed launch returns
 *    CA_EHIP with the HIP error text.  No call aborts or throws.
 *  - Calls are thread-safe; calls that share output or workspace buffers on
 *    one stream are ordered by the stream, on different streams they race.
 *  - Device pointers must be 16-byte aligned.
 *  - Strides are dense except where an argument says otherwise (the
 *    contiguous cache of chunk_prefill_attn, the new tokens of
 *    chunkattn_kv_append); layouts are given per argument.
 *
 * KV cache layouts (B = CA_BLOCK_SIZE = 64 tokens, X = 16 / sizeof(element)):
 *  - CA_KV_CONTIGUOUS: k [capacity, kv_heads, head_dim],
 *                      v [capacity, kv_heads, head_dim_v]  (token-major).
 *  - CA_KV_PAGED:      k pool [num_blocks, kv_heads, head_dim / X, B, X]
 *                      v pool [num_blocks, kv_heads, B / X, head_dim_v, X]
 *    Each (block, KV head) tile is one contiguous run of B*head_dim (K) or
 *    B*head_dim_v (V) elements.  Inside a K tile, 16-byte runs of one token's
 *    features are interleaved across the block's tokens; inside a V tile,
 *    16-byte runs of consecutive tokens for one feature are interleaved across
 *    features.  Logical token t of a sequence lives in physical block
 *    block_table[t / B] at slot t % B.  chunkattn_kv_append() writes this
 *    layout.  Block ids are clamped to [0, num_blocks) on the device, so a bad
 *    table gives wrong numbers but never an access outside the pool.
 */
#ifndef CHUNKATTN_H
#define CHUNKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CA_BLOCK_SIZE 64
#define CHUNKATTN_VERSION 3

typedef enum {
  CA_OK = 0,
  CA_EINVAL = -1,        /* bad argument: null/misaligned pointer, bad size, bad scale */
  CA_EUNSUPPORTED = -2,  /* valid but not implemented: head dims, dtype pair */
  CA_ERANGE = -3,        /* past_len + chunk_len beyond the cache or block table */
  CA_EWORKSPACE = -4,    /* workspace missing or smaller than required */
  CA_EHIP = -5           /* the HIP runtime reported an error */
} ca_status;

/* Enumerated arguments travel as int32_t: the library validates whatever value
 * arrives, so an out-of-range one is an error code, never an invalid enum. */
typedef enum { CA_F32 = 0, CA_BF16 = 1 } ca_dtype;
typedef enum { CA_KV_CONTIGUOUS = 0, CA_KV_PAGED = 1 } ca_kv_layout;

/*
 * Options of chunk_prefill_attn.  Initialise with ca_prefill_opts_init();
 * passing NULL means the defaults below.
 */
typedef struct ca_prefill_opts {
  int32_t dtype;               /* a ca_dtype: element type of q, k, v.  Default CA_BF16. */
  int32_t out_dtype;           /* a ca_dtype: element type of out.  Default CA_BF16.
                                  Supported pairs: (bf16, bf16), (bf16, f32), (f32, f32). */
  int32_t head_dim_v;          /* value head dim; 0 = head_dim.  Must be <= head_dim. */
  int32_t kv_layout;           /* a ca_kv_layout, default CA_KV_CONTIGUOUS */
  int64_t kv_capacity;         /* contiguous: tokens allocated in k and v;
                                  0 = exactly past_len + chunk_len */
  const int32_t* block_table;  /* paged: device int32 [block_table_len] */
  int32_t block_table_len;     /* paged: >= ceil((past_len + chunk_len) / 64) */
  int32_t num_blocks;          /* paged: blocks in the pool */
  float* lse_out;              /* optional device fp32 [heads, chunk_len]:
                                  natural-log sum of exp(scale * logits) per row */
  void* workspace;             /* device scratch: split-KV partials and, for a
                                  bf16 contiguous cache, its re-laid copy */
  size_t workspace_bytes;
  int32_t num_splits;          /* 0 = choose (never needs more workspace than
                                  given; no workspace => no split); 1 = never
                                  split; > 1 = exactly this many key splits
                                  (capped at the number of key tiles) */
  int64_t k_stride_tok;        /* contiguous only, in elements: K[t, g, e] is at
                                  k_cache + t * k_stride_tok + g * k_stride_head + e;
                                  0 = dense (kv_heads * head_dim, head_dim).  Both
                                  must be multiples of 16 bytes (8 bf16 / 4 fp32
                                  elements), e.g. K and V as views into a fused
                                  QKV projection output. */
  int64_t k_stride_head;
  int64_t v_stride_tok;        /* the same for V (dense: kv_heads * head_dim_v, head_dim_v) */
  int64_t v_stride_head;
} ca_prefill_opts;

void ca_prefill_opts_init(ca_prefill_opts* opts);

/*
 * chunk_prefill_attn — one chunk of causal prefill attention (VPP review §2.2
 * Eq. (1) with the causal rule, §2.3 chunked prefill).
 *
 *   q_chunk  [chunk_len, heads, head_dim]        dtype
 *   k_cache, v_cache: layout per opts->kv_layout; the cache already holds the
 *            chunk's own keys and values at positions [past_len, past_len+chunk_len)
 *   out      [chunk_len, heads, head_dim_v]      out_dtype
 *   past_len >= 0, chunk_len >= 0 (0 is a no-op; q_chunk and out may then be
 *   NULL), heads % kv_heads == 0,
 *   (head_dim, head_dim_v) in {(64, 64), (128, 128), (192, 128)},
 *   scale finite and > 0 (1/sqrt(head_dim) in the usual case).
 * Keys at positions >= past_len + chunk_len are never read for V and never
 * influence any row; K/V beyond a row's own position do not change that row.
 * The result is deterministic (bitwise) for fixed arguments and split count.
 *
 * Contiguous bf16 cache with a paged-kernel head-dim pair: when the workspace
 * (256-byte aligned) holds at least the re-layout bytes counted by
 * chunkattn_prefill_contiguous_workspace_size, the prefix [0, past_len +
 * chunk_len) of K and V is first copied into the paged tile layout inside the
 * workspace (an identity block table), and the paged kernel runs on that copy:
 * its output is then bitwise that of the paged layout.  Without that room
 * (no workspace, or split partials only) the cache is read in place: at
 * (head_dim, head_dim_v) = (128, 128) by the same 8-wave kernel, laying each
 * tile out token-major in LDS and transposing its V once per workgroup into
 * the paged order (bitwise the paged result; 7-11% slower), at the other pairs by
 * the 4-wave contiguous kernel (same result within bf16 rounding, ~3x
 * slower at 128K).  Split-KV partials, if any, follow the copy.
 */
ca_status chunk_prefill_attn(const void* q_chunk, const void* k_cache, const void* v_cache,
                             int64_t past_len, int64_t chunk_len,
                             int32_t heads, int32_t kv_heads, int32_t head_dim, float scale,
                             void* out, const ca_prefill_opts* opts, void* stream);

/*
 * Workspace bytes chunk_prefill_attn needs for `num_splits` key splits
 * (0 for num_splits <= 1).
 */
size_t chunkattn_prefill_workspace_size(int64_t chunk_len, int32_t heads, int32_t head_dim_v,
                                        int32_t num_splits);

/*
 * Workspace bytes chunk_prefill_attn uses with a contiguous cache of element
 * type `dtype`: the re-laid K/V prefix (CA_BF16 and a paged-kernel head-dim
 * pair; for other dtypes or dims nothing) plus the split partials of
 * `num_splits` splits (0 = the count it would choose).  Returns 0 for invalid
 * sizes.
 */
size_t chunkattn_prefill_contiguous_workspace_size(int64_t past_len, int64_t chunk_len, int32_t heads,
                                                   int32_t kv_heads, int32_t head_dim, int32_t head_dim_v,
                                                   int32_t dtype, int32_t num_splits);

/*
 * The split count chunk_prefill_attn picks for num_splits = 0 when the
 * workspace is large enough (1 = no split).  Splitting pays when the chunk
 * is short but its prefix is long: too few workgroups would hold the GPU.
 * Returns 0 for invalid sizes.
 */
int32_t chunkattn_prefill_auto_splits(int64_t past_len, int64_t chunk_len, int32_t heads, int32_t kv_heads);

/*
 * chunk_attn_varlen — one batch mixing prefill chunks and decode requests
 * over a paged KV pool (Revisiting Pipeline Parallelism for LLM Serving,
 * preliminaries: prefill requests contribute many tokens, decode requests one;
 * VPP review §2.1: decode reads the whole cache).
 *
 * Sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) of q and
 * out; its kv_lens[s] cached tokens include those rows' own keys, so its
 * queries sit at positions kv_lens[s] - q_len_s .. kv_lens[s] - 1.
 *   q            [total_q, heads, head_dim] bf16
 *   out          [total_q, heads, head_dim_v] in out_dtype: CA_BF16 (rounded to
 *                nearest even) or CA_F32
 *   k_pool, v_pool  paged layout above (bf16)
 *   block_tables [num_seqs, max_blocks_per_seq] device int32
 *   cu_seqlens_q [num_seqs + 1], kv_lens [num_seqs]   device int32
 *   cu_seqlens_q_host, kv_lens_host                   the same values in host memory
 *                (used only to size and plan launches; they must equal the device
 *                copies — if they do not, results are undefined, but every kernel
 *                still keeps its reads and writes inside the buffers described here)
 *   lse_out      optional device fp32 [heads, total_q]
 *   workspace    device scratch of chunkattn_varlen_workspace_size() bytes
 *                (256-byte aligned; needed whenever the batch has query rows)
 * Requires q_len_s <= kv_lens[s] <= 64 * max_blocks_per_seq for every
 * sequence (q_len_s = 0 is allowed and skipped), 1 <= num_seqs <= 65535 and
 * (head_dim, head_dim_v) in {(64, 64), (128, 128), (192, 128)}.  A sequence
 * whose rows per KV head, q_len_s * (heads / kv_heads), are at most 32 takes
 * the split-KV decode path; longer ones take the prefill path.  Both write
 * straight into out.
 * When the batch holds both kinds and neither dwarfs the other, the prefill
 * part (matrix-core bound) and the decode part (HBM bound) run at the same
 * time on two halves of the GPU's CUs: two internal CU-masked streams, made
 * once per device, forked from `stream` and joined back to it with events,
 * so the call still behaves as work enqueued on `stream`.
 */
ca_status chunk_attn_varlen(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t num_blocks,
                            const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                            const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                            int32_t num_seqs, int32_t heads, int32_t kv_heads,
                            int32_t head_dim, int32_t head_dim_v, float scale,
                            void* out, int32_t out_dtype, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes chunk_attn_varlen needs for this batch (host arrays). */
size_t chunkattn_varlen_workspace_size(const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                       int32_t num_seqs, int32_t heads, int32_t kv_heads,
                                       int32_t head_dim_v);

/* Bytes of the per-device scratch array behind chunk_attn_varlen_noalloc. */
#define CHUNKATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * chunk_attn_varlen_noalloc — chunk_attn_varlen for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, layouts and results as
 * chunk_attn_varlen, without the workspace: the batch's per-sequence offsets
 * and decode partials go to a static array of CHUNKATTN_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds on every device it runs on until the
 * process ends.  The call allocates nothing (no hipMalloc or hipFree); its
 * first call on a device looks the array's address up for that device.
 *   Returns CA_EWORKSPACE, before any HIP call, for a batch whose
 *   chunkattn_varlen_workspace_size() exceeds the array (e.g. a mixed batch
 *   of one 2048-token chunk and 256 decodes of up to 32K tokens needs 34 MiB).
 *   All calls on one device share that device's array and it keeps the last
 *   call's contents: calls ordered on one stream are safe, calls that may
 *   overlap on one device (other streams or threads with no ordering between
 *   them) race and must be serialised by the caller.  The batch's own kernels
 *   write every byte they later read, so nothing needs clearing between calls.
 */
ca_status chunk_attn_varlen_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t num_blocks,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                    const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                    int32_t num_seqs, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim, int32_t head_dim_v, float scale,
                                    void* out, int32_t out_dtype, float* lse_out, void* stream);

/*
 * chunkattn_kv_append — write n_tokens new keys/values of one sequence into
 * the paged pool at logical positions [start_pos, start_pos + n_tokens)
 * (the cache write that precedes each chunk's attention, VPP review §2.3).
 *   k_new [n_tokens, kv_heads, head_dim], v_new [n_tokens, kv_heads, head_dim_v]
 *   block_table [block_table_len] device int32, covering start_pos + n_tokens.
 *   src_strides: NULL for dense k_new / v_new, else a host array {k token,
 *   k head, v token, v head} of element strides (element (t, g, e) of k_new at
 *   t * src_strides[0] + g * src_strides[1] + e), each a positive multiple of
 *   16 bytes: e.g. the new tokens' K and V as views into a fused QKV output.
 * Bitwise copy; no arithmetic.  Block ids are clamped to [0, num_blocks).
 */
ca_status chunkattn_kv_append(const void* k_new, const void* v_new, int64_t start_pos, int64_t n_tokens,
                              int32_t kv_heads, int32_t head_dim, int32_t head_dim_v, int32_t dtype,
                              const int32_t* block_table, int32_t block_table_len, int32_t num_blocks,
                              void* k_pool, void* v_pool, const int64_t* src_strides, void* stream);

/*
 * Pipeline schedules that chunked prefill feeds (host only: no GPU work, no
 * stream).  VPP technical review (English edition) §4.1 Eq. (2) (per-stage
 * chunk latency tau_k, near-linear in k), §4.2 Alg. 1 / Eq. (3a)-(3b) (the
 * V-shaped layout: s0, s3 on rank pp0 and s1, s2 on pp1; while pp1 runs chunk
 * k's middle stages pp0 runs s3 of chunk k-1, then s0 of chunk k+1), §4.4
 * (VPP-Async: pp0's pair issued the other way round), §2.4 (the conventional
 * layout: s0, s1 on pp0, s2, s3 on pp1) and §4.5 Alg. 2 / Eq. (4a) (the next
 * request's leading chunks packed into the (N + 1) t drain window).
 */
typedef enum { CA_SCHED_CPP = 0, CA_SCHED_VPP = 1, CA_SCHED_VPP_ASYNC = 2 } ca_sched_kind;

/*
 * chunkattn_sched_simulate — start and end time of every virtual stage of
 * n_chunks chunks on two ranks.
 *   kind            ca_sched_kind.
 *   tau[n_chunks]   host, per-virtual-stage latency of each chunk (finite, >= 0, any time unit).
 *   request         host int32 [n_chunks], non-decreasing request id of each chunk, or NULL (one request).
 *   comm            delay of a hand-off between the two ranks (same unit, >= 0); it occupies neither rank.
 *   pack            0: a request's first stage waits for the previous request's last stage.
 *                   1: under the V layouts the next request's leading entry stages (count from
 *                      chunkattn_sched_drain_pack with t = the current request's first tau) run in
 *                      pp0's drain slot before the current request's last exit stage; under CPP the
 *                      barrier between requests is simply dropped.
 *   stage_start, stage_end   host double [n_chunks * 4] (chunk-major, stage minor) or NULL.
 *   rank_busy       host double [2] or NULL: summed stage time of pp0 and pp1.
 *   makespan        host double, required: the last stage's end time.
 * Every stage of chunk k takes tau[k]; a stage starts when its rank has
 * finished the stage before it in the rank's order and the chunk's previous
 * stage has ended (plus comm when that stage ran on the other rank).
 * Returns CA_OK or CA_EINVAL.  All buffers belong to the caller.
 */
ca_status chunkattn_sched_simulate(int32_t kind, int32_t n_chunks, const double* tau, const int32_t* request,
                                   double comm, int32_t pack, double* stage_start, double* stage_end,
                                   double* rank_busy, double* makespan);

/*
 * chunkattn_sched_drain_pack — Alg. 2 / Eq. (4a): the number of leading
 * chunks of the next request (host tau_next[n_next]) whose latencies fit,
 * in order, into the drain window (n_chunks + 1) * t of the current request;
 * stops at the first chunk that does not fit.  *window_left (optional)
 * receives what is left of the window.  Returns the count (>= 0) or CA_EINVAL.
 */
int32_t chunkattn_sched_drain_pack(int32_t n_chunks, double t, int32_t n_next, const double* tau_next,
                                   double* window_left);

/*
 * Online attention-latency predictor (host only).  "Revisiting Pipeline
 * Parallelism for LLM Serving" paper notes §2.3 (ALP): the attention time of
 * a batch is linear in three features summed over its sequences — past
 * context x new prefill tokens, new tokens squared, and the context of each
 * decode request — with coefficients adapted online by recursive least
 * squares with a forgetting factor.  For the kernel alone a constant term
 * replaces the notes' offline token-linear part:
 *   x = [1, sum(L_past * L_pre) / 1e6, sum(L_pre^2) / 1e6, sum(L_dec) / 1e3, fill]
 * where a sequence with q_len > 1 is a prefill chunk (L_pre = q_len,
 * L_past = kv_len - q_len) and one with q_len == 1 a decode (L_dec = kv_len).
 * The fifth feature, this library's addition, is the GPU fill of the batch's
 * prefill launch: with W the workgroups chunk_attn_varlen launches for its
 * prefill-path sequences (256 query rows each, one per CU) and 256 CUs,
 *   fill = (ceil(W / 256) * 256 / W - 1) * sum over them of causal pairs / 1e6,
 * causal pairs = L_past * L_pre + L_pre (L_pre + 1) / 2: the work the idle
 * CUs of the last round stand for (0 when W fills whole rounds).
 */
#define CA_ALP_FEATURES 5
typedef struct {
  double theta[CA_ALP_FEATURES];                     /* coefficients, time unit of the measurements */
  double info[CA_ALP_FEATURES * CA_ALP_FEATURES];    /* weighted normal matrix R (inverse covariance), row-major */
  double rhs[CA_ALP_FEATURES];                       /* weighted right-hand side b */
  double lambda;                                     /* forgetting factor, 0 < lambda <= 1 */
  int64_t n_obs;                                     /* updates so far */
} ca_alp_state;

/* Feature vector x[CA_ALP_FEATURES] of a batch (host arrays q_lens, kv_lens of
 * num_seqs sequences, kv_len >= q_len >= 0) run with heads query heads over
 * kv_heads KV heads (they size the prefill launch of the fill feature).
 * CA_OK or CA_EINVAL. */
ca_status chunkattn_alp_features(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens, int32_t heads,
                                 int32_t kv_heads, double* x);

/* Start a recursive least-squares fit: theta = 0, R = I / delta (covariance delta * I), b = 0.
 * CA_OK or CA_EINVAL. */
ca_status chunkattn_alp_init(ca_alp_state* state, double lambda, double delta);

/* Predicted time theta . x (NaN for NULL arguments). */
double chunkattn_alp_predict(const ca_alp_state* state, const double* x);

/* One recursive least-squares step with a measured time, in information form:
 * R = lambda R + x x', b = lambda b + x measured, theta = R^-1 b (Cholesky) —
 * the estimate of the gain form g = P x / (lambda + x' P x), theta += g e,
 * P = (P - g x' P) / lambda with P = R^-1, without its loss of precision.
 * *prior_error (optional) receives measured - theta . x before the step.
 * CA_OK, CA_EINVAL, or CA_ERANGE if R stopped being positive definite.
 * The state belongs to the caller; calls on one state must not overlap. */
ca_status chunkattn_alp_update(ca_alp_state* state, const double* x, double measured, double* prior_error);

/*
 * MLA latent (absorbed) attention over a paged latent cache.
 * "02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16" deployment notes §1, §4: an
 * MLA layer caches one latent record per token shared by every query head,
 * 1152 B in bf16 or 656 B in the fp8 latent format (the VPP review's models,
 * DeepSeek-V3.1 and GLM-5.x, use MLA, §6.1).  A record is 512 latent + 64
 * rotary values.  Cache blocks hold 64 tokens, one shared head:
 *   CA_MLA_BF16: [72 runs][64 tokens][8 bf16]                      73728 B per block
 *   CA_MLA_FP8 : two halves of 32 tokens (tokens 0-31, then 32-63), each
 *                [32 runs][32 tokens][16 e4m3] latent codes,
 *                [32 tokens][4 fp32] scales (one per 128 latent values),
 *                [8 runs][32 tokens][8 bf16] rotary                20992 B per half,
 *                                                                  41984 B per block (= 64 x 656)
 * Run r holds values 8r..8r+7 (bf16) or 16r..16r+15 (codes) of every token
 * (of the half).
 * fp8 codes are OCP e4m3 (bias 7, largest normal 448): a group's scale is
 * amax / 448 in fp32 (1 for an all-zero group) and a value's code is its fp32
 * quotient by the scale clamped to +-448, rounded to the nearest code.
 */
typedef enum { CA_MLA_BF16 = 0, CA_MLA_FP8 = 1 } ca_mla_format;

/* Bytes of one 64-token cache block of the format (0 for an unknown format). */
size_t chunkattn_mla_block_bytes(int32_t format);

/*
 * chunkattn_mla_kv_append — write n_tokens records of one sequence at
 * logical positions [start_pos, start_pos + n_tokens) of its block table.
 *   latent [n_tokens, 512] bf16, rope [n_tokens, 64] bf16 (device, 16-byte aligned).
 *   block_table [block_table_len] device int32; pool [num_blocks * block bytes] device.
 * bf16 copies bits; fp8 quantises each 128-value latent group.  Block ids are
 * clamped to [0, num_blocks).  CA_OK, CA_EINVAL, CA_ERANGE or CA_EHIP.
 */
ca_status chunkattn_mla_kv_append(const void* latent, const void* rope, int64_t start_pos, int64_t n_tokens,
                                  int32_t format, const int32_t* block_table, int32_t block_table_len,
                                  int32_t num_blocks, void* pool, void* stream);

/* Workspace bytes chunk_mla_decode needs for these context lengths (host array); 0 for invalid arguments. */
size_t chunkattn_mla_decode_workspace_size(const int32_t* kv_lens_host, int32_t num_seqs, int32_t heads,
                                           int32_t format);

/*
 * chunk_mla_decode — one decode token per sequence attends to its whole
 * latent cache (the query sits at position kv_len - 1, VPP review §2.1: decode
 * reads the entire cache).
 *   q    [num_seqs, heads, 576] bf16: per head, the latent-space projection of
 *        the no-rope query (512) then its rotary part (64).
 *   out  [num_seqs, heads, 512] in out_dtype (CA_BF16, rounded to nearest even, or
 *        CA_F32): the attention output in latent space.
 *   lse_out optional [heads, num_seqs] fp32, natural log of the softmax denominator.
 *   block_tables [num_seqs, max_blocks_per_seq] device; kv_lens on device and host (>= 1).
 *   heads: a positive multiple of 16, at most 1024 (a workgroup serves 16 heads).
 *   num_seqs: 0 .. 65535; the device kv_lens must equal the host ones (the host
 *        copy sizes the work plan, the device copy drives the kernels).
 *   workspace: >= chunkattn_mla_decode_workspace_size bytes, 256-byte aligned:
 *        the work plan (per-sequence step offsets, work-unit starts) and the
 *        unnormalised partial results, combined in a fixed order (deterministic).
 * Keys past kv_len never reach an output.  CA_OK, CA_EINVAL, CA_EUNSUPPORTED,
 * CA_ERANGE (also for a batch of more than 2^31 32-key steps), CA_EWORKSPACE or
 * CA_EHIP; validation precedes any HIP call.
 */
ca_status chunk_mla_decode(const void* q, const void* pool, int32_t format, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t num_blocks, const int32_t* kv_lens_dev,
                           const int32_t* kv_lens_host, int32_t num_seqs, int32_t heads, float scale, void* out,
                           int32_t out_dtype, float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes chunk_mla_prefill needs: 0 for the bf16 cache; for fp8,
 * ceil((past_len + chunk_len) / 64) * 73728 (the visible prefix widened to bf16
 * blocks).  0 for invalid arguments. */
size_t chunkattn_mla_prefill_workspace_size(int64_t past_len, int64_t chunk_len, int32_t format);

/*
 * chunk_mla_prefill — one prompt chunk of one sequence over its latent cache:
 * the tokens at positions [past_len, past_len + chunk_len) (VPP review §2.3:
 * a long prompt is cut into chunks, each attending to the cache of all earlier
 * chunks and causally to itself, §2.2 Eq. (1)).  Every head of the token at
 * position p attends to the records 0 .. p; keys are the 576-value records,
 * values their 512-value latents, and the output stays in latent space — the
 * decode entry's absorbed attention with chunk_len query tokens.
 *   q    [chunk_len, heads, 576] bf16, dense (device, 16-byte aligned).
 *   pool, format: the cache of the sequence, already holding the records of
 *        positions 0 .. past_len + chunk_len - 1 (append the chunk first).
 *        CA_MLA_FP8 records enter the matrix products as bf16(code x scale),
 *        one rounding per value.
 *   block_table [block_table_len] device int32, >= ceil((past_len + chunk_len) / 64)
 *        entries; ids are clamped to [0, num_blocks).
 *   heads: a positive multiple of 16, at most 1024 (a row block is one token's
 *        16 consecutive heads).
 *   out  [chunk_len, heads, 512] in out_dtype (CA_BF16, rounded to nearest even,
 *        or CA_F32); lse_out optional [heads, chunk_len] fp32, natural log.
 *   workspace: >= chunkattn_mla_prefill_workspace_size bytes, 256-byte aligned
 *        (fp8 only; may be NULL for bf16).  Its contents are scratch.
 * Pool slots past the sequence end never reach an output.  Deterministic.
 * CA_OK, CA_EINVAL, CA_EUNSUPPORTED, CA_ERANGE, CA_EWORKSPACE or CA_EHIP;
 * validation precedes any HIP call.
 */
ca_status chunk_mla_prefill(const void* q, const void* pool, int32_t format, const int32_t* block_table,
                            int32_t block_table_len, int32_t num_blocks, int64_t past_len, int64_t chunk_len,
                            int32_t heads, float scale, void* out, int32_t out_dtype, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* chunkattn_last_error(void);

/* CHUNKATTN_VERSION of the built library. */
int32_t chunkattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKATTN_H */
