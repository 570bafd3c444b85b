// C ABI of libchunkattn: argument validation, launch planning and dispatch.
// Every check runs before the first HIP call, so a rejected call touches no
// device state.  See include/chunkattn.h for the contract of each entry point.
#include "chunkattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.h"

using namespace chunkattn;

namespace {

thread_local char g_err[512] = "";

ca_status fail(ca_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ca_status ok() {
  g_err[0] = '\0';
  return CA_OK;
}

ca_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kNumCUs = 256;          // MI355X
constexpr int64_t kMaxTokens = (int64_t)1 << 30;

// Query heads of one KV head that share a prefill workgroup: the largest
// power of two up to the workgroup's wave count dividing the GQA group.  The
// 4-wave kernel (contiguous or fp32 caches) holds 128 query rows, the 8-wave
// paged bf16 kernel 256.
int heads_per_wg(int group, int waves) {
  for (int h = waves; h > 1; h >>= 1)
    if (group % h == 0) return h;
  return 1;
}
constexpr int kWavesSmall = 4, kWavesPaged = 8;

size_t prefill_ws_bytes(int64_t chunk_len, int heads, int dv, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)chunk_len * heads * splits;
  return align_up(rows * dv * sizeof(float), 256) + rows * 2 * sizeof(float);
}

// A bf16 contiguous cache is read by the paged kernel after the K/V prefix is
// re-laid into the workspace: an identity block table, then K and V pools of
// ceil(kv_len / 64) blocks in the paged tile layout.
struct Relayout {
  int64_t blocks = 0;
  size_t table = 0, k = 0, v = 0, bytes = 0;
};
Relayout relayout_plan(int64_t kv_len, int kv_heads, int d, int dv) {
  Relayout r;
  r.blocks = (kv_len + kBlock - 1) / kBlock;
  r.table = align_up((size_t)r.blocks * sizeof(int32_t), 256);
  r.k = (size_t)r.blocks * kv_heads * d * kBlock * 2;
  r.v = (size_t)r.blocks * kv_heads * dv * kBlock * 2;
  r.bytes = r.table + r.k + r.v;
  return r;
}

// Decode split length: aim for enough waves to fill the chip several times
// over, in multiples of the 64-token tile.
int decode_split_tokens(const int32_t* cu, const int32_t* kv, int num_seqs, int kv_heads, int group) {
  int64_t tiles = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = cu[s + 1] - cu[s];
    if (q_len >= 1 && q_len * group <= 32) tiles += (int64_t)(kv[s] + kBlock - 1) / kBlock * kv_heads;
  }
  const int64_t target_waves = (int64_t)kNumCUs * 4 * 16;
  int64_t per = (tiles + target_waves - 1) / target_waves;   // tiles per wave
  if (per < 4) per = 4;
  if (per > 64) per = 64;
  return (int)per * kBlock;
}

// Host plan of a varlen batch, from the host copies of the lengths.  The
// device-side plan kernel derives the same offsets from the device copies.
struct BatchPlan {
  int split_tokens = 0;
  int max_splits = 0;
  int64_t slots = 0;          // decode partial slots
  int64_t prefill_wgs = 0;    // prefill workgroups over all prefill-path sequences
  int n_decode = 0, n_prefill = 0;
  size_t ws_off_bytes = 0, wg_off_bytes = 0, o_bytes = 0, ml_bytes = 0;
  size_t total() const {
    return (n_decode || n_prefill) ? ws_off_bytes + wg_off_bytes + o_bytes + ml_bytes : 0;
  }
};

BatchPlan plan_batch(const int32_t* cu, const int32_t* kv, int num_seqs, int heads, int kv_heads, int dv) {
  BatchPlan p;
  const int group = heads / kv_heads;
  p.split_tokens = decode_split_tokens(cu, kv, num_seqs, kv_heads, group);
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = cu[s + 1] - cu[s];
    if (q_len >= 1 && q_len * group <= 32) {
      const int ns = (kv[s] + p.split_tokens - 1) / p.split_tokens;
      p.slots += (int64_t)q_len * heads * ns;
      if (ns > p.max_splits) p.max_splits = ns;
      ++p.n_decode;
    } else if (q_len > 0) {
      p.prefill_wgs += varlen_prefill_workgroups(q_len, heads, kv_heads);
      ++p.n_prefill;
    }
  }
  p.ws_off_bytes = align_up((size_t)num_seqs * sizeof(int64_t), 256);
  p.wg_off_bytes = align_up((size_t)(num_seqs + 1) * sizeof(int64_t), 256);
  p.o_bytes = align_up((size_t)p.slots * dv * sizeof(float), 256);
  p.ml_bytes = align_up((size_t)p.slots * 2 * sizeof(float), 256);
  return p;
}

// Split count for a short chunk over a long prefix (sized for the 8-wave
// paged kernel, one workgroup per CU): enough workgroups for one per CU, so
// the launch is a single round, each split keeping at least 16 key tiles.
// Measured on MI355X, one round beats two (1.5-16% on chunks of 512 down to
// 128 tokens over 32K-200K prefixes).
int auto_splits(int64_t past_len, int64_t chunk_len, int heads, int kv_heads, int paged_rows) {
  const int hpw = heads_per_wg(heads / kv_heads, kWavesPaged);
  const int tok_wg = paged_rows / hpw;
  const int64_t base = (chunk_len + tok_wg - 1) / tok_wg * (heads / hpw);
  const int64_t n_tiles = (past_len + chunk_len + kBlock - 1) / kBlock;
  if (base == 0 || base >= kNumCUs || n_tiles < 32) return 1;
  int64_t want = (kNumCUs + base - 1) / base;
  const int64_t cap = n_tiles / 16;
  if (want > cap) want = cap;
  return want > 1 ? (int)want : 1;
}

ca_status check_dtype(int d) {
  if (d != CA_F32 && d != CA_BF16) return fail(CA_EINVAL, "unknown dtype %d", d);
  return CA_OK;
}

}  // namespace

namespace chunkattn {
// Workgroups chunk_attn_varlen launches for one sequence's prefill-path rows (0 for a decode-path
// sequence); the latency predictor's fill feature uses the same count.
int64_t varlen_prefill_workgroups(int q_len, int heads, int kv_heads) {
  const int group = heads / kv_heads;
  if (q_len < 1 || q_len * group <= 32) return 0;
  const int hpw = heads_per_wg(group, kWavesPaged);
  const int tok_wg = prefill_paged_rows(0, 0) / hpw;
  return (int64_t)((q_len + tok_wg - 1) / tok_wg) * (heads / hpw);
}
int num_cus() { return kNumCUs; }
// Error string of the calling thread, shared with the host-only entry points.
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = '\0'; }
}  // namespace chunkattn

namespace {

// MLA latent decode plan: keys per split (a multiple of the 32-key step) so
// that about four rounds of waves fill the chip (2 bf16 / 3 fp8 waves per CU
// fit their double-buffered LDS), and the largest split count of any sequence.
// MLA decode plan.  The 32-key steps of all sequences, laid end to end, are
// cut into `units` equal ranges: a multiple of the workgroups the chip holds at
// once (kMlaWgPerCu* per CU, shared by the head blocks), rounded to 8
// so units spread evenly over the XCDs, with at most kMlaMaxUnitSteps steps
// each.  Workspace: per-sequence step prefix sums, each unit's first sequence,
// then per head and slot (num_seqs + units slots) the partial (m, l) and O.
struct MlaPlan {
  int64_t steps = 0;
  int64_t units = 0, slots = 0;
  size_t unit_off = 0, ml_off = 0, o_off = 0, bytes = 0;
};
MlaPlan plan_mla(const int32_t* kv_lens, int num_seqs, int heads, bool fp8) {
  MlaPlan p;
  for (int s = 0; s < num_seqs; ++s) p.steps += (kv_lens[s] + kMlaStepKeys - 1) / kMlaStepKeys;
  const int nhb = heads / 16;
  int per_hb = kNumCUs * (fp8 ? kMlaWgPerCuFp8 : kMlaWgPerCuBf16) / nhb;
  per_hb = per_hb >= 8 ? per_hb / 8 * 8 : 8;
  const int64_t cap = (int64_t)per_hb * kMlaMaxUnitSteps;
  p.units = (p.steps + cap - 1) / cap * per_hb;
  if (p.units > p.steps) p.units = p.steps;
  p.slots = num_seqs + p.units;
  p.unit_off = align_up((size_t)(num_seqs + 1) * sizeof(int64_t), 256);
  p.ml_off = p.unit_off + align_up((size_t)p.units * sizeof(int32_t), 256);
  p.o_off = p.ml_off + align_up((size_t)heads * p.slots * 2 * sizeof(float), 256);
  p.bytes = p.o_off + (size_t)heads * p.slots * kMlaLatent * sizeof(float);
  return p;
}

ca_status check_mla(const int32_t* kv_lens, int num_seqs, int heads, int max_blocks, int format) {
  if (format != CA_MLA_BF16 && format != CA_MLA_FP8) return fail(CA_EINVAL, "unknown MLA cache format %d", format);
  if (num_seqs < 0 || num_seqs > 65535) return fail(CA_EINVAL, "num_seqs must be in [0, 65535]");
  if (heads <= 0 || heads % 16 || heads > 1024)
    return fail(CA_EUNSUPPORTED, "heads must be a positive multiple of 16 up to 1024, got %d", heads);
  if (num_seqs > 0 && !kv_lens) return fail(CA_EINVAL, "kv_lens_host is required");
  for (int s = 0; s < num_seqs; ++s) {
    if (kv_lens[s] < 1) return fail(CA_EINVAL, "sequence %d: kv_len %d < 1", s, kv_lens[s]);
    if ((int64_t)kv_lens[s] > (int64_t)max_blocks * kBlock)
      return fail(CA_ERANGE, "sequence %d: kv_len %d exceeds %d blocks", s, kv_lens[s], max_blocks);
  }
  return CA_OK;
}

}  // namespace

extern "C" {

void ca_prefill_opts_init(ca_prefill_opts* o) {
  if (!o) return;
  std::memset(o, 0, sizeof *o);
  o->dtype = CA_BF16;
  o->out_dtype = CA_BF16;
  o->kv_layout = CA_KV_CONTIGUOUS;
}

const char* chunkattn_last_error(void) { return g_err; }

int32_t chunkattn_version(void) { return CHUNKATTN_VERSION; }

size_t chunkattn_prefill_workspace_size(int64_t chunk_len, int32_t heads, int32_t head_dim_v, int32_t num_splits) {
  if (chunk_len <= 0 || heads <= 0 || head_dim_v <= 0) return 0;
  return prefill_ws_bytes(chunk_len, heads, head_dim_v, num_splits);
}

size_t chunkattn_prefill_contiguous_workspace_size(int64_t past_len, int64_t chunk_len, int32_t heads,
                                                   int32_t kv_heads, int32_t head_dim, int32_t head_dim_v,
                                                   int32_t dtype, int32_t num_splits) {
  if (past_len < 0 || chunk_len <= 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads || head_dim <= 0)
    return 0;
  const int dv = head_dim_v ? head_dim_v : head_dim;
  const int splits =
      num_splits == 0 ? auto_splits(past_len, chunk_len, heads, kv_heads, prefill_paged_rows(head_dim, dv)) : num_splits;
  size_t bytes = prefill_ws_bytes(chunk_len, heads, dv, splits);
  if (dtype == CA_BF16 && prefill_paged_supported(head_dim, dv) && past_len + chunk_len <= kMaxTokens)
    bytes += relayout_plan(past_len + chunk_len, kv_heads, head_dim, dv).bytes;
  return bytes;
}

int32_t chunkattn_prefill_auto_splits(int64_t past_len, int64_t chunk_len, int32_t heads, int32_t kv_heads) {
  if (past_len < 0 || chunk_len < 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads) return 0;
  return auto_splits(past_len, chunk_len, heads, kv_heads, prefill_paged_rows(128, 128));
}

ca_status chunk_prefill_attn(const void* q, const void* k, const void* v, int64_t past_len, int64_t chunk_len,
                             int32_t heads, int32_t kv_heads, int32_t head_dim, float scale, void* out,
                             const ca_prefill_opts* opts_in, void* stream) {
  ca_prefill_opts o;
  ca_prefill_opts_init(&o);
  if (opts_in) o = *opts_in;
  // An empty chunk may come with null q/out (empty tensors have no storage).
  if (!k || !v || (chunk_len != 0 && (!q || !out)))
    return fail(CA_EINVAL, "q, k_cache, v_cache and out must be non-null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(CA_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (past_len < 0 || chunk_len < 0) return fail(CA_EINVAL, "past_len and chunk_len must be >= 0");
  if (past_len + chunk_len > kMaxTokens) return fail(CA_ERANGE, "past_len + chunk_len exceeds 2^30 tokens");
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0)
    return fail(CA_EINVAL, "heads (%d) must be a positive multiple of kv_heads (%d)", heads, kv_heads);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(CA_EINVAL, "scale must be finite and > 0");
  if (ca_status st = check_dtype(o.dtype)) return st;
  if (ca_status st = check_dtype(o.out_dtype)) return st;
  const int dv = o.head_dim_v ? o.head_dim_v : head_dim;
  const DType din = (DType)o.dtype, dout = (DType)o.out_dtype;
  if (!prefill_supported(din, dout, head_dim, dv))
    return fail(CA_EUNSUPPORTED, "unsupported (head_dim, head_dim_v, dtype, out_dtype) = (%d, %d, %d, %d)",
                head_dim, dv, (int)o.dtype, (int)o.out_dtype);
  if (o.lse_out && !aligned(o.lse_out, 4)) return fail(CA_EINVAL, "lse_out must be 4-byte aligned");
  const int64_t kv_len = past_len + chunk_len;
  const bool paged = o.kv_layout == CA_KV_PAGED;
  if (o.kv_layout != CA_KV_CONTIGUOUS && !paged) return fail(CA_EINVAL, "unknown kv_layout %d", (int)o.kv_layout);
  if (paged) {
    if (!o.block_table || !aligned(o.block_table, 4)) return fail(CA_EINVAL, "paged layout needs a block_table");
    if (o.num_blocks <= 0) return fail(CA_EINVAL, "num_blocks must be > 0");
    if ((int64_t)o.block_table_len * kBlock < kv_len)
      return fail(CA_ERANGE, "block table covers %lld tokens, need %lld", (long long)o.block_table_len * kBlock,
                  (long long)kv_len);
  } else {
    const int64_t cap = o.kv_capacity ? o.kv_capacity : kv_len;
    if (cap < kv_len) return fail(CA_ERANGE, "kv_capacity %lld < past_len + chunk_len %lld", (long long)cap,
                                  (long long)kv_len);
  }
  // Contiguous-cache strides in elements (0 = dense); 16-byte multiples keep every load aligned.
  if (paged && (o.k_stride_tok || o.k_stride_head || o.v_stride_tok || o.v_stride_head))
    return fail(CA_EINVAL, "cache strides apply to the contiguous layout only");
  const int64_t ks_tok = o.k_stride_tok ? o.k_stride_tok : (int64_t)kv_heads * head_dim;
  const int64_t ks_head = o.k_stride_head ? o.k_stride_head : head_dim;
  const int64_t vs_tok = o.v_stride_tok ? o.v_stride_tok : (int64_t)kv_heads * dv;
  const int64_t vs_head = o.v_stride_head ? o.v_stride_head : dv;
  {
    const int64_t x = din == DType::BF16 ? 8 : 4;
    if (ks_tok <= 0 || ks_head <= 0 || vs_tok <= 0 || vs_head <= 0 || ks_tok % x || ks_head % x || vs_tok % x ||
        vs_head % x)
      return fail(CA_EINVAL, "cache strides must be positive multiples of 16 bytes (%lld elements)", (long long)x);
  }
  if (o.num_splits < 0) return fail(CA_EINVAL, "num_splits must be >= 0");

  const int group = heads / kv_heads;
  // bf16 contiguous cache: with room in the workspace, re-lay the prefix and run the paged kernel (the
  // fastest path); without it, d = d_v = 128 runs the same 8-wave kernel on the cache in place (its
  // per-lane load offsets, up to 63 token strides, are 32-bit), other head dims the 4-wave kernel
  const bool paged_dims = din == DType::BF16 && prefill_paged_supported(head_dim, dv);
  Relayout rl;
  bool relay = false;
  if (!paged && paged_dims && o.workspace && aligned(o.workspace, 256)) {
    rl = relayout_plan(kv_len, kv_heads, head_dim, dv);
    // An explicit split count keeps its partials' room: re-lay only when both fit,
    // otherwise read the cache in place with the whole workspace for partials.
    const int64_t n_tiles_rl = (kv_len + kBlock - 1) / kBlock;
    const int want_splits = o.num_splits > n_tiles_rl ? (int)n_tiles_rl : o.num_splits;
    relay = o.workspace_bytes >= rl.bytes + prefill_ws_bytes(chunk_len, heads, dv, want_splits);
  }
  // split partials follow the re-laid pools in the workspace
  void* const ws_split = relay ? (void*)((char*)o.workspace + rl.bytes) : o.workspace;
  const size_t ws_split_bytes = relay ? o.workspace_bytes - rl.bytes : o.workspace_bytes;
  const bool contig_native = !paged && !relay && prefill_contig_supported(din, head_dim, dv) &&
                             std::max(ks_tok, vs_tok) * 2 * kBlock < ((int64_t)1 << 31);
  const bool use_paged_kernel = (paged || relay || contig_native) && paged_dims;
  const int hpw = heads_per_wg(group, use_paged_kernel ? kWavesPaged : kWavesSmall);
  const int paged_rows = prefill_paged_rows(head_dim, dv);
  const int tok_wg = (use_paged_kernel ? paged_rows : 128) / hpw;
  const int64_t n_tb = (chunk_len + tok_wg - 1) / tok_wg;
  const int n_hg = heads / hpw;
  const int64_t base = n_tb * n_hg;
  const int64_t n_tiles = (kv_len + kBlock - 1) / kBlock;
  int splits = o.num_splits;
  if (splits == 0) {
    const int want = auto_splits(past_len, chunk_len, heads, kv_heads, paged_rows);
    splits = (want > 1 && ws_split && ws_split_bytes >= prefill_ws_bytes(chunk_len, heads, dv, want)) ? want : 1;
  } else if (splits > n_tiles) {
    splits = (int)(n_tiles > 0 ? n_tiles : 1);
  }
  if (splits > 1) {
    const size_t need = prefill_ws_bytes(chunk_len, heads, dv, splits);
    if (!ws_split || ws_split_bytes < need)
      return fail(CA_EWORKSPACE, "split-KV with %d splits needs %zu workspace bytes%s", splits, need,
                  relay ? " after the re-laid K/V" : "");
    if (!aligned(o.workspace, 256)) return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  }
  if (base * splits > 0x7fffffffLL) return fail(CA_ERANGE, "launch grid too large");
  if (chunk_len == 0) return ok();

  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = o.lse_out;
  a.block_table = o.block_table;
  a.past_len = past_len;
  a.chunk_len = chunk_len;
  a.kv_len = kv_len;
  a.lse_stride = chunk_len;
  a.k_stride_tok = ks_tok;
  a.k_stride_head = ks_head;
  a.v_stride_tok = vs_tok;
  a.v_stride_head = vs_head;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.num_blocks = o.num_blocks;
  a.hpw = hpw;
  a.n_tok_blocks = (int)n_tb;
  a.n_head_groups = n_hg;
  a.num_splits = splits;
  a.xcd_remap = (splits == 1 && n_hg % 8 == 0) ? 1 : 0;
  a.scale_log2 = scale * kLog2e;
  if (splits > 1) {
    const size_t rows = (size_t)chunk_len * heads * splits;
    a.ws_o = (float*)ws_split;
    a.ws_ml = (float*)((char*)ws_split + align_up(rows * dv * sizeof(float), 256));
  }
  hipStream_t s = (hipStream_t)stream;
  if (relay) {
    int32_t* table = (int32_t*)o.workspace;
    void* kpool = (char*)o.workspace + rl.table;
    void* vpool = (char*)o.workspace + rl.table + rl.k;
    hipError_t e = launch_block_iota(table, (int)rl.blocks, s);
    if (e == hipSuccess)
      e = launch_kv_append(DType::BF16, head_dim, dv, k, v, ks_tok, ks_head, vs_tok, vs_head, 0, kv_len, kv_heads,
                           table, (int)rl.blocks, kpool, vpool, s);
    if (e != hipSuccess) return hip_status(e, "contiguous cache re-layout");
    a.k = kpool;
    a.v = vpool;
    a.block_table = table;
    a.num_blocks = (int)rl.blocks;
  }
  hipError_t e = contig_native      ? launch_prefill_contig(dout, a, (int)(base * splits), s)
                 : use_paged_kernel ? launch_prefill_paged(dout, head_dim, dv, a, (int)(base * splits), s)
                                    : launch_prefill(din, dout, head_dim, dv, paged, a, (int)(base * splits), s);
  if (e != hipSuccess) return hip_status(e, "prefill launch");
  if (splits > 1) {
    e = launch_prefill_merge(dout, dv, a, s);
    if (e != hipSuccess) return hip_status(e, "prefill merge launch");
  }
  return ok();
}

size_t chunkattn_varlen_workspace_size(const int32_t* cu, const int32_t* kv, int32_t num_seqs, int32_t heads,
                                       int32_t kv_heads, int32_t head_dim_v) {
  if (!cu || !kv || num_seqs <= 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads || head_dim_v <= 0) return 0;
  // the workspace does not depend on the prefill launch geometry
  return plan_batch(cu, kv, num_seqs, heads, kv_heads, head_dim_v).total();
}

// Scratch of the allocation-free varlen entry: one array per device, in the
// library's code object, reached through the address hipGetSymbolAddress
// returns for the current device (the symbol's name is not a device address
// in host code).  It holds what the caller's workspace holds in
// chunk_attn_varlen: per-sequence offsets and decode partials, all written by
// the batch's own plan and decode kernels before they are read, so nothing
// needs clearing between calls.
static constexpr size_t kNoAllocScratchBytes = CHUNKATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];
static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static ca_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_EUNSUPPORTED, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the static scratch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CA_OK;
}

// ---- co-scheduling of a mixed batch ----------------------------------------------------
// The prefill part of a mixed batch is bound by the matrix cores and the
// decode part by HBM, so they can share the chip.  Measured on MI355X for a
// 2048-token chunk at past 65536 plus 256 decodes (contexts U[1024, 32768]):
// decode alone 3.16 ms on all 256 CUs and 3.58 ms on 128; prefill alone
// 1.73 ms on 256 CUs and 2.90 ms on 128 (two rounds of workgroups, at a
// higher clock when alone); both at once on disjoint halves 3.78 ms against
// 4.92 ms back to back.  Run together, the prefill half takes ~3.5 ms (the
// decode half draws power), so handing decode work to the prefill half after
// its kernel does not pay; each cross-queue event wait costs ~40-50 us.  A prefill workgroup holds 448 of a SIMD's 512 registers, so
// a decode wave cannot share its CU: the halves are CU-masked streams.
struct CoStreams {
  std::mutex mu;
  hipStream_t prefill = nullptr, decode = nullptr;
  hipEvent_t fork = nullptr, join_prefill = nullptr, join_decode = nullptr;
};
static std::mutex g_co_mu;
static CoStreams* g_co[kMaxDevices] = {};
static bool g_co_failed[kMaxDevices] = {};

// Half of the CUs, taken as CUs whose index has bit 3 clear (or set): half of
// every XCD whether mask bits map to XCDs in blocks of 32 or round-robin.
static constexpr int kMaxMaskWords = 64;   // CU masks of up to 2048 CUs
static hipError_t half_chip_stream(int n_cu, int parity, hipStream_t* s) {
  uint32_t mask[kMaxMaskWords] = {};
  const int words = (n_cu + 31) / 32;
  if (words > kMaxMaskWords) return hipErrorInvalidValue;
  for (int i = 0; i < n_cu; ++i)
    if (((i >> 3) & 1) == parity) mask[i >> 5] |= 1u << (i & 31);
  return hipExtStreamCreateWithCUMask(s, (uint32_t)words, mask);
}

// The current device's co-scheduling streams and events, made on first use;
// null (run serially) where they cannot be made.
static CoStreams* co_streams() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_co_mu);
  if (g_co[dev] || g_co_failed[dev]) return g_co[dev];
  int n_cu = 0;
  CoStreams* c = new CoStreams();
  hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && n_cu < 64) e = hipErrorNotSupported;
  if (e == hipSuccess) e = half_chip_stream(n_cu, 0, &c->prefill);
  if (e == hipSuccess) e = half_chip_stream(n_cu, 1, &c->decode);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->join_prefill, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->join_decode, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    g_co_failed[dev] = true;
    return nullptr;   // the streams and events made so far stay with the process
  }
  g_co[dev] = c;
  return c;
}

// Whether the two halves finish before the two parts would back to back:
// both parts must be sizeable, and the prefill on half the CUs (more rounds
// of its workgroups) and the decode on half the CUs must each end before the
// serial pair would.  Rates are MI355X figures for these kernels: ~1.25
// PFLOP/s prefill and ~5.8 TB/s decode on the whole chip; on half of it the
// decode runs 1.13x longer (measured), and the prefill, sharing the power
// budget with the decode, gains no clock.
static bool co_schedule_pays(const int32_t* cu, const int32_t* kv, int num_seqs, int heads, int kv_heads, int d,
                             int dv, int64_t prefill_wgs) {
  const int group = heads / kv_heads;
  double flops = 0, bytes = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t q = cu[s + 1] - cu[s];
    if (q <= 0) continue;
    if (q * group <= 32) {
      bytes += (double)kv[s] * kv_heads * (d + dv) * 2;
    } else {
      const double past = (double)(kv[s] - q);
      flops += (double)heads * (q * past + 0.5 * q * (q + 1)) * 2.0 * (d + dv);
    }
  }
  const double t_prefill = flops / 1.25e15, t_decode = bytes / 5.8e12;
  if (t_prefill < 0.2 * t_decode || t_decode < 0.2 * t_prefill) return false;
  const double rounds_full = (double)((prefill_wgs + kNumCUs - 1) / kNumCUs);
  const double rounds_half = (double)((prefill_wgs + kNumCUs / 2 - 1) / (kNumCUs / 2));
  const double t_serial = t_prefill + t_decode;
  return t_prefill * rounds_half / rounds_full < t_serial && 1.13 * t_decode < t_serial;
}

// The varlen batch, with the caller's workspace or (static_scratch) the
// library's per-device array.
static ca_status varlen_run(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                     int32_t max_blocks, int32_t num_blocks, const int32_t* cu_dev, const int32_t* kv_dev,
                     const int32_t* cu, const int32_t* kv, int32_t num_seqs, int32_t heads, int32_t kv_heads,
                     int32_t head_dim, int32_t head_dim_v, float scale, void* out, int32_t out_dtype, float* lse_out,
                     void* workspace, size_t workspace_bytes, bool static_scratch, void* stream) {
  if (!k_pool || !v_pool || !block_tables || !cu_dev || !kv_dev || !cu || !kv)
    return fail(CA_EINVAL, "null pointer argument");
  if (num_seqs > 0 && num_seqs <= 65535 && cu[num_seqs] != 0 && (!q || !out))
    return fail(CA_EINVAL, "q and out must be non-null when the batch has query rows");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
    return fail(CA_EINVAL, "q, pools and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(cu_dev, 4) || !aligned(kv_dev, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(CA_EINVAL, "int32 and fp32 arrays must be 4-byte aligned");
  if (num_seqs <= 0 || num_seqs > 65535) return fail(CA_EINVAL, "num_seqs must be in [1, 65535]");
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0 || kv_heads > 65535)
    return fail(CA_EINVAL, "heads (%d) must be a positive multiple of kv_heads (%d)", heads, kv_heads);
  if (max_blocks <= 0 || num_blocks <= 0) return fail(CA_EINVAL, "max_blocks_per_seq and num_blocks must be > 0");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(CA_EINVAL, "scale must be finite and > 0");
  if (out_dtype != CA_BF16 && out_dtype != CA_F32) return fail(CA_EINVAL, "out_dtype must be CA_BF16 or CA_F32");
  const DType dout = out_dtype == CA_F32 ? DType::F32 : DType::BF16;
  if (!prefill_supported(DType::BF16, DType::BF16, head_dim, head_dim_v) || !decode_supported(head_dim, head_dim_v))
    return fail(CA_EUNSUPPORTED, "unsupported (head_dim, head_dim_v) = (%d, %d)", head_dim, head_dim_v);
  if (cu[0] != 0) return fail(CA_EINVAL, "cu_seqlens_q[0] must be 0");
  for (int s = 0; s < num_seqs; ++s) {
    const int q_len = cu[s + 1] - cu[s];
    if (q_len < 0) return fail(CA_EINVAL, "cu_seqlens_q must be non-decreasing (sequence %d)", s);
    if (kv[s] < 0 || (q_len > 0 && kv[s] < q_len))
      return fail(CA_EINVAL, "kv_lens[%d] = %d is negative or below q_len %d", s, kv[s], q_len);
    if ((int64_t)kv[s] > (int64_t)max_blocks * kBlock)
      return fail(CA_ERANGE, "kv_lens[%d] = %d exceeds the block table (%d blocks)", s, kv[s], max_blocks);
  }
  const int64_t total_q = cu[num_seqs];
  const int group = heads / kv_heads;
  const int paged_rows = prefill_paged_rows(head_dim, head_dim_v);
  const BatchPlan plan = plan_batch(cu, kv, num_seqs, heads, kv_heads, head_dim_v);
  if (static_scratch) {
    if (plan.total() > kNoAllocScratchBytes)
      return fail(CA_EWORKSPACE, "this batch needs %zu scratch bytes; the allocation-free entry holds %zu",
                  plan.total(), kNoAllocScratchBytes);
  } else if (plan.total()) {
    if (!workspace || workspace_bytes < plan.total())
      return fail(CA_EWORKSPACE, "this batch needs %zu workspace bytes", plan.total());
    if (!aligned(workspace, 256)) return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  }
  if (plan.prefill_wgs > 0x7fffffffLL) return fail(CA_ERANGE, "launch grid too large");
  if (total_q == 0) return ok();
  if (static_scratch) {
    if (ca_status st = device_scratch(&workspace)) return st;
    workspace_bytes = kNoAllocScratchBytes;
  }

  hipStream_t st = (hipStream_t)stream;
  const float cs = scale * kLog2e;
  const int hpw = heads_per_wg(group, kWavesPaged);
  char* ws = (char*)workspace;
  DecodeArgs d{};
  d.q = q;
  d.k = k_pool;
  d.v = v_pool;
  d.block_tables = block_tables;
  d.cu_seqlens_q = cu_dev;
  d.kv_lens = kv_dev;
  d.ws_off = (int64_t*)ws;
  d.wg_off = (int64_t*)(ws + plan.ws_off_bytes);
  d.ws_o = (float*)(ws + plan.ws_off_bytes + plan.wg_off_bytes);
  d.ws_ml = (float*)(ws + plan.ws_off_bytes + plan.wg_off_bytes + plan.o_bytes);
  d.out = out;
  d.lse = lse_out;
  d.total_q = total_q;
  d.total_slots = plan.slots;
  d.num_seqs = num_seqs;
  d.max_blocks = max_blocks;
  d.num_blocks = num_blocks;
  d.heads = heads;
  d.kv_heads = kv_heads;
  d.group = group;
  d.split_tokens = plan.split_tokens;
  d.tok_wg = paged_rows / hpw;
  d.n_head_groups = heads / hpw;
  d.out_f32 = dout == DType::F32 ? 1 : 0;
  d.scale_log2 = cs;
  hipError_t e = launch_batch_plan(d, st);
  if (e != hipSuccess) return hip_status(e, "varlen plan launch");
  if (plan.n_prefill) {
    // Prefill-path sequences: one launch, straight into out.
    PrefillArgs a{};
    a.q = q;
    a.k = k_pool;
    a.v = v_pool;
    a.out = out;
    a.lse = lse_out;
    a.block_table = block_tables;
    a.lse_stride = total_q;
    a.heads = heads;
    a.kv_heads = kv_heads;
    a.group = group;
    a.num_blocks = num_blocks;
    a.hpw = hpw;
    a.n_head_groups = heads / hpw;
    a.num_splits = 1;
    a.xcd_remap = 0;
    a.scale_log2 = cs;
    a.cu_seqlens_q = cu_dev;
    a.kv_lens = kv_dev;
    a.wg_off = d.wg_off;
    a.num_seqs = num_seqs;
    a.max_blocks = max_blocks;
    if (plan.n_decode && !static_scratch &&
        co_schedule_pays(cu, kv, num_seqs, heads, kv_heads, head_dim, head_dim_v, plan.prefill_wgs)) {
      // The prefill part (matrix-bound) and the decode part (HBM-bound) run at
      // the same time on two halves of the chip; the decode half merges its
      // partials before both join the caller's stream.
      CoStreams* cs2 = co_streams();
      if (cs2) {
        std::lock_guard<std::mutex> lock(cs2->mu);
        e = hipEventRecord(cs2->fork, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(cs2->prefill, cs2->fork, 0);
        if (e == hipSuccess) e = hipStreamWaitEvent(cs2->decode, cs2->fork, 0);
        if (e == hipSuccess) e = launch_prefill_paged_varlen(dout, head_dim, head_dim_v, a, (int)plan.prefill_wgs, cs2->prefill);
        if (e == hipSuccess) e = launch_decode(head_dim, head_dim_v, d, plan.max_splits, 0, num_seqs, cs2->decode);
        if (e == hipSuccess) e = launch_decode_merge(head_dim_v, d, cs2->decode);
        if (e == hipSuccess) e = hipEventRecord(cs2->join_prefill, cs2->prefill);
        if (e == hipSuccess) e = hipEventRecord(cs2->join_decode, cs2->decode);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, cs2->join_prefill, 0);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, cs2->join_decode, 0);
        if (e != hipSuccess) return hip_status(e, "co-scheduled varlen launch");
        return ok();
      }
    }
    e = launch_prefill_paged_varlen(dout, head_dim, head_dim_v, a, (int)plan.prefill_wgs, st);
    if (e != hipSuccess) return hip_status(e, "varlen prefill launch");
  }
  if (plan.n_decode) {
    e = launch_decode(head_dim, head_dim_v, d, plan.max_splits, 0, num_seqs, st);
    if (e == hipSuccess) e = launch_decode_merge(head_dim_v, d, st);
    if (e != hipSuccess) return hip_status(e, "varlen decode launch");
  }
  return ok();
}

ca_status chunk_attn_varlen(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                            int32_t max_blocks, int32_t num_blocks, const int32_t* cu_dev, const int32_t* kv_dev,
                            const int32_t* cu, const int32_t* kv, int32_t num_seqs, int32_t heads, int32_t kv_heads,
                            int32_t head_dim, int32_t head_dim_v, float scale, void* out, int32_t out_dtype,
                            float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return varlen_run(q, k_pool, v_pool, block_tables, max_blocks, num_blocks, cu_dev, kv_dev, cu, kv, num_seqs, heads,
                    kv_heads, head_dim, head_dim_v, scale, out, out_dtype, lse_out, workspace, workspace_bytes, false,
                    stream);
}

ca_status chunk_attn_varlen_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
                                    const int32_t* cu_dev, const int32_t* kv_dev, const int32_t* cu, const int32_t* kv,
                                    int32_t num_seqs, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                    int32_t head_dim_v, float scale, void* out, int32_t out_dtype, float* lse_out,
                                    void* stream) {
  return varlen_run(q, k_pool, v_pool, block_tables, max_blocks, num_blocks, cu_dev, kv_dev, cu, kv, num_seqs, heads,
                    kv_heads, head_dim, head_dim_v, scale, out, out_dtype, lse_out, nullptr, 0, true, stream);
}

ca_status chunkattn_kv_append(const void* k_new, const void* v_new, int64_t start_pos, int64_t n_tokens,
                              int32_t kv_heads, int32_t head_dim, int32_t head_dim_v, int32_t dtype,
                              const int32_t* block_table, int32_t block_table_len, int32_t num_blocks, void* k_pool,
                              void* v_pool, const int64_t* src_strides, void* stream) {
  if (!k_new || !v_new || !block_table || !k_pool || !v_pool) return fail(CA_EINVAL, "null pointer argument");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_table, 4))
    return fail(CA_EINVAL, "misaligned pointer argument");
  if (ca_status st = check_dtype(dtype)) return st;
  if (start_pos < 0 || n_tokens < 0) return fail(CA_EINVAL, "start_pos and n_tokens must be >= 0");
  if (kv_heads <= 0 || num_blocks <= 0) return fail(CA_EINVAL, "kv_heads and num_blocks must be > 0");
  const int x = dtype == CA_BF16 ? 8 : 4;
  if (head_dim <= 0 || head_dim_v <= 0 || head_dim % x || head_dim_v % x || head_dim > 1024 || head_dim_v > 1024)
    return fail(CA_EUNSUPPORTED, "head dims must be positive multiples of %d up to 1024", x);
  if (start_pos + n_tokens > (int64_t)block_table_len * kBlock)
    return fail(CA_ERANGE, "block table covers %lld tokens, need %lld", (long long)block_table_len * kBlock,
                (long long)(start_pos + n_tokens));
  int64_t st[4] = {(int64_t)kv_heads * head_dim, head_dim, (int64_t)kv_heads * head_dim_v, head_dim_v};
  if (src_strides) {
    for (int i = 0; i < 4; ++i) {
      if (src_strides[i] <= 0 || src_strides[i] % x)
        return fail(CA_EINVAL, "src_strides[%d] = %lld must be a positive multiple of %d elements", i,
                    (long long)src_strides[i], x);
      st[i] = src_strides[i];
    }
  }
  if (n_tokens == 0) return ok();
  hipError_t e = launch_kv_append((DType)dtype, head_dim, head_dim_v, k_new, v_new, st[0], st[1], st[2], st[3],
                                  start_pos, n_tokens, kv_heads,
                                  block_table, num_blocks, k_pool, v_pool, (hipStream_t)stream);
  return hip_status(e, "kv_append launch");
}

size_t chunkattn_mla_block_bytes(int32_t format) {
  return format == CA_MLA_BF16 ? (size_t)kMlaBf16Block : (format == CA_MLA_FP8 ? (size_t)kMlaFp8Block : 0);
}

size_t chunkattn_mla_decode_workspace_size(const int32_t* kv_lens_host, int32_t num_seqs, int32_t heads,
                                           int32_t format) {
  if (check_mla(kv_lens_host, num_seqs, heads, 1 << 24, format) != CA_OK || num_seqs == 0) return 0;
  return plan_mla(kv_lens_host, num_seqs, heads, format == CA_MLA_FP8).bytes;
}

ca_status chunkattn_mla_kv_append(const void* latent, const void* rope, int64_t start_pos, int64_t n_tokens,
                                  int32_t format, const int32_t* block_table, int32_t block_table_len,
                                  int32_t num_blocks, void* pool, void* stream) {
  if (format != CA_MLA_BF16 && format != CA_MLA_FP8) return fail(CA_EINVAL, "unknown MLA cache format %d", format);
  if (start_pos < 0 || n_tokens < 0) return fail(CA_EINVAL, "start_pos and n_tokens must be >= 0");
  if (n_tokens == 0) return ok();
  if (!latent || !rope || !block_table || !pool) return fail(CA_EINVAL, "null pointer argument");
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(pool, 16) || !aligned(block_table, 4))
    return fail(CA_EINVAL, "misaligned pointer argument");
  if (num_blocks <= 0) return fail(CA_EINVAL, "num_blocks must be > 0");
  if (start_pos + n_tokens > (int64_t)block_table_len * kBlock)
    return fail(CA_ERANGE, "block table covers %lld tokens, need %lld", (long long)block_table_len * kBlock,
                (long long)(start_pos + n_tokens));
  MlaAppendArgs a;
  a.latent = (const uint16_t*)latent;
  a.rope = (const uint16_t*)rope;
  a.block_table = block_table;
  a.pool = (unsigned char*)pool;
  a.start_pos = start_pos;
  a.n_tokens = n_tokens;
  a.num_blocks = num_blocks;
  return hip_status(launch_mla_append(format == CA_MLA_FP8, a, (hipStream_t)stream), "MLA append launch");
}

ca_status chunk_mla_decode(const void* q, const void* pool, int32_t format, const int32_t* block_tables,
                           int32_t max_blocks, int32_t num_blocks, const int32_t* kv_lens_dev,
                           const int32_t* kv_lens_host, int32_t num_seqs, int32_t heads, float scale, void* out,
                           int32_t out_dtype, float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (max_blocks <= 0 || num_blocks <= 0) return fail(CA_EINVAL, "max_blocks and num_blocks must be > 0");
  if (out_dtype != CA_BF16 && out_dtype != CA_F32) return fail(CA_EINVAL, "out_dtype must be CA_BF16 or CA_F32");
  if (ca_status st = check_mla(kv_lens_host, num_seqs, heads, max_blocks, format)) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CA_EINVAL, "scale must be finite and > 0");
  if (num_seqs == 0) return ok();
  if (!q || !pool || !block_tables || !kv_lens_dev || !out) return fail(CA_EINVAL, "null pointer argument");
  if (!aligned(q, 16) || !aligned(pool, 16) || !aligned(out, 16) || !aligned(block_tables, 4) ||
      !aligned(kv_lens_dev, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(CA_EINVAL, "misaligned pointer argument");
  const MlaPlan p = plan_mla(kv_lens_host, num_seqs, heads, format == CA_MLA_FP8);
  // keeps unit * steps products in int64 and the launch grid in int32
  if (p.steps > (int64_t)1 << 31 || p.units * (heads / 16) > 0x7fffffffLL)
    return fail(CA_ERANGE, "the batch holds %lld key steps, too many for one call", (long long)p.steps);
  if (!workspace || workspace_bytes < p.bytes)
    return fail(CA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.bytes, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  MlaArgs a;
  a.q = (const uint16_t*)q;
  a.pool = (const unsigned char*)pool;
  a.block_tables = block_tables;
  a.kv_lens = kv_lens_dev;
  a.seq_steps = (int64_t*)workspace;
  a.unit_seq = (int32_t*)((char*)workspace + p.unit_off);
  a.ws_ml = (float*)((char*)workspace + p.ml_off);
  a.ws_o = (float*)((char*)workspace + p.o_off);
  a.out = out;
  a.out_f32 = out_dtype == CA_F32 ? 1 : 0;
  a.lse = lse_out;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.heads = heads;
  a.units = (int32_t)p.units;
  a.slots = (int32_t)p.slots;
  a.scale_log2 = scale * kLog2e;
  return hip_status(launch_mla_decode(format == CA_MLA_FP8, a, (hipStream_t)stream), "MLA decode launch");
}

size_t chunkattn_mla_prefill_workspace_size(int64_t past_len, int64_t chunk_len, int32_t format) {
  if ((format != CA_MLA_BF16 && format != CA_MLA_FP8) || past_len < 0 || chunk_len < 0 ||
      past_len + chunk_len > ((int64_t)1 << 30))
    return 0;
  return (size_t)mla_prefill_staging_bytes(format == CA_MLA_FP8, past_len + chunk_len);
}

ca_status chunk_mla_prefill(const void* q, const void* pool, int32_t format, const int32_t* block_table,
                            int32_t block_table_len, int32_t num_blocks, int64_t past_len, int64_t chunk_len,
                            int32_t heads, float scale, void* out, int32_t out_dtype, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (format != CA_MLA_BF16 && format != CA_MLA_FP8) return fail(CA_EINVAL, "unknown MLA cache format %d", format);
  if (heads <= 0 || heads % 16 || heads > 1024)
    return fail(CA_EUNSUPPORTED, "heads must be a positive multiple of 16 up to 1024, got %d", heads);
  if (past_len < 0 || chunk_len < 0) return fail(CA_EINVAL, "past_len and chunk_len must be >= 0");
  if (out_dtype != CA_BF16 && out_dtype != CA_F32) return fail(CA_EINVAL, "out_dtype must be CA_BF16 or CA_F32");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CA_EINVAL, "scale must be finite and > 0");
  if (num_blocks <= 0) return fail(CA_EINVAL, "num_blocks must be > 0");
  // positions, row blocks and the grid stay in 32-bit ranges
  if (past_len + chunk_len > ((int64_t)1 << 30) || chunk_len * (heads / 16) > ((int64_t)1 << 31) - 8)
    return fail(CA_ERANGE, "past_len + chunk_len = %lld is too long", (long long)(past_len + chunk_len));
  if (chunk_len == 0) return ok();
  if ((int64_t)block_table_len * kBlock < past_len + chunk_len)
    return fail(CA_ERANGE, "block table covers %lld tokens, need %lld", (long long)block_table_len * kBlock,
                (long long)(past_len + chunk_len));
  if (!q || !pool || !block_table || !out) return fail(CA_EINVAL, "null pointer argument");
  if (!aligned(q, 16) || !aligned(pool, 16) || !aligned(out, 16) || !aligned(block_table, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return fail(CA_EINVAL, "misaligned pointer argument");
  const size_t need = (size_t)mla_prefill_staging_bytes(format == CA_MLA_FP8, past_len + chunk_len);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (need && !aligned(workspace, 256)) return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  MlaPrefillArgs a;
  a.q = (const uint16_t*)q;
  a.pool = (const unsigned char*)pool;
  a.block_table = block_table;
  a.out = out;
  a.lse = lse_out;
  a.past_len = past_len;
  a.chunk_len = chunk_len;
  a.num_blocks = num_blocks;
  a.heads = heads;
  a.out_f32 = out_dtype == CA_F32 ? 1 : 0;
  a.scale_log2 = scale * kLog2e;
  return hip_status(launch_mla_prefill(format == CA_MLA_FP8, a, workspace, (hipStream_t)stream), "MLA prefill launch");
}

}  // extern "C"
