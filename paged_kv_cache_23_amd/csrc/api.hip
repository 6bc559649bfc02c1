// C ABI of libpkv: host-side argument checks, worker count, workspace layout
// and kernel dispatch.  Declarations and contracts: include/pkv.h.

#include "pkv.h"
#include "pkv_internal.h"

#include <stdint.h>

#include <atomic>

namespace {

using pkv::DecodeArgs;

constexpr size_t kWsAlign = 256;
static_assert(pkv::kStaticScratchBytes == PKV_STATIC_SCRATCH_BYTES, "static scratch size in pkv.h");

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// log2 of a supported block size (16, 32, 64, 128, 256), else -1.
int block_shift(int32_t bs) {
  for (int s = 4; s <= 8; ++s)
    if (bs == (1 << s)) return s;
  return -1;
}

int check_desc(const pkv_cache_desc* d) {
  if (!d) return PKV_EINVAL;
  if (d->num_blocks <= 0 || d->num_kv_heads <= 0 || d->num_q_heads <= 0 || d->head_dim <= 0)
    return PKV_EINVAL;
  if (block_shift(d->block_size) < 0) return PKV_EINVAL;
  if (d->flags & ~PKV_KV_REREAD) return PKV_EINVAL;
  if (d->num_q_heads % d->num_kv_heads != 0) return PKV_EINVAL;
  if (d->num_q_heads / d->num_kv_heads > pkv::kMaxGroup) return PKV_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_EUNSUPPORTED;
  const int kv = d->kv_dtype, qd = d->q_dtype;
  if (kv < PKV_F32 || kv > PKV_FP8_E4M3 || qd < PKV_F32 || qd > PKV_FP8_E4M3) return PKV_EINVAL;
  const bool ok = (kv == PKV_F32 && qd == PKV_F32) || (kv == PKV_BF16 && qd == PKV_BF16) ||
                  (kv == PKV_FP8_E4M3 && qd == PKV_BF16);
  if (!ok) return PKV_EUNSUPPORTED;
  if (kv == PKV_FP8_E4M3) {
    if (!d->k_scale || !d->v_scale) return PKV_EINVAL;
  } else if (d->k_scale || d->v_scale) {
    return PKV_EINVAL;
  }
  return PKV_OK;
}

// Compute units of the current device, cached per device (the value never
// changes while the process runs).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Default number of worker waves: one per SIMD (4 per compute unit), all
// resident at once; no more than there can be 32-token chunks in the batch.
// With two per SIMD the second wave mostly waits for the first one's memory
// traffic and only adds split pairs (measured slower on MI355X).
int32_t default_workers(const pkv_cache_desc* d, int32_t num_seqs, int32_t max_ctx) {
  const int cus = device_cus();
  if (cus <= 0) return PKV_ELAUNCH;
  const int64_t full = (int64_t)cus * 4 * pkv::kWavesPerSimd;
  const int64_t chunks = (int64_t)num_seqs * d->num_kv_heads *
                         (((int64_t)max_ctx + pkv::kChunkTokens - 1) / pkv::kChunkTokens);
  int64_t w = chunks < full ? chunks : full;
  w = (w + pkv::kDecodeWaves - 1) / pkv::kDecodeWaves * pkv::kDecodeWaves;
  return (int32_t)(w < pkv::kDecodeWaves ? pkv::kDecodeWaves : w);
}

int32_t resolve_workers(const pkv_cache_desc* d, int32_t num_seqs, int32_t max_ctx, int32_t workers) {
  if (workers == 0) return default_workers(d, num_seqs, max_ctx);
  if (workers < 0 || workers % pkv::kDecodeWaves != 0 || workers > (1 << 24)) return PKV_EINVAL;
  return workers;
}

// Workspace: partial accumulators, then (max, sum) pairs, then one (first
// wave, parts) record per (sequence, kv head) pair; each region starts on a
// 256-byte boundary.
size_t align_up(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Partial-state rows: (workers + pairs) pieces of q_len * group columns.
size_t partial_rows(const pkv_cache_desc* d, int32_t num_seqs, int32_t q_len, int32_t workers) {
  return ((size_t)workers + (size_t)num_seqs * d->num_kv_heads) * (size_t)q_len *
         (d->num_q_heads / d->num_kv_heads);
}

size_t acc_bytes(const pkv_cache_desc* d, int32_t num_seqs, int32_t q_len, int32_t workers) {
  return align_up(partial_rows(d, num_seqs, q_len, workers) * d->head_dim * sizeof(float));
}

size_t ml_bytes(const pkv_cache_desc* d, int32_t num_seqs, int32_t q_len, int32_t workers) {
  return align_up(partial_rows(d, num_seqs, q_len, workers) * 2 * sizeof(float));
}

size_t workspace_bytes(const pkv_cache_desc* d, int32_t num_seqs, int32_t q_len, int32_t workers) {
  return acc_bytes(d, num_seqs, q_len, workers) + ml_bytes(d, num_seqs, q_len, workers) +
         align_up((size_t)num_seqs * d->num_kv_heads * 2 * sizeof(int32_t));
}

// Query columns (query token, head) per (sequence, kv head) pair.
int64_t query_cols(const pkv_cache_desc* d, int32_t q_len) {
  return (int64_t)q_len * (d->num_q_heads / d->num_kv_heads);
}

// Up to 16 columns share one MFMA column tile and run on the split decode
// kernels; more run on the many-query (prefill) kernel.
bool many_queries(const pkv_cache_desc* d, int32_t q_len) { return query_cols(d, q_len) > pkv::kMaxGroup; }

constexpr int64_t kMaxCols = int64_t(1) << 24;

int check_q_len(const pkv_cache_desc* d, int32_t q_len) {
  if (q_len < 1) return PKV_EINVAL;
  if (query_cols(d, q_len) > kMaxCols) return PKV_EUNSUPPORTED;
  return PKV_OK;
}

int check_decode_args(const pkv_cache_desc* d, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                      int32_t num_seqs, int32_t max_ctx, const void* out) {
  int st = check_desc(d);
  if (st != PKV_OK) return st;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PKV_EINVAL;
  if (num_seqs < 0 || max_blocks <= 0 || max_ctx < 0) return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PKV_EINVAL;
  return PKV_OK;
}

DecodeArgs make_args(const pkv_cache_desc* d, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                     int32_t num_seqs, int32_t q_len, int32_t max_ctx, float scale, int32_t workers, void* out,
                     void* workspace) {
  DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_scale = d->k_scale;
  a.v_scale = d->v_scale;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.q_len = q_len;
  a.cols = q_len * a.group;
  a.block_size = d->block_size;
  a.block_shift = block_shift(d->block_size);
  a.kv_reread = (d->flags & PKV_KV_REREAD) ? 1 : 0;
  a.head_dim = d->head_dim;
  a.max_blocks = max_blocks;
  a.num_blocks = d->num_blocks;
  a.max_context_len = max_ctx;
  a.num_workers = workers;
  a.kv_dtype = d->kv_dtype;
  a.scale = scale;
  if (!workspace) return a;   // the prefill kernel takes none
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + acc_bytes(d, num_seqs, q_len, workers));
  a.pair_meta = reinterpret_cast<int2*>(ws + acc_bytes(d, num_seqs, q_len, workers) +
                                        ml_bytes(d, num_seqs, q_len, workers));
  return a;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

// Shared-prefix decode: key segments of the prefix pass.  About one
// workgroup per compute unit (each segment adds a float32 partial per query
// head that is written and read back), at least kMinSegChunks chunks of 32
// keys per segment, and no segment left empty.
constexpr int64_t kSegGroupsPerCu = 1;
constexpr int64_t kMinSegChunks = 4;

int32_t prefix_segments(const pkv_cache_desc* d, int32_t num_seqs, int32_t prefix_tokens) {
  const int cus = device_cus();
  if (cus <= 0) return PKV_ELAUNCH;
  const int64_t cols = (int64_t)num_seqs * (d->num_q_heads / d->num_kv_heads);
  const int64_t gc = pkv::prefill_group_cols(d->kv_dtype);
  const int64_t groups = (cols + gc - 1) / gc * d->num_kv_heads;
  if (groups == 0) return 1;   // no sequences: one (empty) segment
  const int64_t chunks = ((int64_t)prefix_tokens + pkv::kChunkTokens - 1) / pkv::kChunkTokens;
  int64_t s = (kSegGroupsPerCu * cus + groups - 1) / groups;
  const int64_t cap = chunks / kMinSegChunks;
  if (s > cap) s = cap;
  if (s > 1024) s = 1024;
  if (s < 1) s = 1;
  const int64_t per = (chunks + s - 1) / s;   // the kernel's chunks per segment
  return (int32_t)((chunks + per - 1) / per);
}

// Prefix partials after the decode workspace: accumulators [S][B*Hq][D] in
// the output's type (the merge's other inputs are float32; the prefix
// partials are the bulk of what it reads), then float32 (max, sum) pairs
// [S][B*Hq][2].
// One-launch shared-prefix decode (the tail walk and the prefix part share
// every SIMD): taken when the tails alone give every SIMD a tail wave and the
// cache is bf16; otherwise the prefix pass runs on the prefill kernel before
// the tail walk.
bool shared_one_launch(const pkv_cache_desc* d, int32_t workers) {
  if (d->kv_dtype != PKV_BF16) return false;
  const int cus = device_cus();
  return cus > 0 && workers == (int64_t)cus * 4 * pkv::kWavesPerSimd;
}

// Key segments of the shared-prefix decode for `workers` tail waves.  In one
// launch: about one (kv head, workgroup's column groups, segment) item per
// workgroup (workers / 4 of them), at least kMinSegChunks chunks per
// segment, none empty.
int32_t shared_segments(const pkv_cache_desc* d, int32_t num_seqs, int32_t prefix_tokens, int32_t workers) {
  if (!shared_one_launch(d, workers)) return prefix_segments(d, num_seqs, prefix_tokens);
  const int64_t cols = (int64_t)num_seqs * (d->num_q_heads / d->num_kv_heads);
  const int64_t gc = pkv::shared_workgroup_cols(d->head_dim);
  const int64_t groups = (cols + gc - 1) / gc * d->num_kv_heads;
  if (groups == 0) return 1;   // no sequences: one (empty) segment
  const int64_t chunks = ((int64_t)prefix_tokens + pkv::kChunkTokens - 1) / pkv::kChunkTokens;
  int64_t s = workers / pkv::kDecodeWaves / groups;
  const int64_t cap = chunks / kMinSegChunks;
  if (s > cap) s = cap;
  if (s > 1024) s = 1024;
  if (s < 1) s = 1;
  const int64_t per = (chunks + s - 1) / s;   // the kernel's chunks per segment
  return (int32_t)((chunks + per - 1) / per);
}

size_t prefix_acc_bytes(const pkv_cache_desc* d, int32_t num_seqs, int32_t segments) {
  const size_t elt = d->kv_dtype == PKV_F32 ? 4 : 2;
  return align_up((size_t)segments * num_seqs * d->num_q_heads * d->head_dim * elt);
}
size_t prefix_ml_bytes(const pkv_cache_desc* d, int32_t num_seqs, int32_t segments) {
  return align_up((size_t)segments * num_seqs * d->num_q_heads * 2 * sizeof(float));
}

// Shared-prefix decode pays off once the prefix bytes that the plain decode
// would read again (num_seqs - 1 more times) outweigh its two extra launches
// and the partials it writes: measured on MI355X with 32 q / 8 kv heads,
// head_dim 128, bf16, the cascade is faster from about 190 MB of avoided
// re-reads (2,000-token prefix: 32 sequences; 4,096: 16), slower below.
constexpr double kSharedMinSavedBytes = 192.0 * 1024 * 1024;

// The decode's tail part only reads the tokens after the prefix.
int32_t tail_ctx(int32_t max_ctx, int32_t prefix_tokens) {
  return max_ctx > prefix_tokens ? max_ctx - prefix_tokens : 0;
}

// The prefix is whole blocks of the table, and no longer than the caller's
// bound on the lengths (every sequence holds at least the prefix).
int check_prefix(const pkv_cache_desc* d, int32_t prefix_tokens, int32_t max_blocks, int32_t max_ctx) {
  if (prefix_tokens < 0 || prefix_tokens % d->block_size != 0) return PKV_EINVAL;
  if (prefix_tokens / d->block_size > max_blocks || prefix_tokens > max_ctx) return PKV_EINVAL;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_kv_append(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int32_t num_tokens, void* k_pool, void* v_pool,
                  void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool) return PKV_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool)) return PKV_EINVAL;
  pkv::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  a.num_tokens = num_tokens;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.num_blocks = desc->num_blocks;
  a.block_size = desc->block_size;
  a.kv_dtype = desc->kv_dtype;
  return launch_status(pkv::launch_append(a, static_cast<hipStream_t>(stream)));
}

int pkv_copy_blocks(const pkv_cache_desc* desc, void* k_pool, void* v_pool, const int32_t* src,
                    const int32_t* dst, int32_t num_pairs, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_EINVAL;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_EINVAL;
  const size_t elt = desc->kv_dtype == PKV_F32 ? 4 : desc->kv_dtype == PKV_BF16 ? 2 : 1;
  pkv::CopyArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.src = src;
  a.dst = dst;
  a.block_bytes = (size_t)desc->num_kv_heads * desc->block_size * desc->head_dim * elt;
  a.num_pairs = num_pairs;
  a.num_blocks = desc->num_blocks;
  const size_t slice = pkv::copy_slice_bytes();
  a.slices_per_block = (uint32_t)((a.block_bytes + slice - 1) / slice);
  if ((uint64_t)num_pairs * 2u * a.slices_per_block > 0x7FFFFFFFu) return PKV_EUNSUPPORTED;
  return launch_status(pkv::launch_copy(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_decode_workers(const pkv_cache_desc* desc, int32_t num_seqs, int32_t max_context_len) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len < 0) return PKV_EINVAL;
  return default_workers(desc, num_seqs, max_context_len);
}

size_t pkv_attention_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs, int32_t q_len,
                                     int32_t max_context_len, int32_t num_workers) {
  if (check_desc(desc) != PKV_OK || num_seqs < 0 || max_context_len < 0) return 0;
  if (check_q_len(desc, q_len) != PKV_OK) return 0;
  const int32_t w = resolve_workers(desc, num_seqs, max_context_len, num_workers);
  if (w <= 0) return 0;
  if (many_queries(desc, q_len)) return kWsAlign;   // nominal: the prefill kernel needs none
  return workspace_bytes(desc, num_seqs, q_len, w);
}

size_t pkv_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs, int32_t max_context_len,
                                  int32_t num_workers) {
  return pkv_attention_workspace_bytes(desc, num_seqs, 1, max_context_len, num_workers);
}

int pkv_paged_attention(const pkv_cache_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t q_len, int32_t max_context_len, float scale, int32_t num_workers,
                        void* out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_decode_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, max_context_len, out);
  if (st != PKV_OK) return st;
  st = check_q_len(desc, q_len);
  if (st != PKV_OK) return st;
  const int32_t w = resolve_workers(desc, num_seqs, max_context_len, num_workers);
  if (w <= 0) return w == 0 ? PKV_EINVAL : w;
  if (num_seqs == 0) return PKV_OK;
  if (many_queries(desc, q_len)) {
    DecodeArgs a = make_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                             q_len, max_context_len, scale, w, out, nullptr);
    if (pkv::prefill_groups(a) > 0x7FFFFFFF) return PKV_EUNSUPPORTED;
    return launch_status(pkv::launch_prefill(a, static_cast<hipStream_t>(stream)));
  }
  if (!workspace || ws_bytes < workspace_bytes(desc, num_seqs, q_len, w)) return PKV_EWORKSPACE;
  if (!aligned16(workspace)) return PKV_EINVAL;
  DecodeArgs a = make_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                           q_len, max_context_len, scale, w, out, workspace);
  return launch_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int pkv_paged_decode_ex(const pkv_cache_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_context_len, float scale, int32_t num_workers, void* out,
                        void* workspace, size_t ws_bytes, void* stream) {
  return pkv_paged_attention(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs, 1,
                             max_context_len, scale, num_workers, out, workspace, ws_bytes, stream);
}

int pkv_paged_decode(const pkv_cache_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t max_context_len, float scale, void* out, void* workspace,
                     size_t ws_bytes, void* stream) {
  return pkv_paged_decode_ex(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                             max_context_len, scale, 0, out, workspace, ws_bytes, stream);
}

int pkv_paged_decode_static(const pkv_cache_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, float scale, void* out, void* stream) {
  int st = check_decode_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                             max_context_len, out);
  if (st != PKV_OK) return st;
  const int32_t w = resolve_workers(desc, num_seqs, max_context_len, 0);
  if (w <= 0) return w == 0 ? PKV_EINVAL : w;
  if (num_seqs == 0) return PKV_OK;
  if (workspace_bytes(desc, num_seqs, 1, w) > pkv::kStaticScratchBytes) return PKV_ESCRATCH;
  void* scratch = pkv::static_scratch();
  if (!scratch) return PKV_ELAUNCH;
  DecodeArgs a = make_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs, 1,
                           max_context_len, scale, w, out, scratch);
  return launch_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_shared_prefix_pays(const pkv_cache_desc* desc, int32_t num_seqs, int32_t prefix_tokens) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || prefix_tokens < 0) return PKV_EINVAL;
  if (num_seqs < 2 || prefix_tokens == 0) return 0;
  const double elt = desc->kv_dtype == PKV_F32 ? 4.0 : desc->kv_dtype == PKV_BF16 ? 2.0 : 1.0;
  const double per_token = 2.0 * desc->num_kv_heads * desc->head_dim * elt;   // K and V
  return (double)(num_seqs - 1) * prefix_tokens * per_token >= kSharedMinSavedBytes ? 1 : 0;
}

size_t pkv_shared_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs, int32_t max_context_len,
                                         int32_t prefix_tokens, int32_t num_workers) {
  if (check_desc(desc) != PKV_OK || num_seqs < 0 || max_context_len < 0 || prefix_tokens < 0) return 0;
  if (prefix_tokens % desc->block_size != 0 || prefix_tokens > max_context_len) return 0;
  const int32_t w = resolve_workers(desc, num_seqs, tail_ctx(max_context_len, prefix_tokens), num_workers);
  if (w <= 0) return 0;
  const int32_t s = prefix_tokens > 0 ? shared_segments(desc, num_seqs, prefix_tokens, w) : 0;
  if (s < 0) return 0;
  return workspace_bytes(desc, num_seqs, 1, w) + prefix_acc_bytes(desc, num_seqs, s) +
         prefix_ml_bytes(desc, num_seqs, s);
}

int pkv_paged_decode_shared(const pkv_cache_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t prefix_tokens, float scale,
                            int32_t num_workers, void* out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_decode_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                             max_context_len, out);
  if (st != PKV_OK) return st;
  st = check_prefix(desc, prefix_tokens, max_blocks_per_seq, max_context_len);
  if (st != PKV_OK) return st;
  if (prefix_tokens == 0)
    return pkv_paged_decode_ex(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                               max_context_len, scale, num_workers, out, workspace, ws_bytes, stream);
  const int32_t tctx = tail_ctx(max_context_len, prefix_tokens);
  const int32_t w = resolve_workers(desc, num_seqs, tctx, num_workers);
  if (w <= 0) return w == 0 ? PKV_EINVAL : w;
  if (num_seqs == 0) return PKV_OK;
  const int32_t segs = shared_segments(desc, num_seqs, prefix_tokens, w);
  if (segs < 0) return segs;
  const size_t dec = workspace_bytes(desc, num_seqs, 1, w);
  if (!workspace || ws_bytes < dec + prefix_acc_bytes(desc, num_seqs, segs) + prefix_ml_bytes(desc, num_seqs, segs))
    return PKV_EWORKSPACE;
  if (!aligned16(workspace)) return PKV_EINVAL;
  char* ws = static_cast<char*>(workspace);
  void* pre_acc = ws + dec;
  float* pre_ml = reinterpret_cast<float*>(ws + dec + prefix_acc_bytes(desc, num_seqs, segs));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t pblocks = prefix_tokens / desc->block_size;

  if (shared_one_launch(desc, w)) {
    // the tail walk (every sequence's tokens after the prefix, all as
    // partials) and the prefix part in one launch, then the merge
    DecodeArgs ta = make_args(desc, q, k_pool, v_pool, block_tables + pblocks, max_blocks_per_seq, context_lens,
                              num_seqs, 1, max_context_len, scale, w, out, workspace);
    ta.table_offset = pblocks;
    ta.tail_pass = 1;
    ta.prefix_tokens = prefix_tokens;
    ta.pre_segments = segs;
    ta.pre_acc = pre_acc;
    ta.pre_ml = pre_ml;
    return launch_status(pkv::launch_shared(ta, s));
  }

  // 1. the prefix for every sequence at once: one virtual sequence whose
  //    query tokens are the batch's sequences, over row 0's prefix blocks
  DecodeArgs pa = make_args(desc, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, 1, num_seqs,
                            max_context_len, scale, w, out, nullptr);
  pa.prefix_mode = 1;
  pa.prefix_tokens = prefix_tokens;
  pa.pre_segments = segs;
  pa.pre_acc = pre_acc;
  pa.pre_ml = pre_ml;
  if (pkv::prefill_groups(pa) > 0x7FFFFFFF) return PKV_EUNSUPPORTED;
  hipError_t e = pkv::launch_prefill(pa, s);
  if (e != hipSuccess) return PKV_ELAUNCH;
  // 2. every sequence's own tokens after the prefix, all as partials
  //    (each row read from its first block after the prefix; the row stride
  //    stays max_blocks_per_seq)
  DecodeArgs ta = make_args(desc, q, k_pool, v_pool, block_tables + pblocks, max_blocks_per_seq, context_lens,
                            num_seqs, 1, max_context_len, scale, w, out, workspace);
  ta.table_offset = pblocks;
  ta.tail_pass = 1;
  e = pkv::launch_split(ta, s);
  if (e != hipSuccess) return PKV_ELAUNCH;
  // 3. merge the tail pieces with the prefix segments
  ta.pre_acc = pre_acc;
  ta.pre_ml = pre_ml;
  ta.pre_segments = segs;
  return launch_status(pkv::launch_merge(ta, s));
}

const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported dtype, head_dim or group size";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_ELAUNCH: return "HIP launch failed";
    case PKV_ENOSPACE: return "not enough free blocks";
    case PKV_ESCRATCH: return "the decode needs more than the library's static 32 MiB scratch buffer";
    default: return "unknown status";
  }
}

const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

}  // extern "C"
