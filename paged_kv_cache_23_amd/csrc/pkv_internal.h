// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;    // default tokens per cache block (also 32 ... 256)
constexpr int kChunkTokens = 32;    // tokens one wave consumes per step: two blocks
constexpr int kDecodeWaves = 4;     // worker waves per decode workgroup
constexpr int kMaxGroup = 16;       // query heads per kv head that one MFMA column tile holds
constexpr int kWavesPerSimd = 1;    // worker waves per SIMD: a second one mostly waits on the first
// Prefix columns one wave of the one-launch shared-prefix decode owns (two
// 16-column MFMA tiles), and one workgroup's four prefix waves together.
constexpr int shared_group_cols(int) { return 32; }
constexpr int shared_workgroup_cols(int head_dim) { return 4 * shared_group_cols(head_dim); }

enum KvType : int32_t { kF32 = 0, kBF16 = 1, kFP8 = 2 };

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  void* out;
  float* ws_acc;   // [num_workers + pairs][cols][head_dim]  partial accumulators
  float* ws_ml;    // [num_workers + pairs][cols][2]         (max in log2 units, sum)
  int2* pair_meta;      // [pairs] (first wave, parts) of each non-empty pair
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_context_len;
  int32_t block_size;    // tokens per block: 16, 32, 64, 128 or 256
  int32_t block_shift;   // log2(block_size)
  int32_t kv_reread;     // blocks are read more than once per call: keep K/V cached
  int32_t q_len;         // query tokens per sequence (1 for decode)
  int32_t cols;          // q_len * group: query columns per (sequence, kv head) pair
  int32_t num_workers;   // decode worker waves; a multiple of kDecodeWaves
  int32_t kv_dtype;
  float scale;
  // Shared-prefix decode (all zero otherwise).
  int32_t table_offset;   // tail pass: prefix blocks (block_tables points past them)
  int32_t tail_pass;      // split kernel: tail pass (lengths minus the prefix, every pair leaves partials)
  // merge input: prefix partial accumulators [pre_segments][num_seqs * num_q_heads][head_dim],
  // in the output's type (float32 for a float32 cache, else bf16)
  void* pre_acc;
  float* pre_ml;          // [pre_segments][num_seqs * num_q_heads][2]  (max in log2 units, sum)
  int32_t pre_segments;   // merge: prefix pieces per column; prefill kernel: key segments
  int32_t prefix_tokens;  // prefill kernel in prefix mode: keys every column sees
  int32_t prefix_mode;    // prefill kernel: columns are the batch's query heads, output partials
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  const float* k_scale;
  const float* v_scale;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t block_size;
  int32_t kv_dtype;
};

struct CopyArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* src;
  const int32_t* dst;
  size_t block_bytes;          // bytes of one block in one pool (all kv heads)
  int32_t num_pairs;
  int32_t num_blocks;
  uint32_t slices_per_block;   // 8 KiB slices per block and pool
};

// Split kernel then merge kernel, on `stream` (cols <= kMaxGroup).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Many-query kernel (cols > kMaxGroup): one workgroup per tile of columns
// of a (sequence, kv head) pair; uses no workspace.
hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream);
// Workgroups launch_prefill starts for these arguments.
int64_t prefill_groups(const DecodeArgs& a);
// Query columns one prefill workgroup owns.
int prefill_group_cols(int kv_dtype);
// Split kernel alone, then merge kernel alone (shared-prefix decode runs the
// prefix pass between them).
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream);
// Shared-prefix decode, tail walk and prefix part in one launch (bf16
// caches): num_workers / 4 eight-wave workgroups; the prefix partials go to
// pre_acc / pre_ml in pre_segments key segments per column.  A merge kernel
// launched after it finishes every pair.
hipError_t launch_shared(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// The library's static decode workspace: kStaticScratchBytes of device memory
// per device, at the address static_scratch() returns for the current device
// (nullptr if the runtime cannot resolve it).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
void* static_scratch();
hipError_t launch_copy(const CopyArgs& a, hipStream_t stream);
size_t copy_slice_bytes();

}  // namespace pkv
