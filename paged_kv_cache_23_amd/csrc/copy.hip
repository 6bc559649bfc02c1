// Block copy for copy-on-write.
//
// Habr KV-Cache article (habr.com/ru/articles/1021832), section 4,
// subsection "Copy-on-Write for parallel sampling": sequences share blocks
// through reference counts; one that must modify a shared block gets a copy
// first and the original stays as it is.  Section 8 applies the same rule
// to a speculative correction inside a shared block.  The host allocator
// picks the fresh block; this kernel moves the bytes.
//
// A block of one pool is num_kv_heads tiles of 16 x head_dim elements, one
// contiguous run (16 * head_dim * bytes per element is a multiple of 1 KiB).
// One workgroup copies one 8 KiB slice of one pool's block for one pair:
// every lane moves two 16-byte vectors, loads first, then stores.  The copy
// is HBM-bound: it reads and writes 2 * num_kv_heads * 16 * head_dim
// elements per pair.

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr size_t kSliceBytes = 2 * 16 * kCopyThreads;   // 8 KiB per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a, const int32_t* __restrict__ src,
                                                                   const int32_t* __restrict__ dst) {
  const unsigned per_pool = a.slices_per_block;
  const unsigned pair = blockIdx.x / (2 * per_pool);
  const unsigned rest = blockIdx.x % (2 * per_pool);
  const unsigned pool = rest / per_pool;
  const unsigned slice = rest % per_pool;
  const int s = src[pair];
  const int d = dst[pair];
  if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks) return;   // skipped pair
  uint8_t* base = static_cast<uint8_t*>(pool ? a.v_pool : a.k_pool);
  const size_t lo = (size_t)slice * kSliceBytes;
  const u32x4* from = reinterpret_cast<const u32x4*>(base + (size_t)s * a.block_bytes + lo);
  u32x4* to = reinterpret_cast<u32x4*>(base + (size_t)d * a.block_bytes + lo);
  const size_t n = min(kSliceBytes, a.block_bytes - lo) / 16;   // vectors in this slice
  const unsigned i0 = threadIdx.x, i1 = threadIdx.x + kCopyThreads;
  u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
  // bytes pass through once: non-temporal loads and stores keep them out of the caches
  if (i0 < n) v0 = __builtin_nontemporal_load(from + i0);
  if (i1 < n) v1 = __builtin_nontemporal_load(from + i1);
  if (i0 < n) __builtin_nontemporal_store(v0, to + i0);
  if (i1 < n) __builtin_nontemporal_store(v1, to + i1);
}

}  // namespace

hipError_t launch_copy(const CopyArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_pairs * 2u * a.slices_per_block;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(kCopyThreads), 0, stream, a, a.src, a.dst);
  return hipGetLastError();
}

size_t copy_slice_bytes() { return kSliceBytes; }

}  // namespace pkv
