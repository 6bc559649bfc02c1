// Paged decode attention for gfx950: stream-K split kernel + merge kernel.
//
// What is computed (Habr KV-Cache article, habr.com/ru/articles/1021832):
//  - section 3 "Recalling FlashAttention": exact softmax(q K^T * scale) V,
//    evaluated tile by tile with a running max m and running sum l, earlier
//    partial results rescaled by exp(m_old - m_new) when the max grows;
//  - section 4 "Recalling PagedAttention": K and V of a sequence live in
//    16-token blocks scattered over a pool, found through the block table;
//  - section 5 "How vLLM combines FlashAttention and PagedAttention": one
//    fused kernel gathers the scattered blocks itself and attends;
//  - section 2 "GQA: 8x reduction": several query heads share one kv head.
// "Chapter 8 - Next-generation KV cache" (LLM Primer VI), section 8.1: the
// kernel reads keys and values by indirect addressing through the table.
//
// Work decomposition.  The batch is a list of 32-token chunks (two blocks)
// of every (sequence, kv head) pair, head-major (all of kv head 0's
// sequences, then kv head 1's, ...).  One worker wave per SIMD slot of the
// GPU takes an equal contiguous range of that list (stream-K style), so all
// waves stream the same bytes, and the workgroups of one XCD take adjacent
// ranges, so a block shared by many sequences is re-read from that XCD's L2.
// Each wave keeps a running max / sum / accumulator per
// pair segment for the pair's whole query group.  A pair that one wave covers
// completely is finished by that wave; a pair split between waves leaves one
// float32 partial per wave, combined by decode_merge_kernel.
//
// Tile math (CDNA4 MFMA, 64-lane waves).  Scores are computed transposed,
// S^T[token][head] = K q^T, so that the MFMA output layout (lane l holds rows
// 4*(l/16)..+3 of column l%16) is already the layout of the B operand of the
// P.V product: acc^T[dim][head] += V^T[dim][token] P^T[token][head].  Query
// heads sit on the 16 MFMA columns (padded with zero queries), tokens on
// the rows.  With the V tile stored dim-major in the pool, every K and V
// operand is a direct 16-byte load from HBM, with no LDS transpose.
//
// Chunk layout.  For the chunk's two blocks A and B, score row r of group
// x in {0,1} holds token 8*((r/4)%2) + 4*x + (r%4) of block r/8.  The MFMA
// output then gives lane (r, j = l/16) the eight tokens 8*j .. 8*j+7 of the
// chunk for head r, exactly the eight tokens it supplies for P.V.
//
// Every wave-level arithmetic order depends only on logical token positions,
// the context length and the partition size, never on physical block ids, so
// permuting the pool or sharing blocks leaves the output bit-identical.

#include "pkv_internal.h"
#include "split_body.h"
#include "tile_math.h"

#include <atomic>

namespace pkv {
namespace {

// Tables, lengths and scales are passed again as restrict parameters: nothing
// the kernel writes aliases them, so their wave-uniform reads go through the
// scalar cache and never wait behind the vector loads in flight.  Registers
// are capped at 256 per wave (two waves per SIMD would fit), although the
// default launch runs one worker wave per SIMD (1024 waves on 256 compute
// units): a second wave per SIMD measured slower.  The float32 path at
// head_dim 128 needs more registers for its double buffer and is built for
// one wave per SIMD instead of spilling.
template <int KV, int D, bool KNT, bool VNT, bool kTail>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                         const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  split_body<KV, D, KNT, VNT, kTail>(a, tables, lens, k_scale, v_scale);
}

template <int KV, int D, bool KNT, bool VNT, bool kTail>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel_wide(DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                              const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  split_body<KV, D, KNT, VNT, kTail>(a, tables, lens, k_scale, v_scale);
}

// ---------------------------------------------------------------------------
// Merge kernel: one workgroup per (sequence, kv head) pair.  Its only input
// besides the partials is the pair's record, written by the split kernel on
// every call: a pair one wave finished (or an empty one, already zeroed)
// returns at once; a split pair combines its partials with the online-softmax
// rescale.  Two dependent round trips: the record, then the partials.
// ---------------------------------------------------------------------------
template <typename OutT, int D, bool kPrefix>
__global__ __launch_bounds__(256) void decode_merge_kernel(const int2* __restrict__ meta,
                                                           const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml, OutT* __restrict__ out,
                                                           int num_seqs, int num_kv_heads, int group, int q_len,
                                                           const OutT* __restrict__ pre_acc,
                                                           const float* __restrict__ pre_ml, int pre_segments) {
  const int pair = blockIdx.x;
  const int2 m = meta[pair];
  // One wave covered the pair and wrote its output (no shared-prefix pieces).
  if (m.y <= 1 && !kPrefix) return;
  const int G = group;
  const int NC = q_len * G;   // (query token, query head) columns of the pair
  const int b = pair / num_kv_heads;
  const int g = pair - b * num_kv_heads;
  const size_t place = (size_t)g * num_seqs + b;   // the pair's place in the head-major chunk order
  const size_t Hq = (size_t)num_kv_heads * G;
  for (int e = threadIdx.x; e < NC * (D / 4); e += blockDim.x) {
    const int c = e / (D / 4);
    const int q4 = e % (D / 4);
    const int qi = c / G;
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int w = m.x; w < m.x + m.y; ++w) {
      const size_t slot = ((size_t)w + place) * NC + c;
      const float2 ml = *reinterpret_cast<const float2*>(ws_ml + slot * 2);
      const f32x4 acc_w = *reinterpret_cast<const f32x4*>(ws_acc + slot * D + 4 * q4);
      const float M2 = fmaxf(M, ml.x);
      const float M2u = M2 == -INFINITY ? 0.f : M2;   // pieces that saw no token weigh 0
      const float f_old = exp2_fast(M - M2u);
      const float f_new = exp2_fast(ml.x - M2u);
      L = L * f_old + ml.y * f_new;
      o = o * f_old + acc_w * f_new;
      M = M2;
    }
    // Shared-prefix pieces: the same column's partials over the prefix's
    // key segments (one query token per sequence here).  Their maximum
    // first, then the weighted sums, so that the pieces' loads do not wait
    // on one another.
    if constexpr (kPrefix) {
      const size_t col = (size_t)b * Hq + (size_t)g * G + (c - qi * G);
      const size_t stride = (size_t)num_seqs * Hq;
      float Mp = -INFINITY;
#pragma unroll 8
      for (int s = 0; s < pre_segments; ++s) Mp = fmaxf(Mp, pre_ml[(s * stride + col) * 2]);
      const float M2 = fmaxf(M, Mp);
      const float M2u = M2 == -INFINITY ? 0.f : M2;
      const float f_old = exp2_fast(M - M2u);
      L *= f_old;
      o *= f_old;
#pragma unroll 8
      for (int s = 0; s < pre_segments; ++s) {
        const size_t slot = s * stride + col;
        const float2 ml = *reinterpret_cast<const float2*>(pre_ml + slot * 2);
        const f32x4 acc_s = load4<OutT>(pre_acc + slot * D + 4 * q4);
        const float w = exp2_fast(ml.x - M2u);
        L += ml.y * w;
        o += acc_s * w;
      }
    }
    OutT* dst = out + (((size_t)b * q_len + qi) * Hq + (size_t)g * G + (c - qi * G)) * D + 4 * q4;
    store4<OutT>(dst, o * (L > 0.f ? 1.f / L : 0.f));
  }
}

template <int KV, int D, bool KNT, bool VNT, bool kTail>
hipError_t launch_split_p(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.num_workers / kDecodeWaves);
  if constexpr (KV == kF32 && D == 128)
    hipLaunchKernelGGL((decode_split_kernel_wide<KV, D, KNT, VNT, kTail>), dim3(grid), dim3(64 * kDecodeWaves), 0, stream,
                       a, a.block_tables, a.context_lens, a.k_scale, a.v_scale);
  else
    hipLaunchKernelGGL((decode_split_kernel<KV, D, KNT, VNT, kTail>), dim3(grid), dim3(64 * kDecodeWaves), 0, stream, a,
                       a.block_tables, a.context_lens, a.k_scale, a.v_scale);
  return hipGetLastError();
}

// Load policy: K and V streamed when every byte is read once.  Cached loads
// for both when blocks are shared (re-read within the call) and at block
// sizes of 64 and more, where a 32-token chunk uses half of each V line and
// the next chunk reads the other half (measured on MI355X: streaming only K,
// or both, is slower there than caching both).
template <int KV, int D, bool kTail>
hipError_t launch_split_l(const DecodeArgs& a, hipStream_t stream) {
  if (a.kv_reread || a.block_size > 32) return launch_split_p<KV, D, false, false, kTail>(a, stream);
  return launch_split_p<KV, D, true, true, kTail>(a, stream);
}

template <int KV, int D>
hipError_t launch_split_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.tail_pass) return launch_split_l<KV, D, true>(a, stream);
  return launch_split_l<KV, D, false>(a, stream);
}


template <typename OutT, int D, bool kPrefix>
hipError_t launch_merge_p(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * (unsigned)a.num_kv_heads;
  // one thread per four output elements of the pair, up to 256
  const unsigned threads = a.q_len * a.group * (D / 4) > 128 ? 256 : 128;
  hipLaunchKernelGGL((decode_merge_kernel<OutT, D, kPrefix>), dim3(grid), dim3(threads), 0, stream,
                     static_cast<const int2*>(a.pair_meta), static_cast<const float*>(a.ws_acc),
                     static_cast<const float*>(a.ws_ml), static_cast<OutT*>(a.out), a.num_seqs, a.num_kv_heads,
                     a.group, a.q_len, static_cast<const OutT*>(a.pre_acc), a.pre_ml, a.pre_segments);
  return hipGetLastError();
}

template <typename OutT, int D>
hipError_t launch_merge_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.pre_segments > 0) return launch_merge_p<OutT, D, true>(a, stream);
  return launch_merge_p<OutT, D, false>(a, stream);
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream) {
  const bool f32 = a.kv_dtype == kF32;
  if (a.head_dim == 64) return f32 ? launch_merge_t<float, 64>(a, stream) : launch_merge_t<__bf16, 64>(a, stream);
  return f32 ? launch_merge_t<float, 128>(a, stream) : launch_merge_t<__bf16, 128>(a, stream);
}

hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) {
    if (a.kv_dtype == kF32) return launch_split_t<kF32, 64>(a, stream);
    if (a.kv_dtype == kBF16) return launch_split_t<kBF16, 64>(a, stream);
    return launch_split_t<kFP8, 64>(a, stream);
  }
  if (a.kv_dtype == kF32) return launch_split_t<kF32, 128>(a, stream);
  if (a.kv_dtype == kBF16) return launch_split_t<kBF16, 128>(a, stream);
  return launch_split_t<kFP8, 128>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const hipError_t e = launch_split(a, stream);
  if (e != hipSuccess) return e;
  return launch_merge(a, stream);
}

// Decode workspace for callers that cannot allocate (see
// pkv_paged_decode_static).  Each device holds its own copy for the life of
// the process.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the address static_scratch() looks
// up per device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

void* static_scratch() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  // first call on this device, with it current: resolve this device's copy
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace pkv
