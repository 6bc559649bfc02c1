// Paged decode attention for gfx950: partition kernel + merge kernel.
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
// Work decomposition.  One workgroup of four waves handles one (sequence,
// kv head, context partition) and the whole query group of that kv head.
// Each wave walks the partition in 32-token chunks (two blocks), chunk c
// going to wave c % 4, and keeps its own running max / sum / accumulator;
// the four states are merged through LDS at the end.  A sequence that fits
// in one partition is finished here; longer ones leave one float32 partial
// state per partition for decode_reduce_kernel.
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

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-head value across the four 16-lane rows (lanes l, l^16,
// l^32, l^48 hold the same head).
__device__ __forceinline__ float row_max4(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)s16[0]), __builtin_bit_cast(float, (uint32_t)s16[1]));
  u = __builtin_bit_cast(uint32_t, v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)s32[0]), __builtin_bit_cast(float, (uint32_t)s32[1]));
}

__device__ __forceinline__ float row_sum4(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)s16[0]) + __builtin_bit_cast(float, (uint32_t)s16[1]);
  u = __builtin_bit_cast(uint32_t, v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)s32[0]) + __builtin_bit_cast(float, (uint32_t)s32[1]);
}

// Score row r of group x -> token offset inside the block r / 8.
__device__ __forceinline__ int row_token(int r, int x) { return 8 * ((r >> 2) & 1) + 4 * x + (r & 3); }

// Keep the first `nvalid` 16-bit lanes of a vector of eight, zero the rest.
__device__ __forceinline__ u32x4 keep16(u32x4 v, int nvalid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (2 * w < nvalid) ? 0x0000FFFFu : 0u;
    const uint32_t hi = (2 * w + 1 < nvalid) ? 0xFFFF0000u : 0u;
    v[w] &= (lo | hi);
  }
  return v;
}

// ---------------------------------------------------------------------------
// bf16 cache, bf16 queries: v_mfma_f32_16x16x32_bf16 for both products.
// QK step s covers head dims 32*s .. 32*s+31; lane group j supplies 8*j..8*j+7.
// ---------------------------------------------------------------------------
template <int D>
struct TileBF16 {
  using Elem = uint16_t;
  static constexpr int kSteps = D / 32;
  static constexpr int kTiles = D / 16;
  struct Q { bf16x8 op[kSteps]; };
  struct K { u32x4 x[kSteps]; u32x4 y[kSteps]; };
  struct V { u32x4 t[kTiles]; };

  __device__ static void load_q(Q& q, const void* row, bool valid, int j) {
    const Elem* p = static_cast<const Elem*>(row);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 v = valid ? *reinterpret_cast<const u32x4*>(p + 32 * s + 8 * j) : u32x4{0, 0, 0, 0};
      q.op[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // tile: K tile [16][D] of block r / 8 for this lane.
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const Elem* rx = tile + row_token(r, 0) * D + 8 * j;
    const Elem* ry = tile + row_token(r, 1) * D + 8 * j;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      k.x[s] = *reinterpret_cast<const u32x4*>(rx + 32 * s);
      k.y[s] = *reinterpret_cast<const u32x4*>(ry + 32 * s);
    }
  }
  // tile: V^T tile [D][16] of block j / 2 for this lane.
  __device__ static void load_v(V& v, const Elem* tile, int r, int j) {
    const Elem* base = tile + r * 16 + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) v.t[t] = *reinterpret_cast<const u32x4*>(base + t * 256);
  }
  __device__ static void scores(const K& k, const Q& q, f32x4& sx, f32x4& sy) {
    sx = f32x4{0.f, 0.f, 0.f, 0.f};
    sy = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.x[s]), q.op[s], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.y[s]), q.op[s], sy, 0, 0, 0);
    }
  }
  __device__ static void mask_v(V& v, int nvalid) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) v.t[t] = keep16(v.t[t], nvalid);
  }
  // Rounds p to bf16 (the MFMA operand) and returns the sum of the rounded values.
  __device__ static float pv(f32x4* acc, const V& v, const float* p) {
    bf16x8 pb;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pb[k] = (__bf16)p[k];
      sum += (float)pb[k];
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.t[t]), pb, acc[t], 0, 0, 0);
    return sum;
  }
};

// ---------------------------------------------------------------------------
// fp8 (E4M3) cache, bf16 queries.  Codes widen exactly to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8) and feed the same bf16 MFMA.  Lane group j
// owns head dims j*D/4 .. (j+1)*D/4-1, so each K row piece is a 16-byte
// load; QK step s uses dims j*D/4 + 8*s .. +7 of that range.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  auto c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  auto c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  auto c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  auto c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, c0), __builtin_bit_cast(uint32_t, c1),
               __builtin_bit_cast(uint32_t, c2), __builtin_bit_cast(uint32_t, c3)};
}

template <int D>
struct TileFP8 {
  using Elem = uint8_t;
  static constexpr int kSteps = D / 32;          // bf16 MFMAs along the head dim
  static constexpr int kLoads = D / 64;          // 16-byte K loads per score row
  static constexpr int kTiles = D / 16;
  struct Q { bf16x8 op[kSteps]; };
  struct K { u32x4 x[kLoads]; u32x4 y[kLoads]; };
  struct V { u32x2 t[kTiles]; };

  __device__ static void load_q(Q& q, const void* row, bool valid, int j) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + j * (D / 4);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 v = valid ? *reinterpret_cast<const u32x4*>(p + 8 * s) : u32x4{0, 0, 0, 0};
      q.op[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const Elem* rx = tile + row_token(r, 0) * D + j * (D / 4);
    const Elem* ry = tile + row_token(r, 1) * D + j * (D / 4);
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      k.x[s] = *reinterpret_cast<const u32x4*>(rx + 16 * s);
      k.y[s] = *reinterpret_cast<const u32x4*>(ry + 16 * s);
    }
  }
  __device__ static void load_v(V& v, const Elem* tile, int r, int j) {
    const Elem* base = tile + r * 16 + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) v.t[t] = *reinterpret_cast<const u32x2*>(base + t * 256);
  }
  __device__ static void scores(const K& k, const Q& q, f32x4& sx, f32x4& sy) {
    sx = f32x4{0.f, 0.f, 0.f, 0.f};
    sy = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const u32x4 ax0 = fp8x8_to_bf16x8(k.x[s][0], k.x[s][1]);
      const u32x4 ax1 = fp8x8_to_bf16x8(k.x[s][2], k.x[s][3]);
      const u32x4 ay0 = fp8x8_to_bf16x8(k.y[s][0], k.y[s][1]);
      const u32x4 ay1 = fp8x8_to_bf16x8(k.y[s][2], k.y[s][3]);
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax0), q.op[2 * s], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ay0), q.op[2 * s], sy, 0, 0, 0);
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax1), q.op[2 * s + 1], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ay1), q.op[2 * s + 1], sy, 0, 0, 0);
    }
  }
  __device__ static void mask_v(V& v, int nvalid) {
    // byte lanes: keep the first nvalid codes (code 0 is +0.0)
    const uint64_t keep = nvalid >= 8 ? ~0ull : ((1ull << (8 * nvalid)) - 1ull);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      v.t[t][0] &= (uint32_t)keep;
      v.t[t][1] &= (uint32_t)(keep >> 32);
    }
  }
  __device__ static float pv(f32x4* acc, const V& v, const float* p) {
    bf16x8 pb;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pb[k] = (__bf16)p[k];
      sum += (float)pb[k];
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const u32x4 a = fp8x8_to_bf16x8(v.t[t][0], v.t[t][1]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, acc[t], 0, 0, 0);
    }
    return sum;
  }
};

// ---------------------------------------------------------------------------
// fp32 cache, fp32 queries: v_mfma_f32_16x16x4_f32 keeps the whole path in
// float32.  MFMA i = 4*a + c contracts head dim 16*a + 4*j + c, so one
// 16-byte load per lane feeds four consecutive MFMAs.
// ---------------------------------------------------------------------------
template <int D>
struct TileF32 {
  using Elem = float;
  static constexpr int kQuads = D / 16;
  static constexpr int kTiles = D / 16;
  struct Q { f32x4 op[kQuads]; };
  struct K { f32x4 x[kQuads]; f32x4 y[kQuads]; };
  struct V { f32x4 t[kTiles][2]; };

  __device__ static void load_q(Q& q, const void* row, bool valid, int j) {
    const float* p = static_cast<const float*>(row) + 4 * j;
#pragma unroll
    for (int a = 0; a < kQuads; ++a)
      q.op[a] = valid ? *reinterpret_cast<const f32x4*>(p + 16 * a) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const float* rx = tile + row_token(r, 0) * D + 4 * j;
    const float* ry = tile + row_token(r, 1) * D + 4 * j;
#pragma unroll
    for (int a = 0; a < kQuads; ++a) {
      k.x[a] = *reinterpret_cast<const f32x4*>(rx + 16 * a);
      k.y[a] = *reinterpret_cast<const f32x4*>(ry + 16 * a);
    }
  }
  __device__ static void load_v(V& v, const Elem* tile, int r, int j) {
    const float* base = tile + r * 16 + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      v.t[t][0] = *reinterpret_cast<const f32x4*>(base + t * 256);
      v.t[t][1] = *reinterpret_cast<const f32x4*>(base + t * 256 + 4);
    }
  }
  __device__ static void scores(const K& k, const Q& q, f32x4& sx, f32x4& sy) {
    sx = f32x4{0.f, 0.f, 0.f, 0.f};
    sy = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < kQuads; ++a) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sx = __builtin_amdgcn_mfma_f32_16x16x4f32(k.x[a][c], q.op[a][c], sx, 0, 0, 0);
        sy = __builtin_amdgcn_mfma_f32_16x16x4f32(k.y[a][c], q.op[a][c], sy, 0, 0, 0);
      }
    }
  }
  __device__ static void mask_v(V& v, int nvalid) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k >= nvalid) v.t[t][k >> 2][k & 3] = 0.f;
  }
  __device__ static float pv(f32x4* acc, const V& v, const float* p) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) sum += p[k];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.t[t][u >> 2][u & 3], p[u], acc[t], 0, 0, 0);
    return sum;
  }
};

template <int KV, int D> struct TileOf;
template <int D> struct TileOf<kF32, D> { using type = TileF32<D>; using Out = float; };
template <int D> struct TileOf<kBF16, D> { using type = TileBF16<D>; using Out = __bf16; };
template <int D> struct TileOf<kFP8, D> { using type = TileFP8<D>; using Out = __bf16; };

template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *reinterpret_cast<bf16x4*>(dst) = o;
}

__device__ __forceinline__ int clamp_len(int n, const DecodeArgs& a) {
  n = min(n, a.max_context_len);
  n = min(n, a.max_blocks * kBlockTokens);
  return max(n, 0);
}

// ---------------------------------------------------------------------------
// Partition kernel
// ---------------------------------------------------------------------------
template <int KV, int D>
__device__ __forceinline__ void decode_partitions_body(const DecodeArgs& a) {
  using T = typename TileOf<KV, D>::type;
  using OutT = typename TileOf<KV, D>::Out;
  using Elem = typename T::Elem;
  constexpr int kTiles = D / 16;

  __shared__ float s_ml[kDecodeWaves][kMaxGroup][2];
  __shared__ f32x4 s_acc[kDecodeWaves][kMaxGroup][D / 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int j = lane >> 4;

  const int P = a.num_parts;
  int item = blockIdx.x;
  const int p = item % P;
  item /= P;
  const int g = item % a.num_kv_heads;
  const int b = item / a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_q_heads;

  const int n = clamp_len(a.context_lens[b], a);
  OutT* out = static_cast<OutT*>(a.out);
  if (n == 0) {
    if (p == 0)
      for (int e = threadIdx.x; e < G * D; e += 64 * kDecodeWaves)
        out[((size_t)b * Hq + g * G) * D + e] = (OutT)0.f;
    return;
  }
  const int start = p * a.part_tokens;
  if (start >= n) return;
  const int end = min(start + a.part_tokens, n);
  const int nchunks = (end - start + kChunkTokens - 1) / kChunkTokens;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const bool single = n <= a.part_tokens;

  // Softmax runs in log2 units: t = score * scale * log2(e).
  float sl = a.scale * kLog2e;
  float out_mul = 1.f;
  if constexpr (KV == kFP8) {
    sl *= a.k_scale[g];
    out_mul = a.v_scale[g];
  }

  // Query operand: lane (r, j) holds head g*G + r (zero for padding columns r >= G).
  constexpr size_t kQBytes = (KV == kF32) ? 4 : 2;
  const uint8_t* q_row =
      static_cast<const uint8_t*>(a.q) + ((size_t)b * Hq + g * G + min(r, G - 1)) * D * kQBytes;
  typename T::Q qop;
  T::load_q(qop, q_row, r < G, j);

  const size_t blk_stride = (size_t)a.num_kv_heads * kBlockTokens * D;   // elements per block
  const Elem* kpool = static_cast<const Elem*>(a.k_pool) + (size_t)g * kBlockTokens * D;
  const Elem* vpool = static_cast<const Elem*>(a.v_pool) + (size_t)g * kBlockTokens * D;

  // Block ids of this partition, one per lane: lane i of id_lo / id_hi holds
  // partition-relative logical block i / 64 + i.  Entries past the
  // sequence's last block are never read (the last valid id repeats).
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const int first_blk = start / kBlockTokens;
  const int last_blk = nblk - 1;
  const int id_lo = table[min(first_blk + lane, last_blk)];
  const int id_hi = a.part_tokens > 64 * kBlockTokens ? table[min(first_blk + 64 + lane, last_blk)] : 0;
  auto block_off = [&](int rel) -> size_t {   // rel: wave-uniform relative block
    int id = rel < 64 ? __builtin_amdgcn_readlane(id_lo, rel) : __builtin_amdgcn_readlane(id_hi, rel - 64);
    id = min(max(id, 0), a.num_blocks - 1);
    return (size_t)id * blk_stride;
  };
  auto issue = [&](typename T::K& kb, typename T::V& vb, int c) {
    const size_t o0 = block_off(2 * c);
    const size_t o1 = block_off(2 * c + 1);
    T::load_k(kb, kpool + ((r >> 3) ? o1 : o0), r, j);
    T::load_v(vb, vpool + ((j >> 1) ? o1 : o0), r, j);
  };

  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto compute = [&](typename T::K& kb, typename T::V& vb, int c) {
    const int t0 = start + c * kChunkTokens;
    f32x4 sx, sy;
    T::scores(kb, qop, sx, sy);
    float t[8] = {sx[0] * sl, sx[1] * sl, sx[2] * sl, sx[3] * sl,
                  sy[0] * sl, sy[1] * sl, sy[2] * sl, sy[3] * sl};
    if (t0 + kChunkTokens > end) {   // tail chunk: mask tokens at or past the end
      const int nvalid = min(max(end - (t0 + 8 * j), 0), 8);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k >= nvalid) t[k] = -INFINITY;
      T::mask_v(vb, nvalid);
    }
    float mloc = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                       fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
    mloc = row_max4(mloc);
    const float m_new = fmaxf(m_run, mloc);
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float corr = exp2_fast(m_run - m_new);
#pragma unroll
      for (int q = 0; q < kTiles; ++q) acc[q] *= corr;
      l_run *= corr;
    }
    m_run = m_new;
    float pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pk[k] = exp2_fast(t[k] - m_new);
    l_run += T::pv(acc, vb, pk);
  };

  // Two register buffers: chunk k+1's loads are in flight while chunk k is
  // computed.  The steady-state loop issues its prefetch unconditionally so
  // that the compiler's load counters wait only for the buffer in use.
  const int my_chunks = wave < nchunks ? (nchunks - 1 - wave) / kDecodeWaves + 1 : 0;
  typename T::K kA, kB;
  typename T::V vA, vB;
  if (my_chunks > 0) {
    issue(kA, vA, wave);
    int k = 0;
    for (; k + 2 < my_chunks; k += 2) {
      issue(kB, vB, wave + (k + 1) * kDecodeWaves);
      compute(kA, vA, wave + k * kDecodeWaves);
      issue(kA, vA, wave + (k + 2) * kDecodeWaves);
      compute(kB, vB, wave + (k + 1) * kDecodeWaves);
    }
    if (k + 1 < my_chunks) {
      issue(kB, vB, wave + (k + 1) * kDecodeWaves);
      compute(kA, vA, wave + k * kDecodeWaves);
      compute(kB, vB, wave + (k + 1) * kDecodeWaves);
    } else {
      compute(kA, vA, wave + k * kDecodeWaves);
    }
  }

  // Per-head totals of this wave; every lane of head r now agrees on m, l.
  l_run = row_sum4(l_run);
  if (j == 0) {
    s_ml[wave][r][0] = m_run;
    s_ml[wave][r][1] = l_run;
  }
  if (r < G) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) s_acc[wave][r][4 * t + j] = acc[t];
  }
  __syncthreads();

  // Merge the four wave states (the same rescaling as within a wave).
  for (int e = threadIdx.x; e < G * (D / 4); e += 64 * kDecodeWaves) {
    const int h = e / (D / 4);
    const int q4 = e % (D / 4);
    float M = s_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = exp2_fast(s_ml[w][h][0] - M);   // a wave without tokens has m = -inf
      L += f * s_ml[w][h][1];
      o += f * s_acc[w][h][q4];
    }
    const int qh = g * G + h;
    if (single) {
      store4<OutT>(out + ((size_t)b * Hq + qh) * D + 4 * q4, o * (out_mul / L));
    } else {
      const size_t slot = ((size_t)b * Hq + qh) * P + p;
      *reinterpret_cast<f32x4*>(a.ws_acc + slot * D + 4 * q4) = o * out_mul;
      if (q4 == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = L;
      }
    }
  }
}

// Two waves per SIMD (at most 256 VGPRs each) keep 8 waves' loads in flight
// per compute unit; the float32 path at head_dim 128 needs more registers
// for its double buffer and runs one wave per SIMD instead of spilling.
template <int KV, int D>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_partitions_kernel(DecodeArgs a) {
  decode_partitions_body<KV, D>(a);
}

template <int KV, int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partitions_kernel_wide(DecodeArgs a) {
  decode_partitions_body<KV, D>(a);
}

// ---------------------------------------------------------------------------
// Merge kernel: one workgroup per (sequence, query head) spanning > 1 partition.
// ---------------------------------------------------------------------------
template <typename OutT, int D>
__global__ __launch_bounds__(128) void decode_reduce_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads;
  const int n = clamp_len(a.context_lens[b], a);
  const int np = min((n + a.part_tokens - 1) / a.part_tokens, a.num_parts);
  if (np <= 1) return;   // finished by the partition kernel
  const float* ml = a.ws_ml + (size_t)bh * a.num_parts * 2;
  const float* acc = a.ws_acc + (size_t)bh * a.num_parts * D;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  for (int d = threadIdx.x; d < D; d += 128) {
    float L = 0.f, o = 0.f;
    for (int p = 0; p < np; ++p) {
      const float f = exp2_fast(ml[2 * p] - M);
      L += f * ml[2 * p + 1];
      o += f * acc[(size_t)p * D + d];
    }
    static_cast<OutT*>(a.out)[(size_t)bh * D + d] = (OutT)(o / L);
  }
}

template <int KV, int D>
hipError_t launch_partitions_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * (unsigned)a.num_kv_heads * (unsigned)a.num_parts;
  if constexpr (KV == kF32 && D == 128)
    hipLaunchKernelGGL((decode_partitions_kernel_wide<KV, D>), dim3(grid), dim3(64 * kDecodeWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partitions_kernel<KV, D>), dim3(grid), dim3(64 * kDecodeWaves), 0, stream, a);
  return hipGetLastError();
}

template <typename OutT, int D>
hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * (unsigned)a.num_q_heads;
  hipLaunchKernelGGL((decode_reduce_kernel<OutT, D>), dim3(grid), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) {
    if (a.kv_dtype == kF32) return launch_partitions_t<kF32, 64>(a, stream);
    if (a.kv_dtype == kBF16) return launch_partitions_t<kBF16, 64>(a, stream);
    return launch_partitions_t<kFP8, 64>(a, stream);
  }
  if (a.kv_dtype == kF32) return launch_partitions_t<kF32, 128>(a, stream);
  if (a.kv_dtype == kBF16) return launch_partitions_t<kBF16, 128>(a, stream);
  return launch_partitions_t<kFP8, 128>(a, stream);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  const bool f32 = a.kv_dtype == kF32;
  if (a.head_dim == 64) return f32 ? launch_reduce_t<float, 64>(a, stream) : launch_reduce_t<__bf16, 64>(a, stream);
  return f32 ? launch_reduce_t<float, 128>(a, stream) : launch_reduce_t<__bf16, 128>(a, stream);
}

}  // namespace pkv
