// Tile math shared by the paged attention kernels (gfx950, 64-lane waves):
// MFMA operand types, the per-dtype score and P.V tiles, lane reductions and
// output stores.  Device-only; included inside namespace pkv's anonymous
// namespace of each kernel source, so every translation unit has its own copy.
//
// Scores are computed transposed, S^T[token][column] = K q^T: the 16 MFMA
// columns are query columns, the rows are key tokens.  The MFMA output layout
// (lane l holds rows 4*(l/16)..+3 of column l%16) is then already the layout
// of the B operand of the P.V product acc^T[dim][column] += V^T[dim][token]
// P^T[token][column], so scores never leave registers.
#pragma once

#include "pkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// A value every lane holds: keep it in a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Operand loads.  With NT the load is non-temporal: bytes read once per call
// stream past the caches (measured on MI355X: random 4 KiB tiles at 6.7 TB/s
// instead of 6.0 with ordinary loads).  Ordinary loads keep lines cached for
// bytes that are read again within the call (blocks shared by several
// sequences; the other half of a V line at block sizes of 64 and more).
template <bool NT, typename V>
__device__ __forceinline__ V op_load(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  return *reinterpret_cast<const V*>(p);
}

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

// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): propagates NaN, so the
// compiler needs no quieting step before it; for scores that are finite or
// -inf it is the ordinary max.
__device__ __forceinline__ float fmax_nq(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// row_max4 for values that are never NaN, without quieting steps.
__device__ __forceinline__ float row_max4_nq(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmax_nq(__builtin_bit_cast(float, (uint32_t)s16[0]), __builtin_bit_cast(float, (uint32_t)s16[1]));
  u = __builtin_bit_cast(uint32_t, v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmax_nq(__builtin_bit_cast(float, (uint32_t)s32[0]), __builtin_bit_cast(float, (uint32_t)s32[1]));
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
  // tile: the first of the 16 token rows of this lane's half-chunk (half
  // r / 8) inside its block's token-major K tile.
  template <bool NT>
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const Elem* rx = tile + row_token(r, 0) * D + 8 * j;
    const Elem* ry = tile + row_token(r, 1) * D + 8 * j;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      k.x[s] = op_load<NT, u32x4>(rx + 32 * s);
      k.y[s] = op_load<NT, u32x4>(ry + 32 * s);
    }
  }
  // tile: this lane's half-chunk inside the V^T tile [D][bs] (dim rows of
  // bs tokens); the lane reads dims 16 t + r, tokens 8 (j % 2) .. +7.
  template <bool NT>
  __device__ static void load_v(V& v, const Elem* tile, int r, int j, int bs) {
    const Elem* base = tile + r * bs + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) v.t[t] = op_load<NT, u32x4>(base + (size_t)t * 16 * bs);
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
  template <bool NT>
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const Elem* rx = tile + row_token(r, 0) * D + j * (D / 4);
    const Elem* ry = tile + row_token(r, 1) * D + j * (D / 4);
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      k.x[s] = op_load<NT, u32x4>(rx + 16 * s);
      k.y[s] = op_load<NT, u32x4>(ry + 16 * s);
    }
  }
  template <bool NT>
  __device__ static void load_v(V& v, const Elem* tile, int r, int j, int bs) {
    const Elem* base = tile + r * bs + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) v.t[t] = op_load<NT, u32x2>(base + (size_t)t * 16 * bs);
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
  template <bool NT>
  __device__ static void load_k(K& k, const Elem* tile, int r, int j) {
    const float* rx = tile + row_token(r, 0) * D + 4 * j;
    const float* ry = tile + row_token(r, 1) * D + 4 * j;
#pragma unroll
    for (int a = 0; a < kQuads; ++a) {
      k.x[a] = op_load<NT, f32x4>(rx + 16 * a);
      k.y[a] = op_load<NT, f32x4>(ry + 16 * a);
    }
  }
  template <bool NT>
  __device__ static void load_v(V& v, const Elem* tile, int r, int j, int bs) {
    const float* base = tile + r * bs + 8 * (j & 1);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      v.t[t][0] = op_load<NT, f32x4>(base + (size_t)t * 16 * bs);
      v.t[t][1] = op_load<NT, f32x4>(base + (size_t)t * 16 * bs + 4);
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

// Four consecutive elements widened to float32 (exact).
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* src);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* src) {
  return *reinterpret_cast<const f32x4*>(src);
}
template <>
__device__ __forceinline__ f32x4 load4<__bf16>(const __bf16* src) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  const u32x2v w = *reinterpret_cast<const u32x2v*>(src);
  return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xFFFF0000u),
               __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xFFFF0000u)};
}

}  // namespace
}  // namespace pkv
