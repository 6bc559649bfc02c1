// Paged attention for many query tokens per sequence (chunked prefill) on
// gfx950.
//
// What is computed (Habr KV-Cache article, habr.com/ru/articles/1021832):
//  - section 6 "Chunked Prefill": a chunk of a prompt's new tokens is
//    processed as its own step and attends to everything cached before it;
//    the chunk's keys and values are already in the paged cache (appended
//    first), so query token i of a chunk of L tokens in a sequence of n
//    cached tokens sits at position n - L + i and sees tokens 0 .. n - L + i;
//  - section 3 "Recalling FlashAttention": exact softmax(q K^T * scale) V
//    reached tile by tile with a running max and sum;
//  - section 4 "Recalling PagedAttention": K and V live in blocks scattered
//    over a pool, found through the block table;
//  - section 2 "GQA": the group's query heads share one kv head.
//
// With many query columns (query token, head) per kv head this is a dense
// contraction, bound by the matrix cores, not by HBM: each K/V chunk is
// loaded once into LDS and used by every column of a workgroup.
//
// Work decomposition.  Columns c = i * G + h of a (sequence, kv head) pair
// are cut into workgroup tiles of kWaves * 16 * kT columns (256: eight waves
// of two 16-column MFMA tiles, two waves per SIMD; float32: four waves, one
// per SIMD); a workgroup owns one tile and walks every 32-token key chunk up
// to the tile's last visible token, so no partial results leave the
// workgroup.  The waves stage each chunk's K (token-major) and V
// (dimension-major) from the pool into LDS together (three groups of three
// chunk buffers, one for float32 tiles; one barrier per group) and each
// reads its operands from
// there; an fp8 cache is widened to bf16 (exactly) as it is staged, so the
// LDS tiles and the operand reads are the bf16 ones.  Workgroups are
// issued largest first (the last column tiles see the most keys), and
// workgroups of the same pair are spaced by the pair count, so with a pair
// count divisible by 8 they land on the same XCD and share its L2.
//
// Tile math: the transposed-score layout of the decode kernel (tile_math.h):
// per chunk and column tile, 2 * D/32 score MFMAs, D/16 P.V MFMAs and one
// row-sum MFMA (bf16 and fp8 caches), all operands read from LDS with
// 16-byte reads.

#include "pkv_internal.h"
#include "tile_math.h"

#include <type_traits>

namespace pkv {
namespace {

// Rescale threshold (log2 units): the running max used in the exponentials
// is only raised when a column's max exceeds it by more than this, so
// weights stay below 2^8 and most chunks skip the accumulator rescale.
constexpr float kRescaleSlack = 8.f;

// s_waitcnt immediate for "vector memory counter 0, others unchanged"
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kVmcntZero = 0x0F70;

// LDS bank rules for 16-byte reads (measured on MI355X with the LDS bank
// conflict counter): lanes r = 0..15 of a quarter-wave reading rows of a
// tile at a row stride S are conflict-free when S is 32 bytes plus a
// multiple of 64 (S = 80, 144 or 272 bytes conflict two-way); the K tiles
// use such strides.  The bf16 V tile is unpadded (64-byte rows, two-way
// conflicts as is) and XOR-swizzles its 16-byte pieces instead, which the
// counter shows conflict-free for the V reads.
//
// LDS row of chunk token t in the K tile.  The 16 lanes of a lane group read
// the rows of tokens 8 (r / 4) + 4 x + (r % 4), r < 16; without this row
// permutation those rows conflict at every stride.
__device__ __forceinline__ int k_row(int t) { return t ^ ((t >> 1) & 12); }

template <int KV, int D>
struct PrefillCfg {
  // fp8 codes are widened to bf16 once, as a chunk is staged into LDS (by
  // the staging threads, not by every wave that reads it), so the LDS tiles
  // and the operand reads are the bf16 ones for both cache dtypes.
  static constexpr int kLds = KV == kFP8 ? kBF16 : KV;           // dtype of the LDS tiles
  using Tile = typename TileOf<kLds, D>::type;                    // operand tiles read from LDS
  using Elem = typename Tile::Elem;                               // LDS element
  using Out = typename TileOf<KV, D>::Out;
  static constexpr int kEs = (int)sizeof(Elem);                  // LDS element bytes
  static constexpr int kPs = KV == kFP8 ? 1 : kEs;               // pool element bytes
  static constexpr int kPerPiece = 16 / kPs;                     // pool elements per 16-byte piece
  // Eight waves of two column tiles (two waves per SIMD, at most 256
  // registers each) for bf16 / fp8; the float32 tiles need more registers
  // and run four waves, one per SIMD.
  static constexpr int kT = 2;                                   // column tiles per wave
  static constexpr int kWaves = KV == kF32 ? 4 : 8;              // waves per workgroup
  static constexpr int kWaveCols = 16 * kT;
  static constexpr int kGroupCols = kWaves * kWaveCols;          // columns per workgroup
  static constexpr int kSK = D + 32 / kEs;                       // K tile row stride: +32 bytes
  // V tile row: bf16 tiles 64 bytes, unpadded, the four 16-byte pieces of
  // dimension d at piece q ^ ((d >> 1) & 3); float32 tiles 160 bytes.
  static constexpr int kSV = kLds == kBF16 ? kChunkTokens : kChunkTokens + 32 / kEs;
  static constexpr int kKRowPieces = D / kPerPiece;
  static constexpr int kVRowPieces = kChunkTokens / kPerPiece;
  static constexpr int kKPieces = kChunkTokens * kKRowPieces;
  static constexpr int kVPieces = D * kVRowPieces;
  static constexpr int kThreads = 64 * kWaves;
  // Chunks per barrier: three (96 keys) for the bf16 tiles (three groups of
  // three chunks: 149 KiB of LDS at head_dim 128), one for the float32 tiles.
  // Each barrier lines the waves of a SIMD up in the same phase; between
  // barriers they drift apart and overlap one's MFMAs with the other's
  // vector work, so fewer barriers pay (three chunks per barrier: +3% over
  // two on MI355X).
  static constexpr int kGroupChunks = KV == kF32 ? 1 : 3;
  static constexpr int kKPerThread = (kKPieces + kThreads - 1) / kThreads;
  static constexpr int kVPerThread = (kVPieces + kThreads - 1) / kThreads;
  static constexpr int kKTileElems = kChunkTokens * kSK;
  static constexpr int kVTileElems = D * kSV;
};

// Zero every byte of a 16-byte piece from byte `keep` on.
__device__ __forceinline__ u32x4 keep_bytes(u32x4 v, int keep) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int nb = keep - 4 * w;
    const uint32_t m = nb >= 4 ? 0xFFFFFFFFu : nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u);
    v[w] &= m;
  }
  return v;
}

// K operand of one chunk from the LDS tile: rows x and y of lane (r, j) are
// chunk tokens 8 (r / 4) + (r % 4) and that + 4 (the decode kernel's chunk
// layout), columns as each dtype's score tile expects.
template <int KV, int D>
__device__ __forceinline__ void lds_k(typename PrefillCfg<KV, D>::Tile::K& k,
                                      const typename PrefillCfg<KV, D>::Elem* ks, int r, int j) {
  using C = PrefillCfg<KV, D>;
  const int tx = 8 * (r >> 2) + (r & 3);
  const typename C::Elem* rx = ks + k_row(tx) * C::kSK;
  const typename C::Elem* ry = ks + k_row(tx + 4) * C::kSK;
  if constexpr (KV == kBF16) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      k.x[s] = *reinterpret_cast<const u32x4*>(rx + 32 * s + 8 * j);
      k.y[s] = *reinterpret_cast<const u32x4*>(ry + 32 * s + 8 * j);
    }
  } else {
#pragma unroll
    for (int a = 0; a < D / 16; ++a) {
      k.x[a] = *reinterpret_cast<const f32x4*>(rx + 4 * j + 16 * a);
      k.y[a] = *reinterpret_cast<const f32x4*>(ry + 4 * j + 16 * a);
    }
  }
}

// V operand: lane (r, j) reads dimension 16 u + r, chunk tokens 8 j .. 8 j + 7.
template <int KV, int D>
__device__ __forceinline__ void lds_v(typename PrefillCfg<KV, D>::Tile::V& v,
                                      const typename PrefillCfg<KV, D>::Elem* vs, int r, int j) {
  using C = PrefillCfg<KV, D>;
  // bf16 tiles: piece j of dimension 16 u + r sits at piece j ^ ((r >> 1) & 3)
  const typename C::Elem* base = vs + r * C::kSV + 8 * (KV == kBF16 ? (j ^ ((r >> 1) & 3)) : j);
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const typename C::Elem* p = base + 16 * u * C::kSV;
    if constexpr (KV == kBF16) {
      v.t[u] = *reinterpret_cast<const u32x4*>(p);
    } else {
      v.t[u][0] = *reinterpret_cast<const f32x4*>(p);
      v.t[u][1] = *reinterpret_cast<const f32x4*>(p + 4);
    }
  }
}

// Flip the sign of every element of a query operand (sign bits only: exact).
template <typename Q>
__device__ __forceinline__ void negate_q(Q& q) {
  for (auto& v : q.op) {
    using V = std::remove_reference_t<decltype(v)>;
    constexpr uint32_t kSign = std::is_same_v<V, f32x4> ? 0x80000000u : 0x80008000u;
    u32x4 w = __builtin_bit_cast(u32x4, v);
    w ^= u32x4{kSign, kSign, kSign, kSign};
    v = __builtin_bit_cast(V, w);
  }
}

// Row sums of the weights by the matrix cores: an all-ones A operand times
// P^T gives, in every row of its output, each column's sum over the chunk's
// 32 tokens (of the bf16-rounded weights the P.V product uses).
__device__ __forceinline__ void pv_ones(f32x4& lsum, const bf16x8& pb) {
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, lsum, 0, 0, 0);
}

// acc^T += V^T P^T with the weights already rounded to bf16.
template <int KV, int D>
__device__ __forceinline__ void pv_bf16(f32x4* acc, const typename PrefillCfg<KV, D>::Tile::V& v, const bf16x8& pb) {
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.t[u]), pb, acc[u], 0, 0, 0);
  }
}

template <int KV, int D, bool kPrefix>
__device__ __forceinline__ void prefill_body(const DecodeArgs& a, const int32_t* __restrict__ tables,
                                             const int32_t* __restrict__ lens, const float* __restrict__ k_scale,
                                             const float* __restrict__ v_scale) {
  using C = PrefillCfg<KV, D>;
  using T = typename C::Tile;
  using Elem = typename C::Elem;
  using OutT = typename C::Out;
  constexpr int kT = C::kT;
  constexpr int kTiles = D / 16;
  constexpr size_t kQBytes = (KV == kF32) ? 4 : 2;

  // Three chunk buffers: chunk c + 2 is staged while chunk c is computed and
  // chunk c + 1's operands are read.
  __shared__ __attribute__((aligned(16))) Elem lds_kt[3 * C::kGroupChunks][C::kKTileElems];
  __shared__ __attribute__((aligned(16))) Elem lds_vt[3 * C::kGroupChunks][C::kVTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int j = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = a.group;
  const int L = a.q_len;
  const int NC = a.cols;
  // Prefix mode (shared-prefix decode): one virtual sequence, the shared
  // prefix, whose "query tokens" are the batch's sequences (q_len = batch,
  // q rows [batch][Hq][D]); every column sees all prefix_tokens keys (no
  // causal mask), the keys are cut into pre_segments ranges, one per
  // workgroup, and each workgroup leaves partials: float32 (max, sum) and
  // the unnormalised accumulator in the output's type.
  // (a run-time value inside the prefix instantiation: folding it there
  // lets the compiler hoist more state than the registers hold)
  const bool pm = kPrefix && a.prefix_mode != 0;
  const int pairs = a.num_seqs * Hkv;
  const int ncb = (NC + C::kGroupCols - 1) / C::kGroupCols;
  int bid = blockIdx.x;
  int seg = 0;
  if (pm) {
    seg = bid / (ncb * pairs);
    bid -= seg * ncb * pairs;
  }
  const int cb = pm ? bid / pairs : ncb - 1 - bid / pairs;   // causal: last column tiles (most keys) first
  const int pair = bid - (bid / pairs) * pairs;
  const int b = pair / Hkv;
  const int g = pair - b * Hkv;

  int n;
  if (pm) {
    n = a.prefix_tokens;
  } else {
    n = min(lens[b], a.max_context_len);
    n = (int)min((int64_t)n, (int64_t)a.max_blocks * a.block_size);
    n = max(n, 0);
  }
  const int base = n - L + 1;   // causal: query token i sees tokens < base + i

  // Columns of this lane: tile t holds column col0 + 16 t + r.
  const int col0 = cb * C::kGroupCols + wave * C::kWaveCols;
  int lim[kT];
  int qi[kT], qh[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const int cc = min(col0 + 16 * t + r, NC - 1);
    qi[t] = cc / G;
    qh[t] = cc - qi[t] * G;
    lim[t] = pm ? n : base + qi[t];
  }
  // Keys this wave and this workgroup need: up to their last column's limit
  // (prefix mode: the segment's end), from chunk c_begin on.
  const int wave_last = min(col0 + C::kWaveCols, NC) - 1;
  const int group_last = min(cb * C::kGroupCols + C::kGroupCols, NC) - 1;
  int kend = max(0, base + group_last / G);
  int kend_w = col0 < NC ? max(0, base + wave_last / G) : 0;
  int lim_lo = base + min(col0, NC - 1) / G;   // smallest limit of the wave
  int c_begin = 0;
  if (pm) {
    const int all = (n + kChunkTokens - 1) / kChunkTokens;
    const int per = (all + a.pre_segments - 1) / a.pre_segments;
    c_begin = min(seg * per, all);
    kend = min(n, (c_begin + per) * kChunkTokens);
    kend_w = col0 < NC ? kend : 0;
    lim_lo = n;
  }
  const int nck = max(0, (kend + kChunkTokens - 1) / kChunkTokens - c_begin);   // chunks from c_begin

  // Score scale in log2 units, kept non-negative: a negative scale flips the
  // sign of the queries instead (exact), so the max of the raw scores times
  // sl is the max of the scaled ones and the scale folds into one fma.
  float sl = a.scale * kLog2e;
  float mul = 1.f;
  if constexpr (KV == kFP8) {
    sl *= k_scale[g];
    mul = v_scale[g];
  }
  const bool neg = sl < 0.f;
  sl = fabsf(sl);

  typename T::Q qop[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const uint8_t* row = static_cast<const uint8_t*>(a.q) +
                         (((size_t)b * L + qi[t]) * Hq + (size_t)g * G + qh[t]) * D * kQBytes;
    T::load_q(qop[t], row, col0 + 16 * t + r < NC, j);
    if (neg) negate_q(qop[t]);
  }

  // ---- chunk staging: pool -> registers -> LDS ----
  // Pieces are ordered half-major (tokens 0-15 of the chunk, then 16-31), so
  // every wave's pieces come from one 16-token half: the half's address in
  // the pool is a per-chunk scalar and each thread adds fixed 32-bit offsets.
  //   K piece p: half p / (16 KR), token (p / KR) % 16, dims (p % KR) * kPerPiece
  //   V piece p: half p / (D VH), dim (p / VH) % D, tokens (p % VH) * kPerPiece
  // (KR = pieces per K row, VH = pieces per 16 tokens of a V row).
  const int bs = a.block_size;
  const int bshift = a.block_shift;
  const int32_t* table = tables + (size_t)b * a.max_blocks;
  // entry i of the row, addressed by a 32-bit byte offset (one scalar load
  // with a register offset)
  auto tbl_at = [&](uint32_t i) -> int {
    return *reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(table) + (i << 2));
  };
  const int last_blk = ((n + bs - 1) >> bshift) - 1;
  // A block of either pool holds Hkv tiles of bs x D elements (the pools
  // share the layout); kbase / vbase: this pair's kv head in block 0.
  const uint32_t blk_bytes = (uint32_t)Hkv * (uint32_t)bs * (uint32_t)(D * C::kPs);
  const char* kbase = static_cast<const char*>(a.k_pool) + (size_t)g * bs * D * C::kPs;
  const char* vbase = static_cast<const char*>(a.v_pool) + (size_t)g * bs * D * C::kPs;
  constexpr int KR = C::kKRowPieces;
  constexpr int VH = C::kVRowPieces / 2;
  constexpr int kPs = C::kPs;   // pool element bytes
  uint32_t k_src[C::kKPerThread], v_src[C::kVPerThread];   // byte offsets inside a half
  // LDS element offsets; v_dst2: of an fp8 V piece's second bf16 piece
  // from its first (the swizzle may put it before)
  int k_dst[C::kKPerThread], v_dst[C::kVPerThread], v_dst2[C::kVPerThread];
  int k_half[C::kKPerThread], v_half[C::kVPerThread], v_tok[C::kVPerThread];
#pragma unroll
  for (int i = 0; i < C::kKPerThread; ++i) {
    const int p = tid + C::kThreads * i;
    const int u = (p / KR) % 16, e = p % KR;
    k_half[i] = uni(p / (16 * KR));
    k_src[i] = (uint32_t)((u * D + e * C::kPerPiece) * kPs);
    k_dst[i] = k_row(16 * k_half[i] + u) * C::kSK + e * C::kPerPiece;
  }
#pragma unroll
  for (int i = 0; i < C::kVPerThread; ++i) {
    const int p = tid + C::kThreads * i;
    const int d = (p / VH) % D, q = p % VH;
    v_half[i] = uni(p / (D * VH));
    v_tok[i] = 16 * v_half[i] + q * C::kPerPiece;
    v_src[i] = (uint32_t)((d * bs + q * C::kPerPiece) * kPs);
    if constexpr (C::kLds == kBF16) {
      const int sw = (d >> 1) & 3, lp = v_tok[i] / 8;
      v_dst[i] = d * C::kSV + 8 * (lp ^ sw);
      v_dst2[i] = 8 * (((lp + 1) ^ sw) - (lp ^ sw));
    } else {
      v_dst[i] = d * C::kSV + v_tok[i];
      v_dst2[i] = 8;
    }
  }
  struct Stage {
    u32x4 k[C::kKPerThread];
    u32x4 v[C::kVPerThread];
  } st;

  auto stage_load = [&](int c) {   // c counts from c_begin
    const int t0 = (c_begin + c) * kChunkTokens;
    // Blocks holding the chunk's two 16-token halves, and where each half
    // starts in its block's K tile and V tile (wave-uniform).
    // One 32 x 32-bit product per block gives its offset in both pools.
    // 16-token blocks: the halves are two blocks, each from its first
    // token; larger blocks (multiples of 32): one block holds both halves.
    const char *kb0, *kb1, *vb0, *vb1;
    if (bs == 16) {
      const uint32_t j = (uint32_t)t0 >> 4;   // both reads in flight before either is used
      const int raw0 = tbl_at(min(j, (uint32_t)last_blk));
      const int raw1 = tbl_at(min(j + 1, (uint32_t)last_blk));
      const size_t o0 = (size_t)(uint32_t)min(max(raw0, 0), a.num_blocks - 1) * blk_bytes;
      const size_t o1 = (size_t)(uint32_t)min(max(raw1, 0), a.num_blocks - 1) * blk_bytes;
      kb0 = kbase + o0;
      kb1 = kbase + o1;
      vb0 = vbase + o0;
      vb1 = vbase + o1;
    } else {
      const int raw = tbl_at(min((uint32_t)t0 >> bshift, (uint32_t)last_blk));
      const size_t o = (size_t)(uint32_t)min(max(raw, 0), a.num_blocks - 1) * blk_bytes;
      const uint32_t off = (uint32_t)(t0 & (bs - 1));
      kb0 = kbase + o + off * (uint32_t)(D * kPs);
      kb1 = kb0 + 16 * D * kPs;
      vb0 = vbase + o + off * (uint32_t)kPs;
      vb1 = vb0 + 16 * kPs;
    }
#pragma unroll
    for (int i = 0; i < C::kKPerThread; ++i)
      if (C::kKPieces % C::kThreads == 0 || tid + C::kThreads * i < C::kKPieces)
        st.k[i] = *reinterpret_cast<const u32x4*>((k_half[i] ? kb1 : kb0) + k_src[i]);
#pragma unroll
    for (int i = 0; i < C::kVPerThread; ++i)
      if (C::kVPieces % C::kThreads == 0 || tid + C::kThreads * i < C::kVPieces)
        st.v[i] = *reinterpret_cast<const u32x4*>((v_half[i] ? vb1 : vb0) + v_src[i]);
    // V rows at or past n may hold anything (NaN too): zero them, since
    // their zero weights would not cancel a NaN.  Only a sequence's last
    // chunk has such rows.
    if (t0 + kChunkTokens > n) {
#pragma unroll
      for (int i = 0; i < C::kVPerThread; ++i) {
        const int valid = n - (t0 + v_tok[i]);
        if (valid < C::kPerPiece) st.v[i] = keep_bytes(st.v[i], max(valid, 0) * kPs);
      }
    }
  };
  // A piece of 16 fp8 codes is widened (exactly) to 16 bf16 values: two
  // 16-byte LDS stores.
  auto put = [&](Elem* dst, const u32x4& w, int second) {
    if constexpr (KV == kFP8) {
      *reinterpret_cast<u32x4*>(dst) = fp8x8_to_bf16x8(w[0], w[1]);
      *reinterpret_cast<u32x4*>(dst + second) = fp8x8_to_bf16x8(w[2], w[3]);
    } else {
      *reinterpret_cast<u32x4*>(dst) = w;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kKPerThread; ++i)
      if (C::kKPieces % C::kThreads == 0 || tid + C::kThreads * i < C::kKPieces) put(&lds_kt[buf][k_dst[i]], st.k[i], 8);
#pragma unroll
    for (int i = 0; i < C::kVPerThread; ++i)
      if (C::kVPieces % C::kThreads == 0 || tid + C::kThreads * i < C::kVPieces) put(&lds_vt[buf][v_dst[i]], st.v[i], v_dst2[i]);
  };

  // Per column tile: accumulator, the reference max m_ref of its
  // exponentials (log2 units; always within kRescaleSlack of the running max
  // from below) and the running sum: a register for float32, an MFMA
  // accumulator (four equal copies) for bf16 weights.
  constexpr bool kMfmaSum = KV != kF32;
  // thr: the largest raw score (q . k, before the scale) that keeps a
  // weight within kRescaleSlack of the reference, (m_ref + slack) / sl; a
  // lane whose scores all stay at or below it needs no cross-lane maximum.
  // neg_m: minus the reference the exponentials use (0 for a column that
  // has seen no token, so its weights are 0, never NaN).
  f32x4 acc[kT][kTiles];
  f32x4 lsum[kT];
  float m_ref[kT], thr[kT], neg_m[kT], l_run[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
#pragma unroll
    for (int u = 0; u < kTiles; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[t] = -INFINITY;
    thr[t] = -INFINITY;
    neg_m[t] = 0.f;
    l_run[t] = 0.f;
  }

  // One chunk for this wave's column tiles, in two straight-line phases so
  // that one tile's MFMAs overlap the other's vector work: (A) scores of all
  // tiles, their scaled maxima; a rarely taken rescale; (B) weights and P.V
  // of all tiles.  `kMask`: some column's causal limit falls in the chunk.
  // The chunk's K and V operands (kf, vf) were read from LDS before; once
  // the score MFMAs have taken kf, the next chunk's K operand is read into
  // it (buffer `nbuf`, when `more`), and vf likewise after the P.V MFMAs, so
  // LDS latency hides behind this chunk's work.
  typename T::K kf;
  typename T::V vf;
  auto compute = [&](int t0, int nbuf, bool more, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    f32x4 sx[kT], sy[kT];
    // Wave priority: raised from the score MFMAs through the softmax and
    // dropped for the P.V MFMAs, so that when both waves of a SIMD are ready
    // the one in the earlier phase issues first and the two drift apart,
    // overlapping one's vector work with the other's MFMAs (+1.3% on MI355X).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < kT; ++t) T::scores(kf, qop[t], sx[t], sy[t]);
    if (more) lds_k<C::kLds, D>(kf, lds_kt[nbuf], r, j);
    float s[kT][8];   // raw scores q . k; scaled inside the exponent
    int nvalid[kT];
    bool over = false;
#pragma unroll
    for (int t = 0; t < kT; ++t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s[t][k] = sx[t][k];
        s[t][k + 4] = sy[t][k];
      }
      if constexpr (kMask) {
        nvalid[t] = min(max(lim[t] - (t0 + 8 * j), 0), 8);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k >= nvalid[t]) s[t][k] = -INFINITY;
      }
      // Scores here are finite or -inf: rows past a sequence's end (which
      // may hold NaN) only occur in masked chunks, where they are -inf.
      const float lmax = fmax_nq(fmax_nq(fmax_nq(s[t][0], s[t][1]), fmax_nq(s[t][2], s[t][3])),
                                 fmax_nq(fmax_nq(s[t][4], s[t][5]), fmax_nq(s[t][6], s[t][7])));
      over |= lmax > thr[t];
    }
    // Rare: some lane's scores passed its column's threshold.  Only then are
    // the column maxima formed across the four lanes of each column, and the
    // reference raised where a column's max passes it by more than the slack
    // (the first chunk with a visible token always does).
    if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        float mraw = fmax_nq(fmax_nq(fmax_nq(s[t][0], s[t][1]), fmax_nq(s[t][2], s[t][3])),
                             fmax_nq(fmax_nq(s[t][4], s[t][5]), fmax_nq(s[t][6], s[t][7])));
        mraw = row_max4_nq(mraw);
        const float mloc = mraw == -INFINITY ? -INFINITY : mraw * sl;   // sl >= 0
        if (mloc > m_ref[t] + kRescaleSlack) {
          // a column's first raise gives factor exp2(-inf) = 0 (nothing to keep)
          const float corr = exp2_fast(m_ref[t] - mloc);
#pragma unroll
          for (int u = 0; u < kTiles; ++u) acc[t][u] *= corr;
          if constexpr (kMfmaSum) lsum[t] *= corr;
          else l_run[t] *= corr;
          m_ref[t] = mloc;
          thr[t] = (mloc + kRescaleSlack) / sl;   // +inf when sl == 0: never raised again
          neg_m[t] = -mloc;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      float pk[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pk[k] = exp2_fast(fmaf(s[t][k], sl, neg_m[t]));
        if constexpr (kMask) pk[k] = k < nvalid[t] ? pk[k] : 0.f;   // also when sl == 0
      }
      if constexpr (kMfmaSum) {
        bf16x8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) pb[k] = (__bf16)pk[k];
        __builtin_amdgcn_s_setprio(0);
        pv_bf16<C::kLds, D>(acc[t], vf, pb);
        pv_ones(lsum[t], pb);
      } else {
        __builtin_amdgcn_s_setprio(0);
        l_run[t] += T::pv(acc[t], vf, pk);
      }
    }
    if (more) lds_v<C::kLds, D>(vf, lds_vt[nbuf], r, j);
  };

  // Pipeline over groups of P = kGroupChunks chunks (one barrier per
  // group).  Chunk c lives in LDS buffer P ((c / P) % 3) + c % P.  Before
  // iteration p (chunks P p ...), groups p and p + 1 are in LDS; iteration
  // p stages group p + 2 into group p - 1's buffers, one chunk after each
  // chunk step; group p - 1's operands were read by the end of iteration
  // p - 1 (before the barrier that ended it).
  constexpr int kP = C::kGroupChunks;
  auto bufof = [](int c) { return kP * ((c / kP) % 3) + c % kP; };
  for (int c = 0; c < 2 * kP && c < nck; ++c) {
    stage_load(c);
    stage_store(bufof(c));
  }
  // Every load issued so far (queries included) has landed: without this
  // wait the compiler's counters would treat the query operands as pending
  // inside the loop and make each iteration wait for its own staging loads.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if (nck > 0 && kend_w > 0) {
    lds_k<C::kLds, D>(kf, lds_kt[0], r, j);
    lds_v<C::kLds, D>(vf, lds_vt[0], r, j);
  }
  // The loop body covers all three groups (3P chunks), so every chunk's
  // LDS buffer is a compile-time constant (immediate LDS offsets).
  constexpr int kRing = 3 * kP;
  for (int c = 0; c < nck; c += kRing) {
#pragma unroll
    for (int h = 0; h < kRing; ++h) {
      const int cc = c + h;   // bufof(cc) == h
      if (cc + 2 * kP < nck) stage_load(cc + 2 * kP);   // its loads fly while chunk cc is computed
      const int t0 = (c_begin + cc) * kChunkTokens;
      if (cc < nck && t0 < kend_w) {
        const bool more = t0 + kChunkTokens < kend_w;   // this wave computes chunk cc + 1 too
        const int nbuf = (h + 1) % kRing;
        if (t0 + kChunkTokens > lim_lo) compute(t0, nbuf, more, std::true_type{});
        else compute(t0, nbuf, more, std::false_type{});
      }
      if (cc + 2 * kP < nck) stage_store((h + 2 * kP) % kRing);
      if (h % kP == kP - 1) __syncthreads();
    }
  }

  if (pm) {   // partials of this key segment: (reference max, sum), unnormalised accumulator
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      float l_tot;
      if constexpr (kMfmaSum) l_tot = lsum[t][0];
      else l_tot = row_sum4(l_run[t]);
      if (col0 + 16 * t + r < NC) {
        const size_t slot = ((size_t)seg * L + qi[t]) * Hq + (size_t)g * G + qh[t];
        OutT* dst = static_cast<OutT*>(a.pre_acc) + slot * D + 4 * j;   // the output's type
#pragma unroll
        for (int u = 0; u < kTiles; ++u) store4<OutT>(dst + 16 * u, acc[t][u] * mul);
        if (j == 0) *reinterpret_cast<float2*>(a.pre_ml + slot * 2) = float2{m_ref[t], l_tot};
      }
    }
    return;
  }
  OutT* out = static_cast<OutT*>(a.out);
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    float l_tot;
    if constexpr (kMfmaSum) l_tot = lsum[t][0];
    else l_tot = row_sum4(l_run[t]);
    if (col0 + 16 * t + r < NC) {
      const float f = l_tot > 0.f ? mul / l_tot : 0.f;   // a query that sees no token gets zeros
      OutT* dst = out + (((size_t)b * L + qi[t]) * Hq + (size_t)g * G + qh[t]) * D + 4 * j;
#pragma unroll
      for (int u = 0; u < kTiles; ++u) store4<OutT>(dst + 16 * u, acc[t][u] * f);
    }
  }
}

// Tables, lengths and scales as restrict parameters: nothing the kernel
// writes aliases them, so their wave-uniform reads use the scalar cache.
template <int KV, int D, bool kPrefix>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                    const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  prefill_body<KV, D, kPrefix>(a, tables, lens, k_scale, v_scale);
}

template <int KV, int D, bool kPrefix>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel_wide(DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                         const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  prefill_body<KV, D, kPrefix>(a, tables, lens, k_scale, v_scale);
}

template <int KV, int D, bool kPrefix>
hipError_t launch_prefill_p(const DecodeArgs& a, hipStream_t stream) {
  using C = PrefillCfg<KV, D>;
  const int64_t ncb = (a.cols + C::kGroupCols - 1) / C::kGroupCols;
  const int64_t grid = ncb * a.num_seqs * a.num_kv_heads * (kPrefix ? a.pre_segments : 1);
  if (grid <= 0) return hipSuccess;
  if constexpr (KV == kF32)
    hipLaunchKernelGGL((prefill_kernel_wide<KV, D, kPrefix>), dim3((unsigned)grid), dim3(C::kThreads), 0, stream,
                       a, a.block_tables, a.context_lens, a.k_scale, a.v_scale);
  else
    hipLaunchKernelGGL((prefill_kernel<KV, D, kPrefix>), dim3((unsigned)grid), dim3(C::kThreads), 0, stream, a,
                       a.block_tables, a.context_lens, a.k_scale, a.v_scale);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_prefill_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.prefix_mode) return launch_prefill_p<KV, D, true>(a, stream);
  return launch_prefill_p<KV, D, false>(a, stream);
}

}  // namespace

int64_t prefill_groups(const DecodeArgs& a) {
  const int cols = a.kv_dtype == kF32 ? PrefillCfg<kF32, 64>::kGroupCols : PrefillCfg<kBF16, 64>::kGroupCols;
  return ((int64_t)a.cols + cols - 1) / cols * a.num_seqs * a.num_kv_heads * (a.prefix_mode ? a.pre_segments : 1);
}

int prefill_group_cols(int kv_dtype) {
  return kv_dtype == kF32 ? PrefillCfg<kF32, 64>::kGroupCols : PrefillCfg<kBF16, 64>::kGroupCols;
}

hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) {
    if (a.kv_dtype == kF32) return launch_prefill_t<kF32, 64>(a, stream);
    if (a.kv_dtype == kBF16) return launch_prefill_t<kBF16, 64>(a, stream);
    return launch_prefill_t<kFP8, 64>(a, stream);
  }
  if (a.kv_dtype == kF32) return launch_prefill_t<kF32, 128>(a, stream);
  if (a.kv_dtype == kBF16) return launch_prefill_t<kBF16, 128>(a, stream);
  return launch_prefill_t<kFP8, 128>(a, stream);
}

}  // namespace pkv
