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

#include <atomic>

#include "pkv_internal.h"
#include "tile_math.h"

namespace pkv {
namespace {

// Tokens of a sequence that this call reads: its length clamped to the
// caller's bound and the table's capacity; in the tail pass of a
// shared-prefix decode (kTail), minus the prefix's table_offset blocks.
template <bool kTail>
__device__ __forceinline__ int clamp_len(int n, const DecodeArgs& a) {
  n = min(n, a.max_context_len);
  n = (int)min((int64_t)n, (int64_t)a.max_blocks * a.block_size);
  if constexpr (kTail) n -= a.table_offset * a.block_size;
  return max(n, 0);
}

// Chunks of one sequence: 32-token steps covering its n tokens.
__device__ __forceinline__ int chunks_of(int n) { return (n + kChunkTokens - 1) / kChunkTokens; }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int t = __shfl_up(v, s);
    if (lane >= s) v += t;
  }
  return v;
}

// Position of a chunk in the global order: pairs (b, g) head-major, chunk c
// of the pair's cb chunks, global chunk index x.  All fields are
// wave-uniform.
struct Pos {
  int b, g, c, cb, n;
  int64_t x;
};

// ---------------------------------------------------------------------------
// Split kernel.
//
// The batch's work is the list of 32-token chunks of every (sequence, kv head)
// pair, pairs ordered head-major.  Worker wave w (one per SIMD slot of the
// GPU, all resident at once) takes the contiguous chunk range
// [w*K, (w+1)*K), K = ceil(chunks / workers), so every wave streams the same
// number of bytes.  It walks its range pair by pair with one online-softmax
// state.  A pair that lies wholly inside the range is finished at once.  A
// pair shared with other waves (at most the first and the last pair of a
// range) leaves a float32 partial (max, sum, unnormalised accumulator) in slot
// w + (the pair's place in the order) of the workspace; slots are unique
// because ranges are contiguous and ordered.  The wave that holds a pair's first chunk records the pair's
// first wave and number of parts for the merge kernel.
// ---------------------------------------------------------------------------
template <int KV, int D, bool KNT, bool VNT, bool kTail>
__device__ __forceinline__ void split_body(const DecodeArgs& a, const int32_t* __restrict__ tables,
                                            const int32_t* __restrict__ lens, const float* __restrict__ k_scale,
                                            const float* __restrict__ v_scale) {
  using T = typename TileOf<KV, D>::type;
  using OutT = typename TileOf<KV, D>::Out;
  using Elem = typename T::Elem;
  constexpr int kTiles = D / 16;
  constexpr size_t kQBytes = (KV == kF32) ? 4 : 2;

  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int j = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round robin; renumber them so that
  // each XCD's workgroups take consecutive ranges (one kv head's chunks each
  // when there are 8 kv heads): blocks shared by several sequences are then
  // re-read from that XCD's own L2.
  int blk = blockIdx.x;
  if ((gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int wid = __builtin_amdgcn_readfirstlane(blk * kDecodeWaves + (threadIdx.x >> 6));
  const int W = a.num_workers;
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int L = a.q_len;       // query tokens per sequence (1 for decode)
  const int NC = a.cols;       // MFMA columns in use: L * G (query token, query head) pairs
  OutT* out = static_cast<OutT*>(a.out);
  // Column r of this lane: query token qi, head qh of the pair's group
  // (padding columns r >= NC repeat the last real one and are never stored).
  const int rc = min(r, NC - 1);
  const int qi = rc / G;
  const int qh = rc - qi * G;

  // ---- chunk totals over the batch ----
  int64_t total = 0;   // chunks per kv head over the batch
  int n_lane = 0;      // length of sequence `lane` (kept when the batch has <= 64 sequences)
  for (int base = 0; base < B; base += 64) {
    const int bi = base + lane;
    n_lane = bi < B ? clamp_len<kTail>(lens[bi], a) : 0;
    total += uni(wave_sum(chunks_of(n_lane)));
  }
  // Length of sequence b: from the registers when the whole batch fits one
  // wave, else a scalar load.
  auto seq_len = [&](int b) -> int {
    if (B <= 64) return uni(__builtin_amdgcn_readlane(n_lane, uni(b)));
    return uni(clamp_len<kTail>(lens[uni(b)], a));
  };
  // Sequences with no tokens: wave b mod W writes their zero output and a
  // (first wave 0, parts 0) record per pair, so every pair has a fresh record
  // and the merge kernel never needs the lengths.
  for (int b = wid; b < B; b += W) {
    if (seq_len(b) != 0) continue;
    if constexpr (!kTail) {   // in the tail pass the merge kernel writes every output
      OutT* o = out + (size_t)b * L * Hq * D;
      for (int e = lane; e < L * Hq * D; e += 64) o[e] = (OutT)0.f;
    }
    for (int g = lane; g < Hkv; g += 64) a.pair_meta[b * Hkv + g] = int2{0, 0};
  }

  const int64_t C = total * Hkv;
  const int64_t K = (C + W - 1) / W;
  const int64_t x0 = (int64_t)wid * K;
  if (x0 >= C) return;
  const int64_t x1 = min(x0 + K, C);
  const int nch = (int)(x1 - x0);

  // Chunks are ordered head-major: kv head g's list is every sequence's
  // chunks in sequence order, total chunks per head.  Chunk x0 is chunk r0 of
  // head g0's list, in the sequence with before(b) <= r0 < before(b) + cb.
  const int g0 = uni((int)(x0 / total));
  const int64_t r0 = x0 - (int64_t)g0 * total;
  int b0 = 0;
  int64_t before0 = 0;
  {
    int64_t run = 0;
    for (int base = 0; base < B; base += 64) {
      const int bi = base + lane;
      const int cb = bi < B ? chunks_of(B <= 64 ? n_lane : clamp_len<kTail>(lens[bi], a)) : 0;
      const int incl = wave_inclusive_scan(cb, lane);
      const int64_t ex = run + incl - cb;
      const bool hit = cb > 0 && ex <= r0 && r0 < ex + cb;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(hit);
      if (mask) {
        const int idx = uni(__builtin_ctzll(mask));
        b0 = uni(base + idx);
        before0 = run + uni(__builtin_amdgcn_readlane(incl - cb, idx));
        break;
      }
      run += uni(__builtin_amdgcn_readlane(incl, 63));
    }
  }
  Pos pos;
  pos.b = b0;
  pos.n = seq_len(b0);
  pos.cb = chunks_of(pos.n);
  pos.x = x0;
  pos.g = g0;
  pos.c = uni((int)(r0 - before0));
  auto advance = [&](Pos q) -> Pos {
    ++q.x;
    if (++q.c == q.cb) {
      q.c = 0;
      do {   // next sequence (then next head), skipping empty ones; a next chunk exists, so this ends
        if (++q.b == B) {
          q.b = 0;
          ++q.g;
        }
        q.n = seq_len(q.b);
        q.cb = chunks_of(q.n);
      } while (q.cb == 0);
    }
    return q;
  };

  const int bsz = a.block_size;         // tokens per block: 16 or a multiple of 32
  const int bshift = a.block_shift;     // log2(bsz)
  const size_t blk_stride = (size_t)Hkv * bsz * D;   // elements per block
  // Physical ids of the blocks holding a chunk's two 16-token halves, tokens
  // 32 c + 16 h of the sequence: logical block (32 c + 16 h) / bsz (two
  // blocks at bsz = 16, one block otherwise).  Scalar loads, fetched one
  // chunk ahead of their use, so the table lookup never delays a prefetch.
  struct Ids {
    int id0, id1;
  };
  auto block_ids = [&](const Pos& q) -> Ids {
    const int32_t* table = tables + (size_t)q.b * a.max_blocks;
    const int last = ((q.n + bsz - 1) >> bshift) - 1;
    const int t0 = q.c * kChunkTokens;
    return Ids{table[uni(min(t0 >> bshift, last))], table[uni(min((t0 + 16) >> bshift, last))]};
  };

  // Query operand (and fp8 scales) of a pair.  Lane (r, j) holds head g*G + r;
  // padding columns r >= G hold zeros.  The chunk that opens a pair loads the
  // pair's query into its own buffer's slot (qA / qB) together with its K/V;
  // the operand qop takes it over when that chunk is computed.  One slot per
  // buffer keeps the load counters exact: a prefetch never writes a register
  // the current chunk reads.
  typename T::Q qop, qA, qB;
  auto load_q = [&](typename T::Q& qq, const Pos& q) {
    const uint8_t* row = static_cast<const uint8_t*>(a.q) +
                         (((size_t)q.b * L + qi) * Hq + q.g * G + qh) * D * kQBytes;
    T::load_q(qq, row, r < NC, j);
  };
  auto log2_scale = [&](int g) -> float {
    float sl = a.scale * kLog2e;
    if constexpr (KV == kFP8) sl *= k_scale[g];
    return sl;
  };
  auto out_scale = [&](int g) -> float {
    if constexpr (KV == kFP8) return v_scale[g];
    return 1.f;
  };

  auto issue = [&](typename T::K& kb, typename T::V& vb, typename T::Q& qn, const Pos& q, const Ids& ids) {
    const int id0 = uni(min(max(ids.id0, 0), a.num_blocks - 1));
    const int id1 = uni(min(max(ids.id1, 0), a.num_blocks - 1));
    const int t0 = q.c * kChunkTokens;
    const int off0 = t0 & (bsz - 1);          // the halves' offsets inside their blocks
    const int off1 = (t0 + 16) & (bsz - 1);
    const Elem* kp = static_cast<const Elem*>(a.k_pool) + (size_t)q.g * bsz * D;
    const Elem* vp = static_cast<const Elem*>(a.v_pool) + (size_t)q.g * bsz * D;
    const bool hk = (r >> 3) != 0;            // K rows: half by score row
    const bool hv = (j >> 1) != 0;            // V rows: half by lane group
    T::template load_k<KNT>(kb, kp + (size_t)(hk ? id1 : id0) * blk_stride + (size_t)(hk ? off1 : off0) * D, r, j);
    T::template load_v<VNT>(vb, vp + (size_t)(hv ? id1 : id0) * blk_stride + (hv ? off1 : off0), r, j, bsz);
    if (q.c == 0) load_q(qn, q);   // first chunk of a pair: its query rides along
  };

  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  float sl = log2_scale(pos.g);
  int seg_c0 = pos.c;      // first chunk of the current segment

  auto flush = [&](const Pos& q) {
    const float l_tot = row_sum4(l_run);
    const float mul = out_scale(q.g);
    const int pair = q.b * Hkv + q.g;
    if (seg_c0 == 0) {   // this wave holds the pair's first chunk: record its parts
      const int64_t s0 = q.x - q.c;
      const int parts = (int)((s0 + q.cb - 1) / K - s0 / K) + 1;
      if (lane == 0) a.pair_meta[pair] = int2{wid, parts};
    }
    if (seg_c0 == 0 && q.c == q.cb - 1 && !kTail) {   // the whole pair: finish it here
      if (r < NC) {
        OutT* dst = out + (((size_t)q.b * L + qi) * Hq + q.g * G + qh) * D + 4 * j;
        const float f = l_tot > 0.f ? mul / l_tot : 0.f;   // a query that sees no token gets zeros
#pragma unroll
        for (int t = 0; t < kTiles; ++t) store4<OutT>(dst + 16 * t, acc[t] * f);
      }
    } else {
      const size_t slot = (size_t)wid + (size_t)q.g * B + q.b;   // wave + the pair's place in the chunk order
      if (r < NC) {
        float* dst = a.ws_acc + (slot * NC + r) * D + 4 * j;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t) = acc[t] * mul;
        if (j == 0) {
          a.ws_ml[(slot * NC + r) * 2] = m_run;
          a.ws_ml[(slot * NC + r) * 2 + 1] = l_tot;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    seg_c0 = 0;
  };

  auto compute = [&](typename T::K& kb, typename T::V& vb, const typename T::Q& qn, const Pos& q,
                     bool last_of_range) {
    if (q.c == 0) {   // a new pair begins: switch query and scales
      qop = qn;
      sl = log2_scale(q.g);
    }
    const int t0 = q.c * kChunkTokens;
    f32x4 sx, sy;
    T::scores(kb, qop, sx, sy);
    float t[8] = {sx[0] * sl, sx[1] * sl, sx[2] * sl, sx[3] * sl,
                  sy[0] * sl, sy[1] * sl, sy[2] * sl, sy[3] * sl};
    // Query token qi sits at position n - L + qi and sees the tokens below
    // n - L + 1 + qi (causal; for decode, L = 1: every token below n).  V
    // rows at or past n are zeroed, since they may hold anything (NaN too).
    if (t0 + kChunkTokens > q.n - L + 1) {
      const int nvalid = min(max(q.n - L + 1 + qi - (t0 + 8 * j), 0), 8);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k >= nvalid) t[k] = -INFINITY;
      T::mask_v(vb, min(max(q.n - (t0 + 8 * j), 0), 8));
    }
    float mloc = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                       fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
    mloc = row_max4(mloc);
    const float m_new = fmaxf(m_run, mloc);
    // A column that has seen no token yet (several query tokens: a chunk past
    // an early query's position) keeps max -inf.  It is exponentiated against
    // 0 instead, so that its weights and its rescale factor are 0, never
    // exp2(-inf - -inf).
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {   // some column's max grew
      const float corr = exp2_fast(m_run - m_use);
#pragma unroll
      for (int u = 0; u < kTiles; ++u) acc[u] *= corr;
      l_run *= corr;
    }
    m_run = m_new;
    float pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pk[k] = exp2_fast(t[k] - m_use);
    l_run += T::pv(acc, vb, pk);
    if (q.c == q.cb - 1 || last_of_range) flush(q);
  };

  // Two register buffers: chunk k+1's loads are in flight while chunk k is
  // computed.  The steady-state loop issues its prefetch unconditionally so
  // that the compiler's load counters wait only for the buffer in use.
  load_q(qop, pos);
  {
    typename T::K kA, kB;
    typename T::V vA, vB;
    Pos pa = pos, pb;
    Ids ia = block_ids(pa), ib;
    issue(kA, vA, qA, pa, ia);
    if (nch > 1) {
      pb = advance(pa);
      ib = block_ids(pb);
    }
    int k = 0;
    for (; k + 2 < nch; k += 2) {
      issue(kB, vB, qB, pb, ib);
      const Pos pn = advance(pb);       // chunk k+2 exists
      ia = block_ids(pn);
      compute(kA, vA, qA, pa, false);
      pa = pn;
      issue(kA, vA, qA, pa, ia);
      // chunk k+3, when there is one (otherwise its ids are not needed)
      const Pos pm = k + 3 < nch ? advance(pa) : pa;
      ib = block_ids(pm);
      compute(kB, vB, qB, pb, false);
      pb = pm;
    }
    if (k + 1 < nch) {
      issue(kB, vB, qB, pb, ib);
      compute(kA, vA, qA, pa, false);
      compute(kB, vB, qB, pb, true);
    } else {
      compute(kA, vA, qA, pa, true);
    }
  }

}

// ---------------------------------------------------------------------------
// Prefix part of the one-launch shared-prefix decode (bf16 caches).  The
// kernel below runs it in waves 4-7 of each workgroup, beside a tail walk in
// waves 0-3, so each SIMD holds one wave of each: the tail wave mostly waits
// on HBM while the prefix wave keeps the matrix cores busy.
//
// For kv head g the batch's query heads are the columns c = b * G + h, every
// one of which sees all prefix tokens (no mask but the prefix's end).  A
// workgroup's kPrefixWaves prefix waves share one (kv head, key segment) and
// own consecutive groups of kCols columns (two 16-column MFMA tiles each):
// work items (kv head, the workgroup's column groups, segment), head-major,
// are dealt to the workgroups, so the workgroups of one XCD read one head's
// prefix blocks from that XCD's L2.  Each 32-token chunk of the segment is
// staged once for all prefix waves into a ring of kRingSlots LDS slots,
// kAhead chunks ahead, by direct pool-to-LDS loads (global_load_lds_dwordx4,
// each wave its share of the chunk's pieces).  A slot holds the chunk as the
// MFMA operand pieces of every lane (piece i of lane l at 1024 i + 16 l: K
// rows, then V dims, as the decode tiles load them), so each wave reads its
// operands back with conflict-free 16-byte reads.
//
// The prefix waves hand slots to each other through two LDS counters per
// slot that only grow: `arrive` (a wave adds 64 once its share of the
// slot's current chunk has landed) and `done` (a wave adds 64 once it has
// read the chunk).  With N = 64 kPrefixWaves, chunk s of the workgroup's
// sequence lives in slot s % kRingSlots; it is staged once done has reached
// N (s / kRingSlots) (chunk s - kRingSlots read by all) and read once arrive
// has reached N (s / kRingSlots + 1).  All prefix waves walk the same chunk
// sequence, so every wait is met: a wave stages chunk s + kAhead only after
// all have read chunk s + kAhead - kRingSlots (the waves may drift apart by
// up to kRingSlots - kAhead - 1 chunks), and each wait is bounded besides.
// The LDS traffic of this part is inline assembly: the compiler would
// otherwise wait for every direct load in flight before any LDS access.
//
// It leaves the segment's partials, (max in log2 units, sum) and the
// unnormalised accumulator in bf16, in the layout the merge kernel reads:
// row s * (B * Hq) + b * Hq + g * G + h for segment s.
// ---------------------------------------------------------------------------
constexpr int kRingSlots = 8;     // 128 KiB of LDS at head_dim 128
constexpr int kAhead = 3;         // chunks staged ahead of the one being read
constexpr int kPrefixWaves = 4;   // prefix waves per workgroup: one per SIMD

template <int D>
struct PrefixRing {
  static constexpr int kPieces = D / 8;                         // 16-byte operand pieces per lane per chunk
  static constexpr int kPerWave = kPieces / kPrefixWaves;       // pieces each prefix wave stages
  static constexpr int kSlotBytes = kPieces * 1024;
  static constexpr uint32_t kGen = 64u * kPrefixWaves;          // counter step per ring generation
  static_assert(kPerWave >= 1 && kPieces % kPrefixWaves == 0, "pieces split over the prefix waves");
};

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The wave adds 64 to an LDS counter, from one lane (64 lanes adding to one
// address would serialise on its bank).
__device__ __forceinline__ void lds_count(uint32_t addr, int lane) {
  if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(64u) : "memory");
}

// Waits until an LDS counter reaches `target` (bounded: 2^22 polls of about
// 64 cycles; never reached when all prefix waves walk the same sequence).
__device__ __forceinline__ void lds_wait_for(uint32_t addr, uint32_t target) {
  for (int it = 0; it < (1 << 22); ++it) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    if (uni((int)v) - (int)target >= 0) return;
    __builtin_amdgcn_s_sleep(1);
  }
}

// The chunk's 16 (head_dim 128) or 8 (head_dim 64) operand pieces of this
// lane, read from a ring slot; returns once they have arrived.
template <int D>
__device__ __forceinline__ void lds_read_chunk(typename TileBF16<D>::K& k, typename TileBF16<D>::V& v,
                                               uint32_t a) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1024\n\t"
        "ds_read_b128 %2, %16 offset:2048\n\tds_read_b128 %3, %16 offset:3072\n\t"
        "ds_read_b128 %4, %16 offset:4096\n\tds_read_b128 %5, %16 offset:5120\n\t"
        "ds_read_b128 %6, %16 offset:6144\n\tds_read_b128 %7, %16 offset:7168\n\t"
        "ds_read_b128 %8, %16 offset:8192\n\tds_read_b128 %9, %16 offset:9216\n\t"
        "ds_read_b128 %10, %16 offset:10240\n\tds_read_b128 %11, %16 offset:11264\n\t"
        "ds_read_b128 %12, %16 offset:12288\n\tds_read_b128 %13, %16 offset:13312\n\t"
        "ds_read_b128 %14, %16 offset:14336\n\tds_read_b128 %15, %16 offset:15360\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k.x[0]), "=&v"(k.x[1]), "=&v"(k.x[2]), "=&v"(k.x[3]), "=&v"(k.y[0]), "=&v"(k.y[1]),
          "=&v"(k.y[2]), "=&v"(k.y[3]), "=&v"(v.t[0]), "=&v"(v.t[1]), "=&v"(v.t[2]), "=&v"(v.t[3]),
          "=&v"(v.t[4]), "=&v"(v.t[5]), "=&v"(v.t[6]), "=&v"(v.t[7])
        : "v"(a)
        : "memory");
  } else {
    static_assert(D == 64, "head_dim 64 or 128");
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k.x[0]), "=&v"(k.x[1]), "=&v"(k.y[0]), "=&v"(k.y[1]), "=&v"(v.t[0]), "=&v"(v.t[1]),
          "=&v"(v.t[2]), "=&v"(v.t[3])
        : "v"(a)
        : "memory");
  }
}

// s_waitcnt immediate for "at most n vector memory operations pending"
// (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int D>
__device__ __forceinline__ void prefix_waves_body(const DecodeArgs& a, const int32_t* __restrict__ tables,
                                                  char* ring, uint32_t* ctr) {
  using T = TileBF16<D>;
  using R = PrefixRing<D>;
  constexpr int kTiles = D / 16;
  constexpr int kCols = shared_group_cols(D);
  constexpr int kT = kCols / 16;   // column tiles per wave
  constexpr int kSteps = D / 32;
  static_assert(kCols * kPrefixWaves == shared_workgroup_cols(D), "columns per workgroup");

  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int j = lane >> 4;
  const int pw = uni((threadIdx.x >> 6) - kDecodeWaves);   // prefix wave of the workgroup
  const int nwg = gridDim.x;
  int blk = blockIdx.x;
  if ((nwg & 7) == 0) blk = (blk & 7) * (nwg >> 3) + (blk >> 3);
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int NCp = B * G;                                    // prefix columns per kv head
  const int QD = (NCp + shared_workgroup_cols(D) - 1) / shared_workgroup_cols(D);   // column groups of a workgroup
  const int P = a.prefix_tokens;                            // whole blocks, > 0
  const int S = a.pre_segments;
  const int all = (P + kChunkTokens - 1) / kChunkTokens;
  const int per = (all + S - 1) / S;                        // every segment holds >= 1 chunk
  const int64_t items = (int64_t)Hkv * QD * S;
  const int bsz = a.block_size;
  const int bshift = a.block_shift;
  const int last_blk = (P >> bshift) - 1;
  const size_t blk_stride = (size_t)Hkv * bsz * D;
  const size_t stride = (size_t)B * Hq;                     // partial rows per segment
  // Row 0 of the table from its first block (the kernel's table pointer is
  // the tail walk's, table_offset blocks in); every row starts with the same
  // prefix blocks.
  const int32_t* table0 = tables - a.table_offset;
  const uint32_t ring0 = lds_u32(ring);
  const uint32_t arrive0 = lds_u32(ctr);
  const uint32_t done0 = lds_u32(ctr + kRingSlots);
  const uint32_t lane_off = 16u * lane;

  uint32_t seq = 0;   // chunks the workgroup has staged before this item
  for (int64_t item = blk; item < items; item += nwg) {
    const int g = uni((int)(item / ((int64_t)QD * S)));
    const int rem = uni((int)(item - (int64_t)g * QD * S));
    const int qd = uni(rem / S);
    const int seg = uni(rem - qd * S);
    const int c0 = seg * per;
    const int n = min(c0 + per, all) - c0;
    const int cg = qd * kPrefixWaves + pw;

    typename T::Q qop[kT];
    int col[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      col[t] = cg * kCols + 16 * t + r;
      const int cc = min(col[t], NCp - 1);
      const int b = cc / G;
      const uint8_t* row = static_cast<const uint8_t*>(a.q) + ((size_t)b * Hq + (size_t)g * G + (cc - b * G)) * D * 2;
      T::load_q(qop[t], row, col[t] < NCp, j);
    }
    // The queries have landed before any chunk is staged: the compiler's
    // load counters then never see them pending inside the chunk loop (where
    // they would make every chunk wait for all staging in flight).
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // Score scale in log2 units, kept non-negative: a negative scale flips
    // the queries' sign bits instead (exact), so the max of the raw scores
    // times sl is the max of the scaled ones and the scale folds into one fma.
    float sl = a.scale * kLog2e;
    if (sl < 0.f) {
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
          qop[t].op[u] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qop[t].op[u]) ^
                                                        u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
      sl = -sl;
    }

    const uint16_t* kp = static_cast<const uint16_t*>(a.k_pool) + (size_t)g * bsz * D;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v_pool) + (size_t)g * bsz * D;
    const bool hk = (r >> 3) != 0;   // K rows: half by score row
    const bool hv = (j >> 1) != 0;   // V rows: half by lane group
    // Stage this wave's quarter of chunk c (item chunk c, sequence number q).
    auto stage = [&](uint32_t q, int c) {
      const uint32_t slot = q % kRingSlots;
      lds_wait_for(done0 + 4 * slot, R::kGen * (q / kRingSlots));   // its previous chunk read by all
      const int t0 = (c0 + c) * kChunkTokens;
      const int id0 = uni(min(max(table0[uni(min(t0 >> bshift, last_blk))], 0), a.num_blocks - 1));
      const int id1 = uni(min(max(table0[uni(min((t0 + 16) >> bshift, last_blk))], 0), a.num_blocks - 1));
      const int off0 = t0 & (bsz - 1);
      const int off1 = (t0 + 16) & (bsz - 1);
      const uint16_t* ktile = kp + (size_t)(hk ? id1 : id0) * blk_stride + (size_t)(hk ? off1 : off0) * D;
      const uint16_t* vtile = vp + (size_t)(hv ? id1 : id0) * blk_stride + (hv ? off1 : off0);
      char* dst = ring + slot * R::kSlotBytes;
#pragma unroll
      for (int e = 0; e < R::kPerWave; ++e) {
        const int i = pw * R::kPerWave + e;   // piece index: K x rows, K y rows, then V dims
        const uint16_t* src;
        if (i < kSteps) src = ktile + row_token(r, 0) * D + 8 * j + 32 * i;
        else if (i < 2 * kSteps) src = ktile + row_token(r, 1) * D + 8 * j + 32 * (i - kSteps);
        else src = vtile + r * bsz + 8 * (j & 1) + (size_t)(i - 2 * kSteps) * 16 * bsz;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 0, 0);
      }
    };

    // Per column tile: accumulator, row sums (an MFMA accumulator: four
    // equal copies) and the reference max m_ref of the exponentials (log2
    // units), raised only when a column's max passes it by more than
    // kSharedSlack, so weights stay below 2^kSharedSlack and most chunks
    // skip the rescale.
    constexpr float kSharedSlack = 8.f;
    f32x4 acc[kT][kTiles];
    f32x4 lsum[kT];
    float m_ref[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
#pragma unroll
      for (int u = 0; u < kTiles; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -INFINITY;
    }
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

    for (int c = 0; c < kAhead && c < n; ++c) stage(seq + c, c);
    for (int c = 0; c < n; ++c) {
      const uint32_t q = seq + c;
      const uint32_t slot = q % kRingSlots;
      if (c + kAhead < n) {
        stage(q + kAhead, c + kAhead);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAhead * R::kPerWave));   // own share of chunk c landed
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      lds_count(arrive0 + 4 * slot, lane);
      lds_wait_for(arrive0 + 4 * slot, R::kGen * (q / kRingSlots + 1));
      typename T::K kb;
      typename T::V vb;
      lds_read_chunk<D>(kb, vb, ring0 + slot * R::kSlotBytes + lane_off);
      lds_count(done0 + 4 * slot, lane);

      const int t0 = (c0 + c) * kChunkTokens;
      // a prefix of 16 (mod 32) tokens ends inside its last chunk: rows past
      // it get weight 0 and zeroed V (they may hold anything, NaN too)
      const int nvalid = min(max(P - (t0 + 8 * j), 0), 8);
      const bool cut = t0 + kChunkTokens > P;
      if (cut) T::mask_v(vb, nvalid);
      f32x4 sx[kT], sy[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t) T::scores(kb, qop[t], sx[t], sy[t]);
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        float sc[8] = {sx[t][0], sx[t][1], sx[t][2], sx[t][3], sy[t][0], sy[t][1], sy[t][2], sy[t][3]};
        if (cut) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k >= nvalid) sc[k] = -INFINITY;
        }
        // raw scores are finite or -inf; the scale (>= 0) applies after the max
        float mraw = fmax_nq(fmax_nq(fmax_nq(sc[0], sc[1]), fmax_nq(sc[2], sc[3])),
                             fmax_nq(fmax_nq(sc[4], sc[5]), fmax_nq(sc[6], sc[7])));
        mraw = row_max4_nq(mraw);
        const float mloc = mraw == -INFINITY ? -INFINITY : mraw * sl;
        const bool raise = mloc > m_ref[t] + kSharedSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
          // a column's first raise gives factor exp2(-inf) = 0 (nothing to keep)
          const float corr = raise ? exp2_fast(m_ref[t] - mloc) : 1.f;
#pragma unroll
          for (int u = 0; u < kTiles; ++u) acc[t][u] *= corr;
          lsum[t] *= corr;
          if (raise) m_ref[t] = mloc;
        }
        const float m_use = m_ref[t] == -INFINITY ? 0.f : m_ref[t];
        bf16x8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float pk = exp2_fast(fmaf(sc[k], sl, -m_use));
          if (cut) pk = k < nvalid ? pk : 0.f;   // also when sl == 0
          pb[k] = (__bf16)pk;
        }
#pragma unroll
        for (int u = 0; u < kTiles; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vb.t[u]), pb, acc[t][u], 0, 0, 0);
        lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, lsum[t], 0, 0, 0);
      }
    }
    seq += n;

#pragma unroll
    for (int t = 0; t < kT; ++t) {
      const float l_tot = lsum[t][0];
      if (col[t] < NCp) {
        const int b = col[t] / G;
        const size_t slot = seg * stride + (size_t)b * Hq + (size_t)g * G + (col[t] - b * G);
        __bf16* dst = static_cast<__bf16*>(a.pre_acc) + slot * D + 4 * j;
#pragma unroll
        for (int u = 0; u < kTiles; ++u) store4<__bf16>(dst + 16 * u, acc[t][u]);
        if (j == 0) *reinterpret_cast<float2*>(a.pre_ml + slot * 2) = float2{m_ref[t], l_tot};
      }
    }
  }
}

// The shared-prefix decode's tail walk and prefix part in one launch:
// eight-wave workgroups, waves 0-3 the tail walk (worker ids as in the split
// kernel), waves 4-7 the prefix part; two waves per SIMD, at most 256
// registers each.  The prefix waves issue first when both kinds are ready
// (wave priority): they are the longer part, and a tail wave's next loads
// are already in flight while it computes.  Measured on MI355X (256
// sequences over a 4,096-token prefix, tails of 64-512 tokens, bf16): 82.2
// µs per call with the merge, 98.7 with equal priorities, 99.3 with the tail
// waves first; the three-launch path takes 95.3.
constexpr int kSharedThreads = 64 * (kDecodeWaves + kPrefixWaves);

template <int D, bool KNT, bool VNT>
__global__ __launch_bounds__(kSharedThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_shared_kernel(DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens) {
  __shared__ __attribute__((aligned(1024))) char ring[kRingSlots * PrefixRing<D>::kSlotBytes];
  __shared__ uint32_t ctr[2 * kRingSlots];   // arrive, then done, per slot
  if (threadIdx.x < 2 * kRingSlots) ctr[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x < 64 * kDecodeWaves) {
    split_body<kBF16, D, KNT, VNT, true>(a, tables, lens, nullptr, nullptr);
  } else {
    __builtin_amdgcn_s_setprio(3);
    prefix_waves_body<D>(a, tables, ring, ctr);
  }
}

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

template <int D>
hipError_t launch_shared_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.num_workers / kDecodeWaves);
  if (a.kv_reread || a.block_size > 32)
    hipLaunchKernelGGL((decode_shared_kernel<D, false, false>), dim3(grid), dim3(kSharedThreads), 0, stream, a,
                       a.block_tables, a.context_lens);
  else
    hipLaunchKernelGGL((decode_shared_kernel<D, true, true>), dim3(grid), dim3(kSharedThreads), 0, stream, a,
                       a.block_tables, a.context_lens);
  return hipGetLastError();
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

hipError_t launch_shared(const DecodeArgs& a, hipStream_t stream) {
  if (a.kv_dtype != kBF16) return hipErrorInvalidValue;
  return a.head_dim == 64 ? launch_shared_t<64>(a, stream) : launch_shared_t<128>(a, stream);
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
