// The split kernel's per-wave body (stream-K walk over a batch's 32-token
// chunks, gfx950): the plain decode kernel and the tail walk of the
// one-launch shared-prefix decode are both built from it.  Device-only; each
// kernel source that includes it gets its own copy (anonymous namespace).
//
// What is computed: the Habr KV-Cache article (habr.com/ru/articles/1021832),
// sections 2-5, as the decode kernel's source states; the block comment
// above split_body gives the schedule.
#pragma once

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

}  // namespace
}  // namespace pkv
