// Shared-prefix decode in one launch for gfx950: the tail walk of every
// sequence and the prefix part, which reads the blocks the batch shares once
// for all its sequences.
//
// What is computed (Habr KV-Cache article, habr.com/ru/articles/1021832):
//  - section 4 "Copy-on-Write for parallel sampling": the variants of one
//    prompt reference the same physical blocks; here they are also read
//    once per call, not once per sequence;
//  - section 3 "Recalling FlashAttention": each sequence's output is the
//    exact softmax over its whole context, reached from partial results
//    (max, sum, unnormalised accumulator) over the prefix's key segments
//    and over the tail, combined by the decode's merge kernel.
// "Chapter 8 - Next-generation KV cache" (LLM Primer VI), section 8.1:
// best-of-n sampling keeps one copy of the prompt's blocks.

#include "pkv_internal.h"
#include "split_body.h"
#include "tile_math.h"

namespace pkv {
namespace {

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
    // skip the rescale.  thr is the largest raw score (before the scale)
    // that stays within the slack, (m_ref + slack) / sl: a lane whose scores
    // all stay at or below it needs no cross-lane maximum.  neg_m is minus
    // the reference the exponentials use (0 before a column's first token).
    constexpr float kSharedSlack = 8.f;
    f32x4 acc[kT][kTiles];
    f32x4 lsum[kT];
    float m_ref[kT], thr[kT], neg_m[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
#pragma unroll
      for (int u = 0; u < kTiles; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -INFINITY;
      thr[t] = -INFINITY;
      neg_m[t] = 0.f;
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
      float sc[kT][8];
      bool over = false;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sc[t][k] = sx[t][k];
          sc[t][k + 4] = sy[t][k];
        }
        if (cut) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k >= nvalid) sc[t][k] = -INFINITY;
        }
        // raw scores are finite or -inf; the scale (>= 0) applies after the max
        const float lmax = fmax_nq(fmax_nq(fmax_nq(sc[t][0], sc[t][1]), fmax_nq(sc[t][2], sc[t][3])),
                                   fmax_nq(fmax_nq(sc[t][4], sc[t][5]), fmax_nq(sc[t][6], sc[t][7])));
        over |= lmax > thr[t];
      }
      // rare: some lane passed its column's threshold; only then the column
      // maxima across lanes, and a raise where one passes the slack
      if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          float mraw = fmax_nq(fmax_nq(fmax_nq(sc[t][0], sc[t][1]), fmax_nq(sc[t][2], sc[t][3])),
                               fmax_nq(fmax_nq(sc[t][4], sc[t][5]), fmax_nq(sc[t][6], sc[t][7])));
          mraw = row_max4_nq(mraw);
          const float mloc = mraw == -INFINITY ? -INFINITY : mraw * sl;
          if (mloc > m_ref[t] + kSharedSlack) {
            // a column's first raise gives factor exp2(-inf) = 0 (nothing to keep)
            const float corr = exp2_fast(m_ref[t] - mloc);
#pragma unroll
            for (int u = 0; u < kTiles; ++u) acc[t][u] *= corr;
            lsum[t] *= corr;
            m_ref[t] = mloc;
            thr[t] = (mloc + kSharedSlack) / sl;   // +inf when sl == 0: never raised again
            neg_m[t] = -mloc;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        bf16x8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float pk = exp2_fast(fmaf(sc[t][k], sl, neg_m[t]));
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

// The merge after the one launch (one query token per sequence, bf16, at
// most kSegs prefix segments).  The same combination, in the same
// order, as the decode's merge kernel in its shared-prefix form: the pair's
// tail pieces with the online-softmax rescale, then the column's prefix
// segments, their maximum first.  Here a column's prefix partials are
// loaded first, before the pair's record is read, so that their round trip
// and the record's overlap and only the tail partials wait for the record.
// Every one of the kSegs loads is made (past the last segment they repeat
// it and are not used), so that they are issued back to back.
template <int D, int kSegs>
__global__ __launch_bounds__(256) void shared_merge_kernel(const int2* __restrict__ meta,
                                                           const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml, __bf16* __restrict__ out,
                                                           int num_seqs, int num_kv_heads, int group,
                                                           const __bf16* __restrict__ pre_acc,
                                                           const float* __restrict__ pre_ml, int pre_segments) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  const int pair = blockIdx.x;
  const int G = group;   // the pair's columns: its G query heads
  const int b = pair / num_kv_heads;
  const int g = pair - b * num_kv_heads;
  const size_t place = (size_t)g * num_seqs + b;   // the pair's place in the head-major chunk order
  const size_t Hq = (size_t)num_kv_heads * G;
  const size_t stride = (size_t)num_seqs * Hq;     // partial rows per prefix segment
  for (int e = threadIdx.x; e < G * (D / 4); e += blockDim.x) {
    const int c = e / (D / 4);
    const int q4 = e % (D / 4);
    const size_t col = (size_t)b * Hq + (size_t)g * G + c;
    float2 pml[kSegs];
    u32x2v pacc[kSegs];   // four bf16 values, widened where they are used
#pragma unroll
    for (int s = 0; s < kSegs; ++s) {
      const size_t slot = (size_t)min(s, pre_segments - 1) * stride + col;
      pml[s] = *reinterpret_cast<const float2*>(pre_ml + slot * 2);
      pacc[s] = *reinterpret_cast<const u32x2v*>(pre_acc + slot * D + 4 * q4);
    }
    // keeps the compiler from reading the record before those loads
    asm volatile("" ::: "memory");
    const int2 m = meta[pair];
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int w = m.x; w < m.x + m.y; ++w) {
      const size_t slot = ((size_t)w + place) * G + c;
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
    float Mp = -INFINITY;
#pragma unroll
    for (int s = 0; s < kSegs; ++s)
      if (s < pre_segments) Mp = fmaxf(Mp, pml[s].x);
    const float M2 = fmaxf(M, Mp);
    const float M2u = M2 == -INFINITY ? 0.f : M2;
    const float f_old = exp2_fast(M - M2u);
    L *= f_old;
    o *= f_old;
#pragma unroll
    for (int s = 0; s < kSegs; ++s) {
      if (s < pre_segments) {
        const f32x4 acc_s = {__builtin_bit_cast(float, pacc[s][0] << 16),
                             __builtin_bit_cast(float, pacc[s][0] & 0xFFFF0000u),
                             __builtin_bit_cast(float, pacc[s][1] << 16),
                             __builtin_bit_cast(float, pacc[s][1] & 0xFFFF0000u)};
        const float w = exp2_fast(pml[s].x - M2u);
        L += pml[s].y * w;
        o += acc_s * w;
      }
    }
    __bf16* dst = out + ((size_t)b * Hq + (size_t)g * G + c) * D + 4 * q4;
    store4<__bf16>(dst, o * (L > 0.f ? 1.f / L : 0.f));
  }
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.q_len != 1 || a.pre_segments < 1 || a.pre_segments > 16) return launch_merge(a, stream);
  const dim3 pairs((unsigned)a.num_seqs * (unsigned)a.num_kv_heads);
  const dim3 threads(a.group * (D / 4) > 128 ? 256 : 128);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, pairs, threads, 0, stream, static_cast<const int2*>(a.pair_meta),
                       static_cast<const float*>(a.ws_acc), static_cast<const float*>(a.ws_ml),
                       static_cast<__bf16*>(a.out), a.num_seqs, a.num_kv_heads, a.group,
                       static_cast<const __bf16*>(a.pre_acc), a.pre_ml, a.pre_segments);
    return hipGetLastError();
  };
  if (a.pre_segments <= 4) return go(shared_merge_kernel<D, 4>);
  if (a.pre_segments <= 8) return go(shared_merge_kernel<D, 8>);
  return go(shared_merge_kernel<D, 16>);
}

}  // namespace

hipError_t launch_shared(const DecodeArgs& a, hipStream_t stream) {
  if (a.kv_dtype != kBF16) return hipErrorInvalidValue;
  return a.head_dim == 64 ? launch_shared_t<64>(a, stream) : launch_shared_t<128>(a, stream);
}

}  // namespace pkv
