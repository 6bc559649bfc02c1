/*
 * pkv.h - paged KV-cache decode attention on AMD MI355X (gfx950).
 *
 * Plain C ABI: device pointers, sizes and a HIP stream handle, nothing else.
 * The library allocates no memory and keeps no pointer after a call returns;
 * its only global state is a per-device cache of the compute-unit count and
 * the static scratch buffer of pkv_paged_decode_static.
 * Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 * NULL for the default stream).
 *
 * The operation follows the source pages:
 *  - Habr KV-Cache article (habr.com/ru/articles/1021832), section 4
 *    "Recalling PagedAttention": the cache is a pool of fixed 16-token
 *    blocks that need not be contiguous; a per-sequence block table maps
 *    logical block j to a physical block id.
 *  - Same article, section 5 "How vLLM combines FlashAttention and
 *    PagedAttention": one decode call takes one query per sequence and head,
 *    the K and V caches, an int32 block table [batch, max_num_blocks] of
 *    physical ids, and the true length of each sequence; the kernel gathers
 *    the scattered blocks itself.
 *  - Same article, section 3 "Recalling FlashAttention": the result is exact
 *    attention softmax(q K^T * scale) V, reached with an online softmax.
 *  - Same article, section 1 "Prefill and Decode": each decode step appends
 *    the new token's K and V to the cache.
 *
 * Layout (this library's choice; one (block, kv head) tile is contiguous):
 *   q       [num_seqs][num_q_heads][head_dim]                 q_dtype
 *   out     [num_seqs][num_q_heads][head_dim]                 q_dtype
 *   k_pool  [num_blocks][num_kv_heads][B][head_dim]           kv_dtype (token-major tile)
 *   v_pool  [num_blocks][num_kv_heads][head_dim][B]           kv_dtype (dim-major tile)
 *   block_tables [num_seqs][max_blocks_per_seq] int32 physical block ids
 *   context_lens [num_seqs] int32, tokens held by each sequence
 *   slot_mapping [num_tokens] int64, slot = block * B + offset
 * where B = desc->block_size tokens per block.
 * Query head h reads kv head h / (num_q_heads / num_kv_heads): contiguous
 * query groups share a kv head (grouped-query attention, Habr article
 * section 2, "GQA: 8x reduction").
 *
 * Status: every function returns PKV_OK (0) or a negative PKV_E* code.
 * Argument checks run on the host before any HIP call.  Data-dependent
 * conditions are not checked on the host; the kernels keep every access in
 * bounds regardless (see each function).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL (-1)       /* null pointer, bad size or shape */
#define PKV_EUNSUPPORTED (-2) /* dtype / head_dim / group size not built */
#define PKV_EWORKSPACE (-3)   /* workspace missing or too small */
#define PKV_ELAUNCH (-4)      /* the HIP runtime reported an error (host: out of memory) */
#define PKV_ENOSPACE (-5)     /* the block pool has too few free blocks */
#define PKV_ESCRATCH (-6)     /* pkv_paged_decode_static: batch too large for the static scratch */

#define PKV_BLOCK_SIZE 16   /* the default; 32, 64, 128 and 256 are supported too */

typedef enum pkv_dtype {
  PKV_F32 = 0,      /* IEEE binary32 */
  PKV_BF16 = 1,     /* bfloat16 */
  PKV_FP8_E4M3 = 2  /* OCP E4M3FN, one float32 scale per kv head */
} pkv_dtype;

/* Shape and format of one layer's cache.
 * Supported: head_dim 64 or 128; block_size 16, 32, 64, 128 or 256 tokens
 * (Habr article, section 4, "Choosing the block size": 16 is the default;
 * larger blocks shrink the table for very long sequences at the cost of up
 * to block_size - 1 unused slots per sequence); num_q_heads a multiple of
 * num_kv_heads with at most 16 query heads per kv head; (kv, q) dtypes
 * (F32, F32), (BF16, BF16) or (FP8_E4M3, BF16).  For FP8 caches, k_scale and
 * v_scale are device arrays [num_kv_heads] of float32: a stored code c of
 * head h means decode(c) * scale[h].  They must be NULL for other dtypes. */
typedef struct pkv_cache_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t kv_dtype;
  int32_t q_dtype;
  const float* k_scale;
  const float* v_scale;
  uint32_t flags;         /* PKV_KV_* hints below; 0 by default */
} pkv_cache_desc;

/* flags: the decode reads blocks that several sequences of the batch share
 * (prefix sharing, parallel sampling; "Why one character breaks the cache",
 * section on a block serving many requests).  K/V are then loaded with
 * ordinary cached loads, so a shared block read again later in the call is
 * served from the caches.  Without it every K/V byte is assumed to be read
 * once and is streamed with non-temporal loads, which are faster on MI355X
 * for data read once.  A hint only: the result is the same bits either way. */
#define PKV_KV_REREAD 1u

/* Write the K and V of num_tokens new tokens into their slots.
 * (Habr article, section 1: one new token per sequence is appended each
 * decode step; section 4, step-by-step example: it goes to the next slot of
 * the sequence's last block, the caller opening a fresh block when full.)
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_dim]; q_dtype for an
 *                 FP8 cache (quantised here), else kv_dtype (bit copy)
 *   slot_mapping  device [num_tokens]; a slot outside [0, num_blocks * B) is
 *                 padding and writes nothing
 *   k_pool, v_pool device pools, updated in place
 * k_new, v_new and the pools must be 16-byte aligned (else PKV_EINVAL).
 * FP8: code = E4M3 round-to-nearest-even, saturating to +-448, of the IEEE
 * float32 quotient x / scale[h].  Slots must be distinct and must not lie in
 * blocks shared with other sequences; what two tokens with the same slot
 * leave there is unspecified.  num_tokens == 0 is a no-op.
 * One kernel.  Below 1,024 tokens (a decode step's appends): one wave per
 * (token, kv head).  From 1,024 tokens: workgroups of one kv head take
 * groups of 16 consecutive new tokens in turn; each token's K row is written
 * as 16-byte pieces, and when the 16 slots are 16 consecutive rows of one
 * block (a prefill chunk's appends) the V tile's 16 columns go through LDS
 * and out row by row, otherwise each V column element by element. */
int pkv_kv_append(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int32_t num_tokens, void* k_pool,
                  void* v_pool, void* stream);

/* Copy whole blocks, for copy-on-write.  For every i < num_pairs, block
 * dst[i] of both pools (all kv heads, all 16 token slots) becomes a copy of
 * block src[i] (all B token slots).  (Habr article, section 4, "Copy-on-Write for parallel
 * sampling": a sequence that must modify a block other sequences reference
 * copies it first and the original stays untouched; section 8 applies it to
 * a speculative correction.  The host allocator chooses dst and moves the
 * sequence's table entry; this call moves the bytes, before any write to
 * dst.)
 *   k_pool, v_pool  device pools as for pkv_kv_append, updated in place
 *   src, dst        device int32 [num_pairs]; a pair with either id outside
 *                   [0, num_blocks) is skipped
 * Destinations must be distinct and none may also be a source in the same
 * call: the pairs are copied in parallel.  Bytes are copied as they are
 * (any dtype; fp8 codes keep their per-head scales).  num_pairs == 0 is a
 * no-op. */
int pkv_copy_blocks(const pkv_cache_desc* desc, void* k_pool, void* v_pool,
                    const int32_t* src, const int32_t* dst, int32_t num_pairs,
                    void* stream);

/* Number of worker waves pkv_paged_decode uses for this batch shape on the
 * current device: one per SIMD (4 per compute unit), fewer for batches with
 * fewer 32-token chunks; always a multiple of 4.  Returns a negative status on bad arguments
 * or when no device is current. */
int32_t pkv_decode_workers(const pkv_cache_desc* desc, int32_t num_seqs,
                           int32_t max_context_len);

/* Device workspace bytes a decode of this shape needs: (num_workers +
 * num_seqs * num_kv_heads) partial states of group * (head_dim + 2) floats,
 * then one (first wave, parts) record of two int32 per (sequence, kv head)
 * pair.  num_workers == 0 means pkv_decode_workers(...).  Returns 0 on bad
 * arguments. */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs,
                                  int32_t max_context_len, int32_t num_workers);

/* Decode attention for one query token per sequence over its paged cache:
 *   out[b][h] = softmax_t(scale * q[b][h] . K_b[t]) V_b[t],  t < context_lens[b]
 * where K_b / V_b are sequence b's tokens gathered through its block table,
 * and h reads kv head h / group.  Only table entries j < ceil(n / B) are
 * read; token slots at or past n in the last block are ignored (they may
 * hold anything, NaN included).  A sequence of length 0 gets a zero output.
 * Lengths are taken as min(context_lens[b], max_context_len,
 * B * max_blocks_per_seq); block ids are clamped into [0, num_blocks).
 * Accumulation is float32; out is rounded once to q_dtype (nearest even).
 *
 * Two kernels on `stream`.  The batch's 32-token chunks of every (sequence,
 * kv head) pair, pairs in kv-head-major order (every sequence of kv head 0,
 * then of kv head 1, ...), are cut into equal contiguous
 * ranges, one per worker wave; each wave runs section 3's online softmax over
 * its range and finishes every pair it covers completely; sequences of length
 * 0 get their zero output there too.  For a pair split between waves each wave
 * leaves a float32 partial state (running max, sum, unnormalised
 * accumulator); the second kernel merges them with the same rescale by
 * exp(m_old - m_new).
 *   workspace  device buffer of pkv_decode_workspace_bytes(..., 0) bytes,
 *              16-byte aligned; scratch, needs no initialisation.  Calls that
 *              share one workspace must be ordered (one stream). */
int pkv_paged_decode(const pkv_cache_desc* desc, const void* q, const void* k_pool,
                     const void* v_pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_decode with an explicit worker count (a positive multiple of 4, or
 * 0 for pkv_decode_workers(...)); the workspace must be sized for that count.
 * Any count gives the same result up to float32 rounding. */
int pkv_paged_decode_ex(const pkv_cache_desc* desc, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_context_len, float scale,
                        int32_t num_workers, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* pkv_paged_decode for callers that cannot allocate device memory at all:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and the default worker count, so the result
 * is pkv_paged_decode's, bit for bit; the workspace is the library's own
 * static device buffer of PKV_STATIC_SCRATCH_BYTES, of which every device
 * the library runs on holds one copy until the process ends.  This call
 * allocates and frees nothing (its first call on a device looks up that
 * device's copy).  A batch whose workspace,
 * pkv_decode_workspace_bytes(desc, num_seqs, max_context_len, 0), exceeds
 * the buffer is refused with PKV_ESCRATCH before any launch.  The buffer
 * needs no initialisation; every call on a device shares it, so calls that
 * overlap on one device (any streams, any threads) race and must be
 * ordered by the caller.  Other arguments, errors and clamping as for
 * pkv_paged_decode. */
#define PKV_STATIC_SCRATCH_BYTES (32u << 20)
int pkv_paged_decode_static(const pkv_cache_desc* desc, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                            void* stream);

/* Decode over a batch whose sequences all begin with the same shared blocks
 * (parallel sampling or best-of-n over one prompt: Habr article, section 4,
 * "Copy-on-Write for parallel sampling", where the variants reference the
 * prompt's physical blocks instead of copies; LLM Primer, "Chapter 8 —
 * Next-generation KV cache", 8.1: best-of-8 on a 2,000-token prompt).  The
 * result is
 * pkv_paged_decode_ex's for the same arguments, up to float32 rounding
 * order; the prefix's blocks are read from HBM once per call instead of once
 * per sequence.
 *   prefix_tokens  tokens at the start of every sequence held in the same
 *                  blocks: entries j < prefix_tokens / B of every table row
 *                  equal row 0's.  A multiple of the block size B, at most
 *                  max_context_len and B * max_blocks_per_seq (else
 *                  PKV_EINVAL); 0 runs pkv_paged_decode_ex.  Every
 *                  sequence's (clamped) length must be at least prefix_tokens;
 *                  for one that is not, or a row that differs in the prefix,
 *                  the output is unspecified (no access leaves the pools).
 * The work: every sequence's query heads over the prefix (row 0's blocks)
 * as the columns of one (virtual) sequence per kv head, the prefix cut into
 * key segments, leaving partials per segment (float32 max and sum; the
 * unnormalised accumulator in the output's type: bf16 unless the cache is
 * float32); each sequence's tokens after the prefix, leaving partials only;
 * then a merge of both sets of partials per (sequence, head) with section
 * 3's rescale, which writes out.  Kernels on `stream`: for a bf16 cache
 * whose worker count gives every SIMD one tail wave (4 per compute unit,
 * the default once the tails have enough 32-token chunks), two: one kernel whose workgroups run the tail walk and the prefix part
 * side by side, then the merge; otherwise three: the many-query kernel
 * over the prefix, the decode split kernel over the tails, the merge.
 *   workspace  pkv_shared_decode_workspace_bytes(...) bytes (same num_workers),
 *              16-byte aligned scratch; calls sharing it must be ordered. */
/* Whether pkv_paged_decode_shared is expected to beat pkv_paged_decode_ex
 * for this batch: 1 when the prefix bytes the plain decode would read again,
 * (num_seqs - 1) * prefix_tokens * 2 * num_kv_heads * head_dim * element
 * size, reach 192 MiB (the crossover measured on MI355X), else 0; a negative
 * PKV_E* code on bad arguments.  Host arithmetic only. */
int32_t pkv_shared_prefix_pays(const pkv_cache_desc* desc, int32_t num_seqs, int32_t prefix_tokens);

size_t pkv_shared_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs,
                                         int32_t max_context_len, int32_t prefix_tokens,
                                         int32_t num_workers);

int pkv_paged_decode_shared(const pkv_cache_desc* desc, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t prefix_tokens,
                            float scale, int32_t num_workers, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Host block pool with a prefix-cache index (no GPU work; not thread-safe:
 * one scheduler thread owns a pool).
 *
 * Habr article, section 7 "That same Cache Read": every full block carries a
 * hash of all tokens from the start of the sequence; a flat table maps block
 * hash -> physical block; a request walks its blocks from block 0 and the
 * first miss ends the hit; hit blocks gain a reference; unreferenced blocks
 * stay cached until memory runs short and then the least recently used one
 * is evicted; cached blocks are never modified.  "Why one character breaks
 * the cache", section on the git-style hash chain: hash(block j) =
 * H(hash(block j-1), extra keys, tokens of block j), block 0's parent being a
 * fixed seed; a hit never covers the request's last token; a hit on a free
 * block takes it out of the LRU queue.
 *
 * Here H is SHA-256 over: the parent hash (32 bytes, all zero for block 0),
 * extra_key (8 bytes little-endian: a tenant salt, adapter id, ...), and the
 * block's token ids (4 bytes little-endian each).  Only full blocks are
 * hashed.  The pool owns no KV memory: block ids index the caller's pools.
 * ------------------------------------------------------------------------- */
typedef struct pkv_block_pool pkv_block_pool;

/* A pool of num_blocks free blocks of block_size tokens, handed out in id
 * order at first.  NULL on bad arguments or when out of host memory. */
pkv_block_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size);
void pkv_pool_destroy(pkv_block_pool* pool);

/* Longest cached prefix of a request of num_tokens tokens: walks the chained
 * hashes of its full blocks from block 0, stops at the first miss and at
 * floor((num_tokens - 1) / block_size) blocks (the last token is always
 * computed), and at cap.  Each hit block gains one reference (a free one
 * leaves the LRU queue); their ids go to blocks_out.  Returns the number of
 * hit blocks (block_size times that many tokens are reusable) or a negative
 * status. */
int32_t pkv_pool_match_prefix(pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens,
                              uint64_t extra_key, int32_t* blocks_out, int32_t cap);

/* Take count blocks from the head of the LRU queue (reference count 1); a
 * cached block is removed from the index first (evicted).  Returns count, or
 * PKV_ENOSPACE (nothing taken) when fewer blocks are free. */
int32_t pkv_pool_allocate(pkv_block_pool* pool, int32_t count, int32_t* blocks_out);

/* Index the full blocks of a request whose K/V are now computed: block
 * blocks[j] holds tokens [j*B, (j+1)*B) of tokens.  A block already indexed,
 * or whose hash another block already holds, is left as it is.  Every listed
 * full block must be referenced.  Returns the number of blocks added. */
int32_t pkv_pool_cache_blocks(pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens,
                              uint64_t extra_key, const int32_t* blocks, int32_t num_blocks);

/* Add one reference to each listed block: another sequence now shares it
 * (a fork for parallel sampling or beam search: Habr article, section 4,
 * "Copy-on-Write for parallel sampling", where the variants point at the
 * prompt's blocks and each block counts its references).  Every listed
 * block must already be referenced (else PKV_EINVAL and nothing changes). */
int pkv_pool_ref(pkv_block_pool* pool, const int32_t* blocks, int32_t num_blocks);

/* Drop one reference from each listed block (a request finished).  Blocks
 * reaching zero join the tail of the LRU queue, the request's last block
 * first, so that a chain's tail is evicted before its head; they stay in the
 * index.  Nothing changes if any id is invalid or over-released. */
int pkv_pool_free(pkv_block_pool* pool, const int32_t* blocks, int32_t num_blocks);

/* Chained hashes (32 bytes each) of the first min(floor(num_tokens / B), cap)
 * full blocks of a token sequence.  Returns how many were written. */
int pkv_pool_block_hash(const pkv_block_pool* pool, const int32_t* tokens, int32_t num_tokens,
                        uint64_t extra_key, uint8_t* hashes_out, int32_t cap);

/* Counters: free blocks, indexed blocks, references of one block, evictions. */
int32_t pkv_pool_num_free(const pkv_block_pool* pool);
int32_t pkv_pool_num_cached(const pkv_block_pool* pool);
int32_t pkv_pool_ref_count(const pkv_block_pool* pool, int32_t block);
int64_t pkv_pool_evictions(const pkv_block_pool* pool);

/* Attention of several query tokens per sequence over its paged cache, for
 * speculative verification and chunked prefill.  (Habr article,
 * section 6 "Chunked Prefill": a chunk of new tokens runs next to decode
 * tokens and attends to everything cached before it; "Chapter 8 -
 * Next-generation KV cache", closing section: speculative decoding verifies
 * several drafted tokens in one pass.)  The q_len new tokens of each
 * sequence are already in the cache (appended first), so sequence b holds
 * n = context_lens[b] >= q_len tokens and query token i sits at position
 * n - q_len + i:
 *   out[b][i][h] = softmax_t(scale * q[b][i][h] . K_b[t]) V_b[t],  t <= n - q_len + i
 *   q, out   [num_seqs][q_len][num_q_heads][head_dim], q_dtype
 * All other arguments, the lengths' clamping and the result for q_len == 1
 * are those of pkv_paged_decode_ex (which is this call with q_len == 1).  A
 * query that sees no token (n < q_len) gets zeros.
 * Kernels: with at most 16 query columns (q_len * (num_q_heads /
 * num_kv_heads) (query token, head) pairs per kv head) the call runs the
 * decode's split and merge kernels, all of a group's columns sharing one
 * 16-column matrix tile; with more (chunked prefill) it runs one many-query
 * kernel in which every workgroup owns up to 256 columns of one (sequence,
 * kv head) pair and walks all its keys, and num_workers and the workspace
 * are not used (workspace may be NULL).  More than 2^24 columns is
 * PKV_EUNSUPPORTED; q_len < 1 is PKV_EINVAL.
 *   workspace  pkv_attention_workspace_bytes(...) bytes, as for decode. */
int pkv_paged_attention(const pkv_cache_desc* desc, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t q_len, int32_t max_context_len, float scale,
                        int32_t num_workers, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes of pkv_paged_attention: as pkv_decode_workspace_bytes with
 * q_len * group columns per partial state; a nominal 256 for more than 16
 * columns (the many-query kernel uses none).  0 on bad arguments. */
size_t pkv_attention_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs, int32_t q_len,
                                     int32_t max_context_len, int32_t num_workers);

/* Static description of a status code. */
const char* pkv_strerror(int status);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
