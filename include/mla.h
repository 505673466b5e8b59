/*
 * mla.h -- C ABI of the MI355X (gfx950) paged MLA decode library (libmla.so).
 *
 * Operation.  Decode attention for Multi-head Latent Attention over a paged
 * latent KV cache.  Every query head attends to one shared latent key row per
 * token: the first 512 dims are the compressed latent c_t, the last 64 the rope
 * key.  Scores use the absorbed query q~ = [W_UK^T q_nope ; q_rope] against the
 * whole 576-wide row (the absorption identity q.(W_UK c) = (W_UK^T q).c of the
 * "FlashMLA inference acceleration" notes, dpshk.com/news/5996785, §2.1), and
 * the output is the softmax-weighted sum of the latent part (the first dv = 512
 * dims); the caller applies W_UV afterwards.  Softmax runs over the whole
 * cached sequence and equals the textbook result (same notes, §2.2, online
 * softmax).  The two calls mirror the FlashMLA API -- one metadata call from the
 * sequence lengths, then the paged decode with 64-token pages addressed through
 * block_table and cache_seqlens, query heads folded onto their KV head
 * ("OpenSourceWeek Day 1 -- Demystifying DeepSeek's FlashMLA",
 * deepseekonline.chat, §II.1, §II.2, §V.2).
 *
 * For batch b, query token s < s_q, query head h, KV head k = h / (h_q / h_kv),
 * L = cache_seqlens[b]:
 *   N        = L, or max(0, L - s_q + s + 1) when causal (the s_q queries are
 *              the newest s_q cached tokens, so query s sees keys t <= L-s_q+s)
 *   K_t      = kcache[block_table[b][t / 64], t % 64, k, 0:576],  t < N
 *   x_t      = softmax_scale * (q[b,s,h,:] . K_t)
 *   out      = sum_t softmax(x)_t * K_t[0:512]          (bf16, round-to-nearest-even)
 *   lse      = ln(sum_t exp(x_t))                       (fp32, natural log)
 *   N == 0   => out = 0, lse = -inf
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers; every buffer is caller-owned; the
 *     library allocates no device memory and keeps no state between calls.
 *   - Calls are asynchronous: they validate their arguments on the host, enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the null stream) and return.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Return value: MLA_OK or a negative status; mla_last_error() then gives a
 *     message (thread-local).  Argument checks run before any HIP call, so an
 *     invalid call touches no device state.
 *   - Data-dependent validity (cache_seqlens <= max_blocks * 64, page ids
 *     referenced by the first ceil(L/64) block_table entries in [0, num_pages))
 *     is the caller's contract.  The kernels never read outside the cache: an
 *     out-of-range page id is read as a page of zeros.
 *   - Layouts are dense row-major: q [batch, s_q, h_q, 576] bf16,
 *     kcache [num_pages, 64, h_kv, 576] bf16, block_table [batch, max_blocks]
 *     int32, cache_seqlens [batch] int32, out [batch, s_q, h_q, 512] bf16,
 *     lse [batch, s_q, h_q] fp32.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID (-1)     /* null pointer, non-positive size, h_q % h_kv != 0, num_parts mismatch */
#define MLA_ERR_UNSUPPORTED (-2) /* d_qk != 576, dv != 512, page size != 64, batch above MLA_MAX_BATCH */
#define MLA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than mla_plan's size */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call failed; see mla_last_error() */
#define MLA_ERR_CAPACITY (-5)    /* page allocator: no free page, or more pages than max_blocks */
#define MLA_ERR_RANGE (-6)       /* mla_pager_page_owner: page id out of range, or state not initialised */

#define MLA_PAGE_BLOCK_SIZE 64
#define MLA_D_QK 576
#define MLA_DV 512
#define MLA_METADATA_INTS 8  /* ints per tile_metadata row */
#define MLA_FP8_ROW_BYTES 656 /* FP8 cache row: 512 e4m3 + 4 fp32 scales + 64 bf16 */
#define MLA_MAX_BATCH 8192   /* sequences per call (metadata kernel keeps prefix sums on chip) */

/*
 * mla_plan -- host only, launches nothing.
 * Chooses the number of parts P the split-KV scheduler cuts the work into and
 * the workspace size mla_decode_paged needs.
 *   batch        number of sequences (1..MLA_MAX_BATCH)
 *   rows_per_kv  s_q * h_q / h_kv: query rows that share one KV head
 *                (the fold of the Day-1 page §II.1 and the second argument of
 *                get_mla_metadata in §V.2)
 *   h_kv         KV heads (>= 1)
 *   dv           value width, must be 512
 *   num_cus      compute units to plan for; 0 = query the current device
 *   num_parts    out: P (>= 1)
 *   workspace_bytes out: bytes of device workspace for mla_decode_paged
 *                (batch + P) * h_kv * rows_per_kv * (dv + 1) * 4
 * Errors: MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP (device query).
 */
int mla_plan(int batch, int rows_per_kv, int h_kv, int dv, int num_cus,
             int* num_parts, size_t* workspace_bytes);

/*
 * mla_tile_rows -- host only.  Query rows one workgroup owns for a given
 * rows_per_kv (16 or 64); the decode grid has ceil(rows/tile) row tiles.
 */
int mla_tile_rows(int rows_per_kv);

/*
 * mla_get_metadata -- split-KV schedule for one decode step (the
 * get_mla_metadata call of the Day-1 page §V.2; the variable-length balancing
 * the "Flash MLA: efficient MLA decoding kernel library for variable-length
 * sequences" page, developer.baidu.com, motivates in §二).
 * One kernel on `stream` reads cache_seqlens and writes
 *   tile_metadata [num_parts, 8] int32: per part
 *       {first_seq, first_block, last_seq, end_block_of_last_seq, first_chunk_ordinal, 0, 0, 0}
 *       (an empty part is {batch, 0, batch, 0, 0, 0, 0, 0});
 *   num_splits [batch + 1] int32: exclusive prefix sum of chunks per sequence.
 * Work is counted in 64-token pages, each sequence costing max(ceil(L/64), 1)
 * pages plus a fixed per-chunk overhead; parts get equal shares.  The result
 * depends only on (cache_seqlens, rows_per_kv, num_parts) and is reused by
 * every layer of the step.  h_kv only enters through num_parts.
 * Errors: MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP (launch).
 */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int rows_per_kv, int h_kv,
                     int num_parts, int32_t* tile_metadata, int32_t* num_splits, void* stream);

/*
 * mla_decode_paged -- the decode (flash_mla_with_kvcache of the Day-1 page §V.2).
 * Enqueues the split-KV decode kernel and, when any sequence is split into
 * more than one chunk, the log-sum-exp combine kernel.
 *   q             bf16 bits [batch, s_q, h_q, d_qk]
 *   kcache        bf16 bits [num_pages, page_block_size, h_kv, d_qk]
 *   num_pages     pages in kcache (used to keep reads inside the cache)
 *   block_table   int32 [batch, max_blocks]; entries past ceil(L/64) are ignored
 *   cache_seqlens int32 [batch], each >= 0
 *   d_qk, dv, page_block_size   must be 576, 512, 64
 *   tile_metadata, num_splits   from mla_get_metadata with the same
 *                 cache_seqlens, rows_per_kv = s_q*h_q/h_kv and num_parts
 *   causal        0/1 (bottom-right aligned when s_q > 1)
 *   softmax_scale scale applied to q.k (e.g. 1/sqrt(192)); finite and > 0
 *   out           bf16 bits [batch, s_q, h_q, dv]
 *   lse           fp32 [batch, s_q, h_q], natural log
 *   workspace     device scratch of at least mla_plan's workspace_bytes, holding
 *                 fp32 partial outputs and their lse for split sequences
 * Errors: MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP.
 */
int mla_decode_paged(const void* q, const void* kcache, int64_t num_pages,
                     const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                     int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                     const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                     int causal, float softmax_scale, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_paged_noalloc -- mla_decode_paged for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments without the workspace; same kernels
 * and results.  The split partials go into a fixed array of the library in
 * device memory, MLA_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library
 * runs on holds until the process ends.  The call allocates nothing (no
 * hipMalloc, no library allocation); the caller still owns every input and
 * output.  A call needing more than the array,
 *   (batch + num_parts) * h_kv * rows_per_kv * (dv + 1) * 4 bytes,
 * returns MLA_ERR_WORKSPACE before any HIP call.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on a GPU (other streams or threads)
 * race and must be serialised by the caller.  The first call on a device looks
 * up the array's address there (hipGetSymbolAddress).
 * Errors: as mla_decode_paged.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (256u << 20)
int mla_decode_paged_noalloc(const void* q, const void* kcache, int64_t num_pages,
                             const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                             int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                             const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                             int causal, float softmax_scale, void* out, float* lse, void* stream);

/*
 * The two stages of mla_decode_paged as separate calls, same arguments and
 * errors.  mla_decode_splitkv enqueues the decode kernel only: sequences kept
 * in one chunk get out/lse, split sequences leave fp32 partials in `workspace`.
 * mla_combine_splits then merges those partials into out/lse (the log-sum-exp
 * combine of the split chunks, the reduction the num_splits output of the
 * Day-1 page §V.2 implies).  Issued in this order on one stream they equal
 * mla_decode_paged; apart they let a caller time or overlap the stages.
 */
int mla_decode_splitkv(const void* q, const void* kcache, int64_t num_pages,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                       int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                       const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                       int causal, float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);
int mla_combine_splits(const void* q, const void* kcache, int64_t num_pages,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                       int batch, int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                       const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                       int causal, float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The absorption GEMMs around the decode (per query head h; d_nope = d_v = 128,
 * latent 512, rope 64).  The weight-absorption identity q.(W_UK c) = (W_UK^T q).c
 * of the "FlashMLA inference acceleration" notes (dpshk.com/news/5996785, §2.1)
 * lets every head score against the one cached latent row c; the value
 * up-projection W_UV commutes with the softmax-weighted sum, so it is applied
 * to the latent output afterwards.  Together with mla_decode_paged they form one
 * MLA decode attention layer: absorb -> decode -> unabsorb.
 *
 * mla_absorb_q:  q_abs[t,h,0:512] = sum_n q_nope[t,h,n] * w_uk[h,n,0:512]
 *                q_abs[t,h,512:576] = q_rope[t,h,0:64]
 *   q_nope  bf16 [tokens, h_q, 128]   (tokens = batch * s_q, any order)
 *   q_rope  bf16 [tokens, h_q, 64]
 *   w_uk    bf16 [h_q, 128, 512]      (the nope key of head h is w_uk[h] . c)
 *   q_abs   bf16 [tokens, h_q, 576]   out: the decode's q; fp32 accumulation,
 *                                     rounded to bf16 (nearest even)
 * mla_unabsorb_out:  out[t,h,v] = sum_c w_uv[h,v,c] * o_lat[t,h,c]
 *   o_lat   bf16 [tokens, h_q, 512]   (the decode's out)
 *   w_uv    bf16 [h_q, 128, 512]      (the value of head h is w_uv[h] . c)
 *   out     bf16 [tokens, h_q, 128]   fp32 accumulation, rounded to bf16
 * All pointers 16-byte aligned device pointers; tokens >= 0 (0 launches
 * nothing and reads no pointer), h_q >= 1.  Errors: MLA_ERR_INVALID, MLA_ERR_HIP.
 */
int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int h_q, void* q_abs,
                 void* stream);
int mla_unabsorb_out(const void* o_lat, const void* w_uv, int tokens, int h_q, void* out, void* stream);

/*
 * Paged KV cache: appending the newest tokens' rows and allocating pages.  The
 * "Flash MLA: efficient MLA decoding kernel library for variable-length
 * sequences" page (developer.baidu.com, §三.1; §四 steps 2 and 5) keeps the
 * cache in fixed-size pages reached through two levels of page tables -- one
 * per sequence, one over the physical pages -- gives a sequence of n tokens
 * ceil(n / page_size) pages, takes pages as it grows and returns them when it
 * ends.  The page size is 64 tokens (the pages' 4096 in that listing is read
 * as the 64 of the kernel's page table).
 *
 * mla_kv_append: for b < batch, j < s_new, k < h_kv, with L = cache_seqlens[b]
 * (the length BEFORE the append; negative counts as 0) and t = L + j:
 *   kcache[block_table[b][t / 64], t % 64, k, :] = new_kv[b, j, k, :]
 * and, when new_seqlens is not NULL, new_seqlens[b] = L + s_new.
 *   new_kv       bf16 [batch, s_new, h_kv, 576] device, 16-byte aligned
 *   cache_seqlens int32 [batch] device
 *   block_table  int32 [batch, max_blocks] device; the entries that cover the
 *                new positions must already hold pages (mla_pager_reserve);
 *                a row whose page id is negative, >= num_pages or past
 *                max_blocks is not written (no fault, nothing reported)
 *   kcache       bf16 [num_pages, 64, h_kv, 576] device, 16-byte aligned, in/out
 *   new_seqlens  int32 [batch] device or NULL; must not alias cache_seqlens
 * batch == 0 launches nothing and reads no pointer.  Rows of different (b, j)
 * must map to different slots (distinct sequences own distinct pages), else
 * which write wins is unspecified.
 * Errors: MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED (more than 2^31 / 72 rows), MLA_ERR_HIP.
 */
int mla_kv_append(const void* new_kv, int batch, int s_new, int h_kv, const int32_t* cache_seqlens,
                  const int32_t* block_table, int max_blocks, void* kcache, int64_t num_pages,
                  int32_t* new_seqlens, void* stream);

/*
 * FP8 latent cache.  The pages name FP8 as the kernel's low-precision mode
 * (FP8/FP16 mixed precision on the FP8 instruction set, "Flash MLA: efficient
 * MLA decoding kernel library for variable-length sequences", developer.baidu.com,
 * §三.2, §四 step 3) but fix no format; this library's format, per token and KV
 * head, is a 656-byte row (MLA_FP8_ROW_BYTES):
 *   bytes   0..511  latent dims 0..511 as e4m3 (OCP E4M3FN: bias 7, 3 mantissa
 *                   bits, largest finite 448, S.1111.111 = NaN)
 *   bytes 512..527  4 fp32 scales, scale g for latent dims 128g .. 128g+127;
 *                   each a power of two (the kernels use only its exponent)
 *   bytes 528..655  rope dims 512..575 as bf16, unchanged
 * The row stands for latent[d] = e4m3(byte d) * scale[d / 128]; with
 * power-of-two scales every such value is a bf16 number, so dequantising is
 * exact and the decode equals the bf16 decode of that cache.
 *
 * mla_kv_append_fp8: as mla_kv_append, but kcache_fp8 is uint8
 *   [num_pages, 64, h_kv, 656] (16-byte aligned) and each bf16 row of new_kv is
 *   quantised on the way in: scale[g] = the smallest 2^e with
 *   max|latent[128g..128g+127]| <= 448 * 2^e (1 for an all-zero group), then
 *   e4m3 = round-to-nearest-even(latent / 2^e).  Non-finite inputs give
 *   unspecified bytes.  Same errors as mla_kv_append.
 * mla_decode_paged_fp8, mla_decode_splitkv_fp8: as mla_decode_paged and
 *   mla_decode_splitkv with kcache_fp8 in that format (the metadata, workspace
 *   and the combine stage, mla_combine_splits, are the same), for any
 *   s_q * h_q / h_kv; the pages are dequantised in the kernels, never written
 *   back.
 */
int mla_kv_append_fp8(const void* new_kv, int batch, int s_new, int h_kv, const int32_t* cache_seqlens,
                      const int32_t* block_table, int max_blocks, void* kcache_fp8, int64_t num_pages,
                      int32_t* new_seqlens, void* stream);
int mla_decode_paged_fp8(const void* q, const void* kcache_fp8, int64_t num_pages, const int32_t* block_table,
                         int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                         int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                         const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_splitkv_fp8(const void* q, const void* kcache_fp8, int64_t num_pages, const int32_t* block_table,
                           int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                           int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                           const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token-sparse decode.  The "Flash MLA: efficient MLA decoding kernel library
 * for variable-length sequences" page (developer.baidu.com, §三.3) adds a
 * token-level sparse mode: each query keeps only its top-k key tokens, the
 * selection stored in CSR form.  How the tokens are scored and picked is the
 * caller's (the page's description of it is garbled); these calls take the
 * selection.  Query row v = b * s_q + s (batch b, query token s) attends, with
 * every head, to the cached tokens of sequence b listed in
 * indices[indptr[v] .. indptr[v+1]) (logical positions); entries outside
 * [0, cache_seqlens[b]) or on a page id outside [0, num_pages) are ignored,
 * listed duplicates count once per listing, and there is no causal mask (the
 * list decides).  A row with no kept entry gives out = 0, lse = -inf.
 *
 * mla_sparse_prepare: keeps the valid entries of every row, in order, as the
 *   byte offsets of their cache rows (KV head 0): offsets[indptr[v] + i] for
 *   i < counts[v].
 *   indices  int32 [indptr[batch*s_q]] device; never NULL, also when every list
 *            is empty (then no entry is read: any valid device address does)
 *   indptr   int32 [batch*s_q + 1] device, non-decreasing, indptr[0] = 0
 *   block_table, cache_seqlens, num_pages, max_blocks, h_kv: as for the decode
 *   offsets  uint32 [indptr[batch*s_q] + 64] device, out (the 64 spare entries
 *            keep the decode's page-wide reads inside the array)
 *   counts   int32 [batch*s_q] device, out
 * mla_sparse_decode: the decode over those rows.  The schedule comes from
 *   mla_plan(batch*s_q, h_q/h_kv, h_kv, ...) and
 *   mla_get_metadata(counts, batch*s_q, h_q/h_kv, h_kv, ...): every query row is
 *   a sequence of counts[v] keys.  q, out, lse as for mla_decode_paged.  Uses
 *   the 64-row kernel for any h_q/h_kv.
 * The cache must hold at most 0xE0000000 bytes (32-bit row offsets), else
 * MLA_ERR_UNSUPPORTED; batch*s_q <= MLA_MAX_BATCH for the decode.  Other
 * errors as for mla_decode_paged.
 */
int mla_sparse_prepare(const int32_t* indices, const int32_t* indptr, int batch, int s_q,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int64_t num_pages,
                       int h_kv, uint32_t* offsets, int32_t* counts, void* stream);
int mla_sparse_decode(const void* q, const void* kcache, int64_t num_pages, const uint32_t* offsets,
                      const int32_t* indptr, const int32_t* counts, int batch, int s_q, int h_q, int h_kv,
                      int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                      const int32_t* num_splits, float softmax_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Host page allocator (no GPU call).  Its whole state -- the free-page stack,
 * the owner of every physical page and the per-sequence page tables, which are
 * the rows of a host block table [max_seqs, max_blocks] int32 (-1 = no page) --
 * lives in one caller-owned host buffer of mla_pager_bytes() bytes (4-byte
 * aligned).  Not thread-safe: calls on one state must be serialised.
 *   mla_pager_bytes      state size, 0 if a size is not positive
 *   mla_pager_init       empty pool of num_pages pages, every table row -1
 *   mla_pager_reserve    grow sequence seq to hold new_len tokens: it gets
 *                        ceil(new_len / 64) pages, the new ones appended to its
 *                        row; a shorter new_len changes nothing.  On
 *                        MLA_ERR_CAPACITY (pool empty, or more than max_blocks
 *                        pages) the state is unchanged.
 *   mla_pager_release    return all pages of seq to the pool; its row becomes -1
 *   mla_pager_free_pages number of free pages (or a negative status)
 *   mla_pager_seq_pages  pages held by seq (or a negative status)
 *   mla_pager_page_owner sequence holding a page (>= 0), -1 if the page is free,
 *                        MLA_ERR_RANGE (a distinct value) for a page id outside
 *                        [0, num_pages) or a state never initialised
 *   mla_pager_block_table pointer to the host block table inside the state
 *                        (NULL if not initialised); copy it to the device for
 *                        mla_kv_append / mla_decode_paged
 * Policy: free pages form a stack (fresh pool: ascending ids; released pages
 * are taken again first).  Errors: MLA_ERR_INVALID, MLA_ERR_WORKSPACE (buffer
 * too small), MLA_ERR_CAPACITY, MLA_ERR_RANGE.
 */
size_t mla_pager_bytes(int num_pages, int max_seqs, int max_blocks);
int mla_pager_init(void* state, size_t bytes, int num_pages, int max_seqs, int max_blocks);
int mla_pager_reserve(void* state, int seq, int64_t new_len);
int mla_pager_release(void* state, int seq);
int mla_pager_free_pages(const void* state);
int mla_pager_seq_pages(const void* state, int seq);
int mla_pager_page_owner(const void* state, int page);
const int32_t* mla_pager_block_table(const void* state);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
