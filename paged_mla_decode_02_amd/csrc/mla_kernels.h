// Internal interface between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;          // tokens per cache page
constexpr int kDqk = 576;          // latent 512 + rope 64
constexpr int kDv = 512;           // value width (latent part of each row)
constexpr int kRowBytes = kDqk * 2;
constexpr int kMdInts = 8;
// MLA head geometry around the latent decode (absorption GEMMs)
constexpr int kNope = 128;         // non-rope query/key dims per head
constexpr int kRope = 64;          // rope dims (kDqk = kLatent + kRope)
constexpr int kLatent = 512;       // compressed latent width (= kDv)
constexpr int kDvOut = 128;        // value dims per head after W_UV
constexpr int kMaxBatch = 8192;
// FP8 cache row: 512 e4m3 latent dims, 4 fp32 power-of-two scales (one per 128
// latent dims), 64 bf16 rope dims = 656 bytes.
constexpr int kF8Group = 128;
constexpr int kF8RowBytes = kLatent + 4 * (kLatent / kF8Group) + 2 * kRope;

// Query rows one workgroup owns: <= 16 rows use the 16-row token-split kernel,
// up to 128 rows the 64-row split-wave kernel (ceil(rows / 64) row tiles),
// more the 128-row kernel (ceil(rows / 128) row tiles).  At 128 rows the
// 128-row kernel would need twice the parts to fill the GPU, and the extra
// split partials cost more than its faster tile saves.  The FP8 and
// token-sparse decodes keep 64-row tiles for any row count (tiles64_for).
__host__ __device__ constexpr int tile_rows_for(int rows) { return rows <= 16 ? 16 : rows <= 128 ? 64 : 128; }
__host__ __device__ constexpr int tiles64_for(int rows) { return (rows + 63) / 64; }
// Fixed per-chunk cost, in page units, that the scheduler charges before each
// sequence: loading the query tile, the end-of-chunk merge and writing /
// re-reading a split partial.  The 16-row token-split kernel's chunk end (a merge
// of four waves' states through LDS) costs about three page loads.
__host__ __device__ constexpr int sched_overhead(int tile) { return tile == 16 ? 3 : tile / 16; }
__host__ __device__ constexpr int sched_min_part(int tile) { return 2 * sched_overhead(tile); }

struct DecodeParams {
  const uint16_t* q;         // [b, s_q, h_q, 576]
  const uint16_t* kcache;    // [num_pages, 64, h_kv, 576]
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* tile_md;    // [num_parts, 8]
  const int32_t* num_splits; // [b + 1]
  uint16_t* out;             // [b, s_q, h_q, 512]
  float* lse;                // [b, s_q, h_q]
  float* o_acc;              // [slots, h_kv, rows, 512]
  float* lse_acc;            // [slots, h_kv, rows]
  int64_t num_pages;
  int batch, s_q, h_q, h_kv, rows, group, max_blocks, num_parts, m_tiles, causal;
  float scale_log2;          // softmax_scale * log2(e)
  int xcd_map;               // workgroup -> (part, row tile, kv head) mapping keeps a part on one XCD
  int kv_fp8;                // kcache rows are the 656-byte FP8 format (kF8RowBytes) instead of bf16
  // token-sparse decode: sequence b of the launch is query row b of the caller;
  // its keys are the cache rows at byte offsets sp_offs[sp_rowptr[b] + i],
  // i < seqlens[b] (the kept entries of its index list)
  const uint32_t* sp_offs;
  const int32_t* sp_rowptr;
  uint32_t sp_cache_bytes;
  int sparse;
};
// byte offset that no cache holds: a transfer from it reads zeros
constexpr uint32_t kSparseNone = 0xF0000000u;
constexpr uint32_t kSparseMaxCacheBytes = 0xE0000000u;

// Records the status of the last C-ABI call on this thread (message for
// mla_last_error) and returns `code`.
int set_status(int code, const char* msg);

// The bf16 paged decode behind mla_decode_paged: validates every argument on
// the host, then enqueues the stages in `stages` (kStageDecode | kStageCombine;
// 0 validates only and launches nothing).  Status as the C ABI.
constexpr int kStageDecode = 1;
constexpr int kStageCombine = 2;
int decode_paged_stages(int stages, const void* q, const void* kcache, int64_t num_pages,
                        const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int batch,
                        int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                        const int32_t* tile_metadata, int num_parts, const int32_t* num_splits, int causal,
                        float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

hipError_t launch_metadata(const int32_t* seqlens, int batch, int rows, int num_parts,
                           int32_t* tile_md, int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_wide(const DecodeParams& p, hipStream_t stream);
// 64-row tiles on bf16 pages with score and value waves (decode_qkpv.hip)
hipError_t launch_decode_qkpv(const DecodeParams& p, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);
hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, int tokens,
                           int h_q, uint16_t* q_abs, hipStream_t stream);
hipError_t launch_kv_append(const uint16_t* new_kv, int batch, int s_new, int h_kv, const int32_t* seqlens,
                            const int32_t* block_table, int max_blocks, uint16_t* kcache, long long num_pages,
                            int32_t* new_seqlens, hipStream_t stream);
hipError_t launch_kv_append_fp8(const uint16_t* new_kv, int batch, int s_new, int h_kv, const int32_t* seqlens,
                                const int32_t* block_table, int max_blocks, uint8_t* kcache, long long num_pages,
                                int32_t* new_seqlens, hipStream_t stream);
hipError_t launch_sparse_prepare(const int32_t* indices, const int32_t* indptr, int rows, int s_q,
                                 const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                                 long long num_pages, int h_kv, uint32_t* offsets, int32_t* counts,
                                 hipStream_t stream);
hipError_t launch_unabsorb_out(const uint16_t* o_lat, const uint16_t* w_uv, int tokens, int h_q, uint16_t* out,
                               hipStream_t stream);

}  // namespace mla
