// Host side of the C ABI declared in include/mla.h: argument validation (all of
// it before any HIP call), planning, and kernel launches on the caller's stream.
#include "mla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "mla_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

}  // namespace

int mla::set_status(int code, const char* msg) {
  std::snprintf(g_err, sizeof g_err, "%s", code == MLA_OK ? "" : msg);
  return code;
}

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_rows(int batch, int rows_per_kv, int h_kv) {
  if (batch <= 0) return fail(MLA_ERR_INVALID, "batch must be positive (got %d)", batch);
  if (batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds MLA_MAX_BATCH (%d)", batch, MLA_MAX_BATCH);
  if (rows_per_kv <= 0) return fail(MLA_ERR_INVALID, "rows_per_kv must be positive (got %d)", rows_per_kv);
  if (h_kv <= 0) return fail(MLA_ERR_INVALID, "h_kv must be positive (got %d)", h_kv);
  return MLA_OK;
}

int m_tiles_for(int rows) {
  const int tile = mla::tile_rows_for(rows);
  return (rows + tile - 1) / tile;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_err; }

int mla_tile_rows(int rows_per_kv) {
  if (rows_per_kv <= 0) return fail(MLA_ERR_INVALID, "rows_per_kv must be positive");
  return mla::tile_rows_for(rows_per_kv);
}

int mla_plan(int batch, int rows_per_kv, int h_kv, int dv, int num_cus, int* num_parts,
             size_t* workspace_bytes) {
  if (!num_parts || !workspace_bytes) return fail(MLA_ERR_INVALID, "null output pointer");
  if (int rc = check_rows(batch, rows_per_kv, h_kv)) return rc;
  if (dv != MLA_DV) return fail(MLA_ERR_UNSUPPORTED, "dv must be %d (got %d)", MLA_DV, dv);
  if (num_cus < 0) return fail(MLA_ERR_INVALID, "num_cus must be >= 0");
  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  }
  // One 256-thread workgroup per CU (each holds ~145-155 KB of LDS); a part
  // occupies m_tiles * h_kv workgroups.
  const int per_part = m_tiles_for(rows_per_kv) * h_kv;
  int P = num_cus / per_part;
  if (P < 1) P = 1;
  // keep the part count a multiple of 8 when a part spans several workgroups so
  // the XCD-aware mapping (8 XCDs, round-robin dispatch) applies
  if (per_part > 1 && P >= 8) P -= P % 8;
  *num_parts = P;
  *workspace_bytes = (size_t)(batch + P) * (size_t)h_kv * (size_t)rows_per_kv * (size_t)(dv + 1) * 4u;
  return ok();
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int rows_per_kv, int h_kv,
                     int num_parts, int32_t* tile_metadata, int32_t* num_splits, void* stream) {
  if (!cache_seqlens || !tile_metadata || !num_splits) return fail(MLA_ERR_INVALID, "null pointer argument");
  if (int rc = check_rows(batch, rows_per_kv, h_kv)) return rc;
  if (num_parts <= 0) return fail(MLA_ERR_INVALID, "num_parts must be positive (got %d)", num_parts);
  hipError_t e = mla::launch_metadata(cache_seqlens, batch, rows_per_kv, num_parts, tile_metadata,
                                      num_splits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "metadata launch");
  return ok();
}

}  // extern "C"

namespace {

constexpr int kDecode = mla::kStageDecode;
constexpr int kCombine = mla::kStageCombine;

struct SparseArgs {
  const uint32_t* offsets;
  const int32_t* indptr;
};

int decode_common(int stages, int kv_fp8, const SparseArgs* sp, const void* q, const void* kcache, int64_t num_pages,
                  const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int batch,
                  int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                  const int32_t* tile_metadata, int num_parts, const int32_t* num_splits, int causal,
                  float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!q || !kcache || (!block_table && !sp) || !cache_seqlens || !tile_metadata || !num_splits || !out || !lse)
    return fail(MLA_ERR_INVALID, "null pointer argument");
  if (sp && (!sp->offsets || !sp->indptr)) return fail(MLA_ERR_INVALID, "null pointer argument");
  if (d_qk != MLA_D_QK) return fail(MLA_ERR_UNSUPPORTED, "d_qk must be %d (got %d)", MLA_D_QK, d_qk);
  if (dv != MLA_DV) return fail(MLA_ERR_UNSUPPORTED, "dv must be %d (got %d)", MLA_DV, dv);
  if (page_block_size != MLA_PAGE_BLOCK_SIZE)
    return fail(MLA_ERR_UNSUPPORTED, "page_block_size must be %d (got %d)", MLA_PAGE_BLOCK_SIZE,
                page_block_size);
  if (s_q <= 0 || h_q <= 0 || h_kv <= 0 || (max_blocks <= 0 && !sp) || num_pages <= 0)
    return fail(MLA_ERR_INVALID, "sizes must be positive (s_q=%d h_q=%d h_kv=%d max_blocks=%d num_pages=%lld)",
                s_q, h_q, h_kv, max_blocks, (long long)num_pages);
  if (h_q % h_kv != 0) return fail(MLA_ERR_INVALID, "h_q (%d) must be a multiple of h_kv (%d)", h_q, h_kv);
  const long long rows_ll = (long long)s_q * (h_q / h_kv);
  if (rows_ll > (1 << 20)) return fail(MLA_ERR_UNSUPPORTED, "s_q * h_q / h_kv too large");
  const int rows = (int)rows_ll;
  if (int rc = check_rows(batch, rows, h_kv)) return rc;
  if (num_parts <= 0) return fail(MLA_ERR_INVALID, "num_parts must be positive (got %d)", num_parts);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID, "softmax_scale must be finite and positive");
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID, "causal must be 0 or 1");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kcache) | reinterpret_cast<uintptr_t>(out)) & 15u)
    return fail(MLA_ERR_INVALID, "q, kcache and out must be 16-byte aligned");
  if ((long long)page_block_size * h_kv * (kv_fp8 ? MLA_FP8_ROW_BYTES : MLA_D_QK * 2) > 0xffffffffLL)
    return fail(MLA_ERR_UNSUPPORTED, "page too large for 32-bit offsets");
  const size_t need = (size_t)(batch + num_parts) * (size_t)h_kv * (size_t)rows * (size_t)(dv + 1) * 4u;
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(MLA_ERR_WORKSPACE, "workspace must be 16-byte aligned");

  mla::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kcache = static_cast<const uint16_t*>(kcache);
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.tile_md = tile_metadata;
  p.num_splits = num_splits;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  const size_t slots_rows = (size_t)(batch + num_parts) * (size_t)h_kv * (size_t)rows;
  p.o_acc = static_cast<float*>(workspace);
  p.lse_acc = p.o_acc + slots_rows * (size_t)dv;
  p.num_pages = num_pages;
  p.batch = batch;
  p.s_q = s_q;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.rows = rows;
  p.group = h_q / h_kv;
  p.max_blocks = max_blocks;
  p.num_parts = num_parts;
  p.m_tiles = m_tiles_for(rows);
  p.causal = causal;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.xcd_map = (p.m_tiles * h_kv > 1 && num_parts % 8 == 0) ? 1 : 0;
  p.kv_fp8 = kv_fp8;
  if (sp) {
    const long long cache_bytes = num_pages * (long long)MLA_PAGE_BLOCK_SIZE * h_kv * MLA_D_QK * 2;
    if (cache_bytes > (long long)mla::kSparseMaxCacheBytes)
      return fail(MLA_ERR_UNSUPPORTED, "the sparse decode addresses caches up to %u bytes", mla::kSparseMaxCacheBytes);
    p.sparse = 1;
    p.sp_offs = sp->offsets;
    p.sp_rowptr = sp->indptr;
    p.sp_cache_bytes = (uint32_t)cache_bytes;
  }

  hipStream_t st = (hipStream_t)stream;
  if (stages & kDecode) {
    hipError_t e = mla::launch_decode(p, st);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  if (stages & kCombine) {
    hipError_t e = mla::launch_combine(p, st);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return ok();
}

}  // namespace

int mla::decode_paged_stages(int stages, const void* q, const void* kcache, int64_t num_pages,
                             const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int batch,
                             int s_q, int h_q, int h_kv, int d_qk, int dv, int page_block_size,
                             const int32_t* tile_metadata, int num_parts, const int32_t* num_splits, int causal,
                             float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode_common(stages & (kDecode | kCombine), 0, nullptr, q, kcache, num_pages, block_table, max_blocks,
                       cache_seqlens, batch, s_q, h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts,
                       num_splits, causal, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

extern "C" {

int mla_decode_paged(const void* q, const void* kcache, int64_t num_pages, const int32_t* block_table,
                     int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                     int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                     const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(kDecode | kCombine, 0, nullptr, q, kcache, num_pages, block_table, max_blocks, cache_seqlens,
                       batch, s_q, h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts,
                       num_splits, causal, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_decode_splitkv(const void* q, const void* kcache, int64_t num_pages, const int32_t* block_table,
                       int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                       const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(kDecode, 0, nullptr, q, kcache, num_pages, block_table, max_blocks, cache_seqlens, batch, s_q,
                       h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits, causal,
                       softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_combine_splits(const void* q, const void* kcache, int64_t num_pages, const int32_t* block_table,
                       int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                       const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(kCombine, 0, nullptr, q, kcache, num_pages, block_table, max_blocks, cache_seqlens, batch, s_q,
                       h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits, causal,
                       softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_decode_paged_fp8(const void* q, const void* kcache_fp8, int64_t num_pages, const int32_t* block_table,
                         int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                         int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                         const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(kDecode | kCombine, 1, nullptr, q, kcache_fp8, num_pages, block_table, max_blocks, cache_seqlens,
                       batch, s_q, h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits,
                       causal, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_decode_splitkv_fp8(const void* q, const void* kcache_fp8, int64_t num_pages, const int32_t* block_table,
                           int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                           int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                           const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(kDecode, 1, nullptr, q, kcache_fp8, num_pages, block_table, max_blocks, cache_seqlens, batch, s_q,
                       h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits, causal,
                       softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

extern "C" {

int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int h_q, void* q_abs,
                 void* stream) {
  if (tokens < 0 || h_q <= 0)
    return fail(MLA_ERR_INVALID, "tokens must be >= 0 and h_q > 0 (got %d, %d)", tokens, h_q);
  if (tokens == 0) return ok();  // nothing to compute; the pointers are not used
  if (!q_nope || !q_rope || !w_uk || !q_abs) return fail(MLA_ERR_INVALID, "null pointer");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(q_abs))
    return fail(MLA_ERR_INVALID, "pointers must be 16-byte aligned");
  hipError_t e = mla::launch_absorb_q(static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                                      static_cast<const uint16_t*>(w_uk), tokens, h_q, static_cast<uint16_t*>(q_abs),
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "absorb launch");
  return ok();
}

int mla_unabsorb_out(const void* o_lat, const void* w_uv, int tokens, int h_q, void* out, void* stream) {
  if (tokens < 0 || h_q <= 0)
    return fail(MLA_ERR_INVALID, "tokens must be >= 0 and h_q > 0 (got %d, %d)", tokens, h_q);
  if (tokens == 0) return ok();  // nothing to compute; the pointers are not used
  if (!o_lat || !w_uv || !out) return fail(MLA_ERR_INVALID, "null pointer");
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out))
    return fail(MLA_ERR_INVALID, "pointers must be 16-byte aligned");
  hipError_t e = mla::launch_unabsorb_out(static_cast<const uint16_t*>(o_lat), static_cast<const uint16_t*>(w_uv),
                                          tokens, h_q, static_cast<uint16_t*>(out), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "unabsorb launch");
  return ok();
}

}  // extern "C"

namespace {
int append_common(int fp8, const void* new_kv, int batch, int s_new, int h_kv, const int32_t* cache_seqlens,
                  const int32_t* block_table, int max_blocks, void* kcache, int64_t num_pages,
                  int32_t* new_seqlens, void* stream) {
  if (batch < 0 || s_new < 0) return fail(MLA_ERR_INVALID, "batch and s_new must be >= 0 (got %d, %d)", batch, s_new);
  if (batch == 0) return ok();  // nothing to write; the pointers are not used
  if (h_kv <= 0 || max_blocks <= 0 || num_pages <= 0)
    return fail(MLA_ERR_INVALID, "h_kv, max_blocks and num_pages must be positive");
  if (!cache_seqlens || !block_table || !kcache || (s_new > 0 && !new_kv))
    return fail(MLA_ERR_INVALID, "null pointer");
  if (new_seqlens && new_seqlens == cache_seqlens)
    return fail(MLA_ERR_INVALID, "new_seqlens must not alias cache_seqlens");
  if ((s_new > 0 && !aligned16(new_kv)) || !aligned16(kcache))
    return fail(MLA_ERR_INVALID, "new_kv and kcache must be 16-byte aligned");
  if ((long long)batch * s_new * h_kv * (MLA_D_QK * 2 / 16) >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "batch * s_new * h_kv too large for one call");
  hipError_t e =
      fp8 ? mla::launch_kv_append_fp8(static_cast<const uint16_t*>(new_kv), batch, s_new, h_kv, cache_seqlens,
                                      block_table, max_blocks, static_cast<uint8_t*>(kcache), num_pages,
                                      new_seqlens, (hipStream_t)stream)
          : mla::launch_kv_append(static_cast<const uint16_t*>(new_kv), batch, s_new, h_kv, cache_seqlens,
                                  block_table, max_blocks, static_cast<uint16_t*>(kcache), num_pages, new_seqlens,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv append launch");
  return ok();
}
}  // namespace

extern "C" {

int mla_kv_append(const void* new_kv, int batch, int s_new, int h_kv, const int32_t* cache_seqlens,
                  const int32_t* block_table, int max_blocks, void* kcache, int64_t num_pages,
                  int32_t* new_seqlens, void* stream) {
  return append_common(0, new_kv, batch, s_new, h_kv, cache_seqlens, block_table, max_blocks, kcache, num_pages,
                       new_seqlens, stream);
}

int mla_kv_append_fp8(const void* new_kv, int batch, int s_new, int h_kv, const int32_t* cache_seqlens,
                      const int32_t* block_table, int max_blocks, void* kcache_fp8, int64_t num_pages,
                      int32_t* new_seqlens, void* stream) {
  return append_common(1, new_kv, batch, s_new, h_kv, cache_seqlens, block_table, max_blocks, kcache_fp8,
                       num_pages, new_seqlens, stream);
}

}  // extern "C"

extern "C" {

int mla_sparse_prepare(const int32_t* indices, const int32_t* indptr, int batch, int s_q,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int64_t num_pages,
                       int h_kv, uint32_t* offsets, int32_t* counts, void* stream) {
  if (batch < 0 || s_q <= 0 || h_kv <= 0 || max_blocks <= 0 || num_pages <= 0)
    return fail(MLA_ERR_INVALID, "batch >= 0 and s_q, h_kv, max_blocks, num_pages > 0 required");
  if (batch == 0) return ok();
  if (!indices || !indptr || !block_table || !cache_seqlens || !offsets || !counts)
    return fail(MLA_ERR_INVALID, "null pointer");
  if ((long long)batch * s_q > (1 << 24)) return fail(MLA_ERR_UNSUPPORTED, "batch * s_q too large");
  if (num_pages * (long long)MLA_PAGE_BLOCK_SIZE * h_kv * MLA_D_QK * 2 > (long long)mla::kSparseMaxCacheBytes)
    return fail(MLA_ERR_UNSUPPORTED, "the sparse decode addresses caches up to %u bytes", mla::kSparseMaxCacheBytes);
  hipError_t e = mla::launch_sparse_prepare(indices, indptr, batch * s_q, s_q, block_table, max_blocks,
                                            cache_seqlens, num_pages, h_kv, offsets, counts, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sparse prepare launch");
  return ok();
}

int mla_sparse_decode(const void* q, const void* kcache, int64_t num_pages, const uint32_t* offsets,
                      const int32_t* indptr, const int32_t* counts, int batch, int s_q, int h_q, int h_kv,
                      int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                      const int32_t* num_splits, float softmax_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (batch <= 0 || s_q <= 0) return fail(MLA_ERR_INVALID, "batch and s_q must be positive");
  if ((long long)batch * s_q > MLA_MAX_BATCH)
    return fail(MLA_ERR_UNSUPPORTED, "batch * s_q query rows exceed MLA_MAX_BATCH (%d)", MLA_MAX_BATCH);
  const SparseArgs sp{offsets, indptr};
  // every query token is a sequence of its own: [batch * s_q, 1, h_q, ...] views of q, out and lse
  return decode_common(kDecode | kCombine, 0, &sp, q, kcache, num_pages, nullptr, 0, counts, batch * s_q, 1, h_q,
                       h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits, 0, softmax_scale, out,
                       lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
