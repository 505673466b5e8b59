// Token-sparse decode, the preparation step.  The "Flash MLA: efficient MLA
// decoding kernel library for variable-length sequences" page (developer.baidu.com,
// §三.3) describes a token-level sparse mode that keeps only the top-k key
// tokens of each query and stores the sparse selection in CSR form.  Here the
// selection is given: query row v = b * s_q + s attends to the cached tokens
// listed in indices[indptr[v] .. indptr[v+1]) (logical positions in sequence
// b).  This step keeps the entries that address a cached token (0 <= pos <
// cache_seqlens[b] and a page id in range), in their order, and turns each into
// the byte offset of its cache row (KV head 0), so that the decode moves rows
// without looking up pages; counts[v] is the number kept.
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void sparse_prepare_kernel(const int32_t* __restrict__ indices,
                                                                  const int32_t* __restrict__ indptr, int s_q,
                                                                  const int32_t* __restrict__ block_table,
                                                                  int max_blocks,
                                                                  const int32_t* __restrict__ seqlens,
                                                                  long long num_pages, int h_kv,
                                                                  uint32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ counts) {
  __shared__ int wave_kept[kThreads / 64];
  const int v = blockIdx.x;
  const int b = v / s_q;
  const int beg = indptr[v], end = indptr[v + 1];
  const int L = seqlens[b] > 0 ? seqlens[b] : 0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int kept = 0;  // entries kept before the current chunk
  for (int base = beg; base < end; base += kThreads) {
    const int i = base + threadIdx.x;
    bool keep = false;
    uint32_t off = 0;
    if (i < end) {
      const int pos = indices[i];
      if (pos >= 0 && pos < L && pos / kPage < max_blocks) {
        const int pid = block_table[(long long)b * max_blocks + pos / kPage];
        if (pid >= 0 && pid < num_pages) {
          keep = true;
          off = (uint32_t)((((long long)pid * kPage + pos % kPage) * h_kv) * kRowBytes);
        }
      }
    }
    const unsigned long long ballot = __ballot(keep);
    const int rank = __popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) wave_kept[wv] = __popcll(ballot);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) {
      before += k < wv ? wave_kept[k] : 0;
      total += wave_kept[k];
    }
    if (keep) offsets[beg + kept + before + rank] = off;
    kept += total;
    __syncthreads();  // wave_kept is rewritten by the next chunk
  }
  if (threadIdx.x == 0) counts[v] = kept;
}

}  // namespace

hipError_t launch_sparse_prepare(const int32_t* indices, const int32_t* indptr, int rows, int s_q,
                                 const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                                 long long num_pages, int h_kv, uint32_t* offsets, int32_t* counts,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(sparse_prepare_kernel, dim3(rows), dim3(kThreads), 0, stream, indices, indptr, s_q,
                     block_table, max_blocks, seqlens, num_pages, h_kv, offsets, counts);
  return hipGetLastError();
}

}  // namespace mla
