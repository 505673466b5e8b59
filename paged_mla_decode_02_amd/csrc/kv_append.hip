// Paged KV append: the step before the decode that writes the newest tokens'
// cache rows (latent + rope, 576 bf16) into their pages.  The "Flash MLA:
// efficient MLA decoding kernel library for variable-length sequences" page
// (developer.baidu.com, §三.1 and §四 step 2) describes the paged cache: a
// sequence's pages are found through its page table and new pages are taken
// as the sequence grows; the page size here is 64 tokens.
//
// Token j of sequence b (j < s_new) lands at logical position t = L_b + j,
// i.e. page block_table[b][t / 64], slot t % 64.  The work is a scatter of
// 1152-byte rows, bound by HBM: one 16-byte chunk per thread, consecutive
// threads on consecutive chunks of a row, so every store is part of a
// contiguous 1152-byte run.
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kChunks = kRowBytes / 16;  // 72 chunks of 16 bytes per cache row

__global__ __launch_bounds__(kThreads) void kv_append_kernel(const uint4* __restrict__ new_kv, int batch, int s_new,
                                                             int h_kv, const int32_t* __restrict__ seqlens,
                                                             const int32_t* __restrict__ block_table,
                                                             int max_blocks, uint4* __restrict__ kcache,
                                                             long long num_pages, int total,
                                                             int32_t* __restrict__ new_seqlens) {
  const int stride = gridDim.x * kThreads;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int c = i % kChunks;
    const int r = i / kChunks;  // ((b * s_new) + j) * h_kv + k
    // the row chunk does not depend on the page lookup: its load overlaps the
    // two dependent loads (length, then page id)
    const uint4 v = new_kv[(long long)r * kChunks + c];
    const int k = r % h_kv;
    const int bj = r / h_kv;
    const int j = bj % s_new;
    const int b = bj / s_new;
    const int L = seqlens[b] > 0 ? seqlens[b] : 0;
    const long long t = (long long)L + j;
    const long long blk = t / kPage;
    if (blk >= max_blocks) continue;  // past the table: not written
    const int pid = block_table[(long long)b * max_blocks + blk];
    if (pid < 0 || pid >= num_pages) continue;  // unassigned page: not written
    const long long row = ((long long)pid * kPage + t % kPage) * h_kv + k;
    kcache[row * kChunks + c] = v;
  }
  if (new_seqlens) {
    for (int b = blockIdx.x * kThreads + threadIdx.x; b < batch; b += stride)
      new_seqlens[b] = (seqlens[b] > 0 ? seqlens[b] : 0) + s_new;
  }
}

}  // namespace

hipError_t launch_kv_append(const uint16_t* new_kv, int batch, int s_new, int h_kv, const int32_t* seqlens,
                            const int32_t* block_table, int max_blocks, uint16_t* kcache, long long num_pages,
                            int32_t* new_seqlens, hipStream_t stream) {
  const long long total = (long long)batch * s_new * h_kv * kChunks;
  long long blocks = (total + kThreads - 1) / kThreads;
  if (blocks < (batch + kThreads - 1) / kThreads) blocks = (batch + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (const uint4*)new_kv,
                     batch, s_new, h_kv, seqlens, block_table, max_blocks, (uint4*)kcache, num_pages, (int)total,
                     new_seqlens);
  return hipGetLastError();
}

}  // namespace mla
