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

// e4m3 (OCP E4M3FN) code of y, |y| <= 448, rounded to nearest, ties to the even
// code: normal results keep 3 mantissa bits of the fp32 pattern (the carry of
// the rounding moves into the exponent), results below 2^-6 are multiples of
// 2^-9.  The sign is kept, -0 included.
__device__ __forceinline__ unsigned e4m3_rne(float y) {
  const unsigned bits = __float_as_uint(y);
  const unsigned a = bits & 0x7fffffffu;
  unsigned code;
  if (a < 0x3c800000u) {  // |y| < 2^-6: subnormal e4m3 (or zero)
    code = (unsigned)__builtin_rintf(__uint_as_float(a) * 512.f);
  } else {
    const unsigned r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // exponent | 3 mantissa bits, rounded
    code = r - ((127u - 7u) << 3);
    if (code > 0x7eu) code = 0x7eu;  // 448 is the largest finite value
  }
  return code | ((bits >> 24) & 0x80u);
}

// One wave per appended row: lane l quantises latent dims 8l .. 8l+7 (group
// l / 16); the group's max |x| goes over its 16 lanes, the scale is the
// smallest power of two 2^e with max |x| <= 448 * 2^e (1 for an all-zero group).
__global__ __launch_bounds__(kThreads) void kv_append_fp8_kernel(const uint16_t* __restrict__ new_kv, int batch,
                                                                 int s_new, int h_kv,
                                                                 const int32_t* __restrict__ seqlens,
                                                                 const int32_t* __restrict__ block_table,
                                                                 int max_blocks, uint8_t* __restrict__ kcache,
                                                                 long long num_pages, int rows,
                                                                 int32_t* __restrict__ new_seqlens) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r < rows) {
    const uint4 v = *(const uint4*)(new_kv + (long long)r * kDqk + 8 * lane);
    const uint4 rope = lane < kRope / 8 ? *(const uint4*)(new_kv + (long long)r * kDqk + kLatent + 8 * lane)
                                        : make_uint4(0, 0, 0, 0);
    const int k = r % h_kv;
    const int bj = r / h_kv;
    const int j = bj % s_new;
    const int b = bj / s_new;
    const int L = seqlens[b] > 0 ? seqlens[b] : 0;
    const long long t = (long long)L + j;
    const long long blk = t / kPage;
    int pid = -1;
    if (blk < max_blocks) pid = block_table[(long long)b * max_blocks + blk];
    if (pid >= 0 && pid < num_pages) {  // uniform over the wave: one row
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
      float x[8];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      int e = 0;
      if (amax > 0.f) {
        int ea;
        const float m = frexpf(amax, &ea);  // amax = m * 2^ea, m in [0.5, 1); 448 = 0.875 * 2^9
        e = ea - 9 + (m > 0.875f ? 1 : 0);
      }
      unsigned q[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i >> 2] |= e4m3_rne(ldexpf(x[i], -e)) << (8 * (i & 3));
      uint8_t* row = kcache + (((long long)pid * kPage + t % kPage) * h_kv + k) * kF8RowBytes;
      *(uint2*)(row + 8 * lane) = make_uint2(q[0], q[1]);
      if ((lane & 15) == 0) *(float*)(row + kLatent + 4 * (lane >> 4)) = ldexpf(1.f, e);
      if (lane < kRope / 8) *(uint4*)(row + kLatent + 16 + 16 * lane) = rope;
    }
  }
  if (new_seqlens) {
    const int stride = gridDim.x * kThreads;
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < batch; i += stride)
      new_seqlens[i] = (seqlens[i] > 0 ? seqlens[i] : 0) + s_new;
  }
}

}  // namespace

hipError_t launch_kv_append_fp8(const uint16_t* new_kv, int batch, int s_new, int h_kv, const int32_t* seqlens,
                                const int32_t* block_table, int max_blocks, uint8_t* kcache, long long num_pages,
                                int32_t* new_seqlens, hipStream_t stream) {
  const long long rows = (long long)batch * s_new * h_kv;
  long long blocks = (rows + 3) / 4;
  if (blocks < (batch + kThreads - 1) / kThreads) blocks = (batch + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, new_kv, batch, s_new,
                     h_kv, seqlens, block_table, max_blocks, kcache, num_pages, (int)rows, new_seqlens);
  return hipGetLastError();
}

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
