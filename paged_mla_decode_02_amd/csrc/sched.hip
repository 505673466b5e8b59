// Split-KV scheduler: tile metadata and cumulative split counts from the
// sequence lengths, computed on the GPU by one workgroup.
//
// The FlashMLA API computes this once per decode step from cache_seqlens and
// the number of query rows per KV head ("OpenSourceWeek Day 1 -- Demystifying
// DeepSeek's FlashMLA", deepseekonline.chat, §V.2); the variable-length page
// balancing it serves is the theme of the "Flash MLA: efficient MLA decoding
// kernel library for variable-length sequences" page (developer.baidu.com, §二).
// The pages name the call only, so the partition below is this library's own:
//
//   work is measured in 64-token pages; sequence i costs m_i = max(ceil(L_i/64), 1)
//   pages after a fixed overhead of OVH pages (query load, chunk-end merge,
//   split partial), laid end to end: A_i = C_i + OVH, B_i = A_i + m_i,
//   C_{i+1} = B_i, T = C_b.
//   Parts are equal slices of q = max(ceil(T/P), QMIN) units of that line.
//   Sequence i is split into part(B_i - 1) - part(A_i) + 1 chunks.
//
// Every step is integer arithmetic on prefix sums, so the result is exact and
// independent of thread scheduling.
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;

template <typename T>
__device__ T block_inclusive_scan(T v, T* wave_tot) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  if (lane == 63) wave_tot[wid] = v;
  __syncthreads();
  if (wid == 0) {
    T t = lane < kThreads / 64 ? wave_tot[lane] : T(0);
#pragma unroll
    for (int off = 1; off < kThreads / 64; off <<= 1) {
      T n = __shfl_up(t, off, 64);
      if (lane >= off) t += n;
    }
    if (lane < kThreads / 64) wave_tot[lane] = t;
  }
  __syncthreads();
  if (wid > 0) v += wave_tot[wid - 1];
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kThreads) void metadata_kernel(const int32_t* __restrict__ seqlens,
                                                            int batch, int rows, int num_parts,
                                                            int32_t* __restrict__ tile_md,
                                                            int32_t* __restrict__ num_splits) {
  __shared__ long long A[kMaxBatch];
  __shared__ long long B[kMaxBatch];
  __shared__ long long wave_tot[kThreads / 64];
  __shared__ int wave_tot_i[kThreads / 64];

  const int tile = tile_rows_for(rows);
  const long long ovh = sched_overhead(tile);
  const long long qmin = sched_min_part(tile);

  // prefix sums of (OVH + m_i): B_i is the end of sequence i's work on the line
  long long carry = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int i = base + threadIdx.x;
    long long m = 0;
    if (i < batch) {
      const long long L = seqlens[i] > 0 ? seqlens[i] : 0;
      const long long nb = (L + kPage - 1) / kPage;
      m = nb > 1 ? nb : 1;
    }
    const long long inc = block_inclusive_scan<long long>(i < batch ? ovh + m : 0, wave_tot) + carry;
    if (i < batch) {
      B[i] = inc;
      A[i] = inc - m;
    }
    __syncthreads();
    carry = B[min(base + kThreads, batch) - 1];
    __syncthreads();
  }
  const long long T = B[batch - 1];
  long long q = (T + num_parts - 1) / num_parts;
  if (q < qmin) q = qmin;

  // chunks per sequence -> exclusive prefix sum
  int icarry = 0;
  if (threadIdx.x == 0) num_splits[0] = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int i = base + threadIdx.x;
    int chunks = 0;
    if (i < batch) chunks = (int)((B[i] - 1) / q - A[i] / q + 1);
    const int inc = block_inclusive_scan<int>(chunks, wave_tot_i) + icarry;
    if (i < batch) num_splits[i + 1] = inc;
    // the last thread of this slab holds the running total
    __shared__ int slab_total;
    if (i == min(base + kThreads, batch) - 1) slab_total = inc;
    __syncthreads();
    icarry = slab_total;
    __syncthreads();
  }

  // one metadata row per part: binary searches on the monotone A and B
  for (int p = threadIdx.x; p < num_parts; p += kThreads) {
    int32_t* row = tile_md + (long long)p * kMdInts;
    const long long lo = (long long)p * q;
    if (lo >= T) {
      row[0] = batch; row[1] = 0; row[2] = batch; row[3] = 0;
      row[4] = 0; row[5] = 0; row[6] = 0; row[7] = 0;
      continue;
    }
    const long long hi = lo + q < T ? lo + q : T;
    // first i with B_i > lo
    int a = 0, z = batch;
    while (a < z) {
      const int mid = (a + z) >> 1;
      if (B[mid] > lo) z = mid; else a = mid + 1;
    }
    const int i = a;
    // first j with A_j >= hi, minus one
    a = i; z = batch;
    while (a < z) {
      const int mid = (a + z) >> 1;
      if (A[mid] >= hi) z = mid; else a = mid + 1;
    }
    const int j = a - 1;
    const long long first = lo > A[i] ? lo : A[i];
    const long long last = (hi < B[j] ? hi : B[j]) - 1;
    row[0] = i;
    row[1] = (int32_t)(first - A[i]);
    row[2] = j;
    row[3] = (int32_t)(last - A[j] + 1);
    row[4] = (int32_t)(p - A[i] / q);
    row[5] = 0; row[6] = 0; row[7] = 0;
  }
}

}  // namespace

hipError_t launch_metadata(const int32_t* seqlens, int batch, int rows, int num_parts,
                           int32_t* tile_md, int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kThreads), 0, stream, seqlens, batch, rows,
                     num_parts, tile_md, num_splits);
  return hipGetLastError();
}

}  // namespace mla
