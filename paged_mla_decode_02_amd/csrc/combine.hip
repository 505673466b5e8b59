// Log-sum-exp combine of split-KV partial results.
//
// A sequence cut into several chunks by the scheduler (the num_splits output of
// the metadata call, "OpenSourceWeek Day 1 -- Demystifying DeepSeek's FlashMLA",
// deepseekonline.chat, §V.2) leaves one normalised partial output o_s and one
// log-sum-exp l_s per chunk and row.  With M = max_s l_s and w_s = 2^(l_s - M):
//   out = sum_s w_s o_s / sum_s w_s,   lse = M + log2(sum_s w_s)
// which is the softmax over the union of the chunks' keys (the online-softmax
// rescaling of the "FlashMLA inference acceleration" notes, dpshk.com, §2.2,
// applied once per chunk instead of once per block).  Chunks are summed in a
// fixed order, so the result is deterministic.  A chunk with no visible key has
// l_s = -inf and weight 0; if every chunk is empty the row is out = 0, lse = -inf.
#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRowsPerBlock = 2;
constexpr int kThreadsPerRow = kDv / 4;  // 4 dims per thread
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

__global__ __launch_bounds__(kRowsPerBlock * kThreadsPerRow) void combine_kernel(DecodeParams p) {
  const int b = blockIdx.x;
  const int kvh = blockIdx.z;
  const int base = p.num_splits[b];
  const int nsp = p.num_splits[b + 1] - base;
  if (nsp <= 1) return;  // written directly by the decode kernel
  if (base < 0 || (long long)base + nsp > (long long)p.batch + p.num_parts) return;  // foreign metadata
  const int row = blockIdx.y * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  if (row >= p.rows) return;
  const int d0 = (threadIdx.x % kThreadsPerRow) * 4;

  const long long stride = (long long)p.h_kv * p.rows;  // rows between consecutive slots
  const long long r0 = ((long long)base * p.h_kv + kvh) * p.rows + row;
  float M = -INFINITY;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, p.lse_acc[r0 + s * stride]);

  const int sq = row / p.group;
  const int h = kvh * p.group + row % p.group;
  const long long o = ((long long)b * p.s_q + sq) * p.h_q + h;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsp; ++s) {
      const float l = p.lse_acc[r0 + s * stride];
      const float wgt = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l - M);
      const f32x4_t v = *(const f32x4_t*)(p.o_acc + (r0 + s * stride) * kDv + d0);
      acc += wgt * v;
      wsum += wgt;
    }
    acc *= 1.f / wsum;
  }
  u32x2_t pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  *(u32x2_t*)(p.out + o * kDv + d0) = pk;
  if (d0 == 0) p.lse[o] = (M == -INFINITY) ? -INFINITY : (M + __builtin_amdgcn_logf(wsum)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.batch, (p.rows + kRowsPerBlock - 1) / kRowsPerBlock, p.h_kv);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kRowsPerBlock * kThreadsPerRow), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
