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

constexpr int kThreadsPerRow = kDv / 4;  // 4 dims per thread, two waves per row
constexpr int kTile = 256;               // chunk weights staged in LDS at a time
constexpr int kUnroll = 8;               // partial loads in flight per thread
constexpr int kFew = 8;                  // up to this many chunks: single-pass path
static_assert(kFew == 8, "combine_few is instantiated for 2..8 chunks");
struct LDS_float_pair {
  float v[2];
};
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// Few chunks: every thread reads the row's NC lse values itself and all NC
// partial quads at once (two dependent loads in all, no barrier).
template <int NC>
__device__ __forceinline__ void combine_few(const DecodeParams& p, long long r0, long long stride, long long o,
                                            int d0, bool write_lse) {
  float l[NC];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NC; ++s) {
    l[s] = p.lse_acc[r0 + s * stride];
    M = fmaxf(M, l[s]);
  }
  f32x4_t v[NC];
#pragma unroll
  for (int s = 0; s < NC; ++s) v[s] = *(const f32x4_t*)(p.o_acc + (r0 + s * stride) * kDv + d0);
  float wsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < NC; ++s) {
      const float wgt = (l[s] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l[s] - M);
      wsum += wgt;
      acc += wgt * v[s];
    }
    acc *= 1.f / wsum;
  }
  u32x2_t pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  *(u32x2_t*)(p.out + o * kDv + d0) = pk;
  if (write_lse) p.lse[o] = (M == -INFINITY) ? -INFINITY : (M + __builtin_amdgcn_logf(wsum)) * kLn2;
}

// Maximum and sum over the kThreadsPerRow threads (two waves) of one row.
__device__ __forceinline__ float row_reduce(float v, bool is_max, LDS_float_pair* red, int rl, int wv) {
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if ((threadIdx.x & 63) == 0) red[rl].v[wv] = v;
  __syncthreads();
  const float r = is_max ? fmaxf(red[rl].v[0], red[rl].v[1]) : red[rl].v[0] + red[rl].v[1];
  __syncthreads();
  return r;
}

// One workgroup merges R rows of one (sequence, KV head): each row's
// 128 threads first reduce max_s l_s and sum_s 2^(l_s - M) over the chunks, then
// normalised chunk weights go through LDS kTile at a time and every thread
// accumulates its 4 dims over the chunks with kUnroll loads in flight.
template <int R>
__global__ __launch_bounds__(R * kThreadsPerRow) void combine_kernel(DecodeParams p) {
  __shared__ float wts[R][kTile];
  __shared__ LDS_float_pair red[R];
  const int b = blockIdx.x;
  const int kvh = blockIdx.z;
  const int base = p.num_splits[b];
  const int nsp = p.num_splits[b + 1] - base;
  if (nsp <= 1) return;  // written directly by the decode kernel
  if (base < 0 || (long long)base + nsp > (long long)p.batch + p.num_parts) return;  // foreign metadata
  const int rl = threadIdx.x / kThreadsPerRow;
  const int t = threadIdx.x % kThreadsPerRow;
  const int wv = t / 64;
  const int row = blockIdx.y * R + rl;
  const bool row_ok = row < p.rows;  // uniform over the row's two waves
  const int d0 = t * 4;

  const long long stride = (long long)p.h_kv * p.rows;  // rows between consecutive slots
  const long long r0 = ((long long)base * p.h_kv + kvh) * p.rows + (row_ok ? row : 0);
  const int sq = row / p.group;
  const int h = kvh * p.group + row % p.group;
  const long long o = ((long long)b * p.s_q + sq) * p.h_q + h;

  if (nsp <= kFew) {
    if (!row_ok) return;
    switch (nsp) {
      case 2: combine_few<2>(p, r0, stride, o, d0, t == 0); break;
      case 3: combine_few<3>(p, r0, stride, o, d0, t == 0); break;
      case 4: combine_few<4>(p, r0, stride, o, d0, t == 0); break;
      case 5: combine_few<5>(p, r0, stride, o, d0, t == 0); break;
      case 6: combine_few<6>(p, r0, stride, o, d0, t == 0); break;
      case 7: combine_few<7>(p, r0, stride, o, d0, t == 0); break;
      default: combine_few<8>(p, r0, stride, o, d0, t == 0); break;
    }
    return;
  }

  // The first kPre partials do not depend on the weights: their loads go out
  // together with the lse loads, so the two round trips overlap.  Only in the
  // one-row form, which serves rows with many chunks: the registers they take
  // would cost the two-row form a wave per SIMD.
  constexpr int kPre = R == 1 ? 4 : 0;
  const long long cstride = stride * kDv;  // floats between consecutive chunks' partials
  f32x4_t v0[kPre > 0 ? kPre : 1];
  if (row_ok) {
    const float* src = p.o_acc + r0 * kDv + d0;
#pragma unroll
    for (int u = 0; u < kPre; ++u) v0[u] = *(const f32x4_t*)(src + u * cstride);  // nsp > kFew > kPre
  }
  // With at most one chunk per thread (nsp <= kThreadsPerRow) each lse is read
  // once and kept for the sum and the weights.
  const bool one = nsp <= kThreadsPerRow;
  float lt = -INFINITY;
  float M = -INFINITY;
  if (row_ok)
    for (int s = t; s < nsp; s += kThreadsPerRow) {
      const float l = p.lse_acc[r0 + s * stride];
      if (s == t) lt = l;
      M = fmaxf(M, l);
    }
  M = row_reduce(M, true, red, rl, wv);
  float wsum = 0.f;
  if (row_ok && M != -INFINITY) {
    if (one) {
      wsum = (lt == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lt - M);
    } else {
      for (int s = t; s < nsp; s += kThreadsPerRow) {
        const float l = p.lse_acc[r0 + s * stride];
        wsum += (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l - M);
      }
    }
  }
  wsum = row_reduce(wsum, false, red, rl, wv);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsp; s0 += kTile) {
    const int n = min(kTile, nsp - s0);
    for (int j = t; j < kTile; j += kThreadsPerRow) {
      float wgt = 0.f;
      if (row_ok && j < n && M != -INFINITY) {
        const float l = one ? lt : p.lse_acc[r0 + (s0 + j) * stride];  // one: s0 = 0 and j = t
        wgt = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l - M) * inv;
      }
      wts[rl][j] = wgt;
    }
    __syncthreads();
    if (row_ok) {
      const float* src = p.o_acc + (r0 + s0 * stride) * kDv + d0;
      int jb = 0;
      if (s0 == 0) {  // the first kPre chunks, already loaded (n > kPre)
#pragma unroll
        for (int u = 0; u < kPre; ++u) acc += wts[rl][u] * v0[u];
        jb = kPre;
      }
      for (int j0 = jb; j0 < n; j0 += kUnroll) {
        f32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int j = min(j0 + u, n - 1);  // past the end: weight 0, any valid slot
          v[u] = *(const f32x4_t*)(src + j * cstride);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += wts[rl][min(j0 + u, kTile - 1)] * (j0 + u < n ? v[u] : f32x4_t{});
      }
    }
    __syncthreads();
  }
  if (!row_ok) return;
  u32x2_t pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  *(u32x2_t*)(p.out + o * kDv + d0) = pk;
  if (t == 0) p.lse[o] = (M == -INFINITY) ? -INFINITY : (M + __builtin_amdgcn_logf(wsum)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  // Rows per workgroup.  When sequences average more than 8 chunks (more parts
  // than 8 per sequence), rows take the many-chunk path, which is bound by the
  // partial loads a CU keeps in flight: one row per workgroup doubles the
  // workgroups, and so the loads in flight.  With few chunks per row, two rows
  // per workgroup halve the workgroups to launch, which costs less.
  if ((long long)p.num_parts > 8LL * p.batch) {
    dim3 grid(p.batch, p.rows, p.h_kv);
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(kThreadsPerRow), 0, stream, p);
  } else {
    dim3 grid(p.batch, (p.rows + 1) / 2, p.h_kv);
    hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(2 * kThreadsPerRow), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
