// The two weight-absorption GEMMs around the latent decode, per query head h:
//
//   before:  q~[t,h,0:512]   = sum_n q_nope[t,h,n] W_UK[h,n,:]     (q~ = W_UK^T q_nope)
//            q~[t,h,512:576] = q_rope[t,h,:]
//   after:   out[t,h,v]      = sum_c W_UV[h,v,c] o_lat[t,h,c]       (out = W_UV o_lat)
//
// The identity q.(W_UK c) = (W_UK^T q).c lets every head score against the one
// cached latent row c instead of a per-head key, and the value up-projection
// commutes with the softmax-weighted sum ("FlashMLA inference acceleration"
// notes, dpshk.com/news/5996785, §2.1).  With d_nope = d_v = 128 and a 512-wide
// latent, W_UK[h] and W_UV[h] are [128, 512] each (latent index fastest).
//
// Decode has few query tokens per step, so both GEMMs are bound by streaming
// their weights and activations.  On gfx950 both compute C^T[32 columns x 32
// tokens] tiles on v_mfma_f32_32x32x16_bf16 with the weights as the A operand
// (8 consecutive reduction indices per lane) and the activations as B; each
// C^T tile goes through LDS so that every lane stores 16 contiguous bytes of one
// token's output row.  W_UK's columns are the latent index, contiguous in
// memory, so its slice is transposed once through LDS; W_UV already has the
// reduction (latent) index contiguous and goes straight to registers.
#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 32;                 // tokens per MFMA tile, columns per MFMA tile
constexpr int kChunk = 4 * kTile;         // absorb: tokens per workgroup (one tile per wave)
constexpr int kWtStride = kNope + 8;      // LDS row (one output column) of the transposed W_UK slice, padded
constexpr int kObStride = kLatent + 8;    // LDS row (one token) of the staged o_lat tile, padded
constexpr int kOutStride = kTile + 8;     // LDS row (one token) of a staged output tile, padded

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// C^T tile -> LDS -> global.  The MFMA leaves lane l with token t0 + (l & 31)
// and columns 8 (r / 4) + 4 (l / 32) + r % 4 (r = 0..15); after the LDS pass
// lane l stores columns 8 (l & 3) .. +7 of tokens t0 + l / 4 and t0 + 16 + l / 4.
__device__ __forceinline__ void store_tile(uint16_t* stage, uint16_t* out, long long token_stride, int tokens,
                                           int t0, const f32x16_t& acc, int lane) {
  uint16_t* srow = stage + (lane & 31) * kOutStride + 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2_t pk = {pack_bf16(acc[4 * g], acc[4 * g + 1]), pack_bf16(acc[4 * g + 2], acc[4 * g + 3])};
    *(u32x2_t*)(srow + 8 * g) = pk;
  }
  __builtin_amdgcn_wave_barrier();  // the stage is this wave's own: order its LDS writes before the reads
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int tr = half * 16 + (lane >> 2);
    const int t = t0 + tr;
    const uint4 v = *(const uint4*)(stage + tr * kOutStride + 8 * (lane & 3));
    if (t < tokens) *(uint4*)(out + (long long)t * token_stride + 8 * (lane & 3)) = v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): reads done before the stage is rewritten
  __builtin_amdgcn_wave_barrier();
}

// Grid (h_q, kLatent / kCols, ceil(tokens / kChunk)); 4 waves.  The workgroup
// owns kCols output columns of one head and kChunk tokens: the transposed
// 128 x kCols W_UK slice sits in LDS and every wave applies all of it to its
// own 32-token tile, so each q_nope row is read once per column group and each
// weight slice once per token chunk.  kCols = 128 (4 column tiles per wave)
// when there are workgroups enough to fill the GPU, else 32: four times the
// workgroups, each with a quarter of the weight slice to bring in.
template <int kCols>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ q_rope,
                                                            const uint16_t* __restrict__ w_uk, int tokens, int h_q,
                                                            uint16_t* __restrict__ q_abs) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kCols * kWtStride];  // [column][nope index]
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][kTile * kOutStride];
  const int h = blockIdx.x;
  const int col0 = blockIdx.y * kCols;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;

  // W_UK[h][n][col0 .. col0+127] -> wt[col][n]: a thread reads 8 columns of one
  // nope row (16 bytes) and scatters them; consecutive threads take consecutive n
  const uint16_t* wsrc = w_uk + (long long)h * kNope * kLatent + col0;
  for (int i = threadIdx.x; i < kNope * (kCols / 8); i += kThreads) {
    const int n = i % kNope, c8 = (i / kNope) * 8;
    const uint4 v = *(const uint4*)(wsrc + (long long)n * kLatent + c8);
    const uint16_t e[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                           (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
    for (int j = 0; j < 8; ++j) wt[(c8 + j) * kWtStride + n] = e[j];
  }
  __syncthreads();

  const int t0 = blockIdx.z * kChunk + w * kTile;
  if (t0 < tokens) {
    const int t = t0 + (lane & 31);
    const bf16x8_t* bsrc = (const bf16x8_t*)(q_nope + (long long)(t < tokens ? t : 0) * h_q * kNope +
                                             (long long)h * kNope + 8 * (lane >> 5));
    bf16x8_t bq[kNope / 16];
#pragma unroll
    for (int ks = 0; ks < kNope / 16; ++ks) bq[ks] = bsrc[2 * ks];
#pragma unroll
    for (int ct = 0; ct < kCols / kTile; ++ct) {
      // A operand: column col0 + 32 ct + (lane & 31), nope indices 16 ks + 8 (lane >> 5) .. +7
      const uint16_t* arow = wt + (ct * kTile + (lane & 31)) * kWtStride + 8 * (lane >> 5);
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < kNope / 16; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(arow + 16 * ks), bq[ks], acc, 0, 0, 0);
      store_tile(stage[w], q_abs + (long long)h * kDqk + col0 + ct * kTile, (long long)h_q * kDqk, tokens, t0,
                 acc, lane);
    }
    // the rope part passes through (first column group)
    if (blockIdx.y == 0) {
      const int tend = min(tokens, t0 + kTile);
      for (int i = lane; i < (tend - t0) * (kRope / 8); i += 64) {
        const int tt = t0 + i / (kRope / 8), r8 = (i % (kRope / 8)) * 8;
        *(uint4*)(q_abs + ((long long)tt * h_q + h) * kDqk + kLatent + r8) =
            *(const uint4*)(q_rope + ((long long)tt * h_q + h) * kRope + r8);
      }
    }
  }
}

// Grid (h_q, kDvOut / kTile, ceil(tokens / kTile)); 4 waves; for few tokens,
// when the kernel below would leave most of the GPU idle.  The workgroup owns
// one 32-column x 32-token output tile of one head; wave w sums latent indices
// 128 w .. 128 w + 127 (its W_UV block and o_lat block go straight to
// registers), and the four partial tiles are added through LDS.
__global__ __launch_bounds__(kThreads) void unabsorb_out_split_kernel(const uint16_t* __restrict__ o_lat,
                                                                      const uint16_t* __restrict__ w_uv,
                                                                      int tokens, int h_q,
                                                                      uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float part[3][16][64];  // waves 1..3: [wave - 1][element][lane]
  __shared__ __attribute__((aligned(16))) uint16_t stage[kTile * kOutStride];
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * kTile;
  const int t0 = blockIdx.z * kTile;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = t0 + (lane & 31);
  const int kb = kLatent / 4 * w + 8 * (lane >> 5);
  // A operand: row c0 + (lane & 31) of W_UV[h]; B operand: token t (token 0's
  // row past the last token, never stored); latent indices kb + 16 ks .. +7
  const bf16x8_t* asrc = (const bf16x8_t*)(w_uv + ((long long)h * kDvOut + c0 + (lane & 31)) * kLatent + kb);
  const bf16x8_t* bsrc = (const bf16x8_t*)(o_lat + ((long long)(t < tokens ? t : 0) * h_q + h) * kLatent + kb);
  constexpr int kSteps = kLatent / 4 / 16;
  bf16x8_t a[kSteps], b[kSteps];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    a[ks] = asrc[2 * ks];
    b[ks] = bsrc[2 * ks];
  }
  f32x16_t acc = {};
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
  if (w > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[w - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += part[0][r][lane] + part[1][r][lane] + part[2][r][lane];
    store_tile(stage, out + (long long)h * kDvOut + c0, (long long)h_q * kDvOut, tokens, t0, acc, lane);
  }
}

// Grid (h_q, ceil(tokens / kTile)); 4 waves.  The workgroup owns all 128
// output columns of one head (wave w: columns 32 w .. +31, its W_UV rows held
// in registers) for one 32-token tile, whose o_lat rows are staged once in LDS.
__global__ __launch_bounds__(kThreads) void unabsorb_out_kernel(const uint16_t* __restrict__ o_lat,
                                                                const uint16_t* __restrict__ w_uv, int tokens,
                                                                int h_q, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t ob[kTile * kObStride];  // [token][latent]
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][kTile * kOutStride];
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * kTile;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // o_lat rows of the tile -> LDS (rows past the last token are not read)
  for (int i = threadIdx.x; i < kTile * (kLatent / 8); i += kThreads) {
    const int r = i / (kLatent / 8), c8 = (i % (kLatent / 8)) * 8;
    const int t = t0 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < tokens) v = *(const uint4*)(o_lat + ((long long)t * h_q + h) * kLatent + c8);
    *(uint4*)(ob + r * kObStride + c8) = v;
  }
  // A operand: row v = 32 w + (lane & 31) of W_UV[h], latent indices 16 ks + 8 (lane >> 5) .. +7
  const bf16x8_t* asrc =
      (const bf16x8_t*)(w_uv + ((long long)h * kDvOut + w * kTile + (lane & 31)) * kLatent + 8 * (lane >> 5));
  bf16x8_t a[kLatent / 16];
#pragma unroll
  for (int ks = 0; ks < kLatent / 16; ++ks) a[ks] = asrc[2 * ks];
  __syncthreads();
  // B operand: token (lane & 31), latent indices 16 ks + 8 (lane >> 5) .. +7
  const uint16_t* brow = ob + (lane & 31) * kObStride + 8 * (lane >> 5);
  f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
  for (int ks = 0; ks < kLatent / 16; ks += 2) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], *(const bf16x8_t*)(brow + 16 * ks), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks + 1], *(const bf16x8_t*)(brow + 16 * ks + 16), acc1, 0, 0, 0);
  }
  store_tile(stage[w], out + (long long)h * kDvOut + w * kTile, (long long)h_q * kDvOut, tokens, t0, acc0 + acc1,
             lane);
}

}  // namespace

// The narrow forms are chosen when the wide ones would launch fewer
// workgroups than twice (absorb) or once (unabsorb) the GPU's 256 CUs.
static bool absorb_narrow(int tokens, int h_q) {
  return h_q * (kLatent / 128) * ((tokens + kChunk - 1) / kChunk) < 512;
}
static bool unabsorb_split(int tokens, int h_q) { return h_q * ((tokens + kTile - 1) / kTile) < 256; }

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, int tokens,
                           int h_q, uint16_t* q_abs, hipStream_t stream) {
  const int chunks = (tokens + kChunk - 1) / kChunk;
  if (absorb_narrow(tokens, h_q))
    hipLaunchKernelGGL(absorb_q_kernel<32>, dim3(h_q, kLatent / 32, chunks), dim3(kThreads), 0, stream, q_nope,
                       q_rope, w_uk, tokens, h_q, q_abs);
  else
    hipLaunchKernelGGL(absorb_q_kernel<128>, dim3(h_q, kLatent / 128, chunks), dim3(kThreads), 0, stream, q_nope,
                       q_rope, w_uk, tokens, h_q, q_abs);
  return hipGetLastError();
}

hipError_t launch_unabsorb_out(const uint16_t* o_lat, const uint16_t* w_uv, int tokens, int h_q, uint16_t* out,
                               hipStream_t stream) {
  const int tiles = (tokens + kTile - 1) / kTile;
  if (unabsorb_split(tokens, h_q))
    hipLaunchKernelGGL(unabsorb_out_split_kernel, dim3(h_q, kDvOut / kTile, tiles), dim3(kThreads), 0, stream,
                       o_lat, w_uv, tokens, h_q, out);
  else
    hipLaunchKernelGGL(unabsorb_out_kernel, dim3(h_q, tiles), dim3(kThreads), 0, stream, o_lat, w_uv, tokens, h_q,
                       out);
  return hipGetLastError();
}

}  // namespace mla
