// Paged MLA decode for gfx950 (CDNA4): split-KV attention of absorbed queries
// over one shared latent KV head stored in 64-token pages.
//
// Method.  For each query row, softmax(scale * q.K^T) . V over the cached
// sequence, where K is the whole 576-wide latent+rope row and V its first 512
// dims (the absorbed form of MLA: q.(W_UK c) = (W_UK^T q).c, "FlashMLA inference
// acceleration" notes, dpshk.com/news/5996785, §2.1).  The softmax is computed
// online, block by block, with a running max and sum; earlier blocks are
// rescaled when the max grows, which gives exactly the textbook softmax (same
// notes, §2.2).  All query heads that share the KV head are folded into the
// rows of one problem (Day-1 page "OpenSourceWeek Day 1 -- Demystifying
// DeepSeek's FlashMLA", deepseekonline.chat, §II.1), so every latent page read
// from HBM is multiplied against all of them: a dense contraction per page.
//
// gfx950 design (the pages' Hopper kernel -- cp.async into shared memory and
// warpgroup MMA, Day-1 page §II.3 -- is prior art only):
//   * pages move HBM -> LDS with buffer_load ... lds (16 bytes per lane, no
//     register staging); out-of-range slots of the last page read as zeros
//     through the buffer descriptor's size, so stale cache bits never reach V;
//   * a page lives in LDS as four 16-token slices; a slice is laid out
//     [9 groups of 8 chunks][16 tokens][8 chunks of 16 B] with the chunk index
//     XOR-swizzled inside its 128-byte group, so that the K-operand reads (16
//     tokens x 16 B per quarter wave) and the transposed V-operand reads
//     (ds_read_b64_tr_b16, 4 tokens x 64 B per half wave) are bank-conflict free,
//     and every read or DMA address is one of a few per-lane bases plus an
//     immediate offset;
//   * QK^T and PV run on v_mfma_f32_32x32x16_bf16 (16x16 shapes for <= 16
//     rows), accumulating in fp32; P is rounded to bf16 for PV and the row sum
//     uses the fp32 P;
//   * the running max is only moved when it grows by more than 2^8 (in log2
//     units), so the O rescale is rare; the final normalisation uses the same
//     reference max, which keeps the result exact up to rounding.
//
// Two kernels:
//   decode_tokensplit  (<= 16 query rows per KV head, memory-bound shapes):
//     each of the 4 waves owns 16 tokens of every page and an independent online
//     softmax over them; the 4 states merge at the end of a chunk through LDS.
//   decode_pairsplit  (64-row tiles, compute-bound shapes):
//     QK^T is split 2 x 2 over rows and tokens (32 rows per wave, queries
//     resident in registers), P goes through LDS, and PV is split by output dims
//     (128 per wave), so each V element of a page is read from LDS once per
//     workgroup.
// Both also run on the FP8 cache (656-byte rows, see kF8RowBytes): the 16-row
// kernel dequantises each slice in LDS, the 64-row kernel keeps FP8 pages in
// LDS and dequantises its MFMA operands in registers.
#include <type_traits>
#include <utility>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))


constexpr int kThreads = 256;
constexpr int kSlice = 16;                         // tokens one wave moves per page
constexpr int kSliceBytes = kSlice * kRowBytes;    // 18432 = 18 x 1 KB DMA instructions
constexpr int kSliceDma = kSliceBytes / 1024;
constexpr int kGroupBytes = 16 * 128;              // 8 chunks x 16 tokens
constexpr int kPageBytes = kPage * kRowBytes;      // 73728
constexpr float kTau = 8.0f;                       // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

// XOR applied to a chunk's position inside its 8-chunk group, by token (0..15).
// Over the 8 even (or 8 odd) tokens of a slice it is a permutation of 0..7, and
// tokens 4u and 4u+2 (4u+1 and 4u+3) differ in bit 2.
__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
// byte offset of (token t in 0..15, chunk c in 0..71) inside a 16-token slice
__device__ __forceinline__ int slice_off(int t, int c) {
  return (c >> 3) * kGroupBytes + t * 128 + (((c & 7) ^ swz(t)) << 4);
}

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Explicit waits: the LDS-DMA loads are tracked by hand, never by a compiler fence.
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Wait for every vector-memory operation, visibly to the compiler (vmcnt(0)).
// The compiler counts only the loads it issued itself; a wait it places before
// the first use of such a load would also cover every page transfer issued
// since, so loads whose results are used across page transfers (queries, page
// ids, lengths of the next sequence) are drained here, at points where nothing
// else is in flight that the kernel does not need at once anyway.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float wave_max16(float v) {  // max over lanes l, l^16, l^32, l^48
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}
// reduction across the two wave halves (lane l and l ^ 32)
__device__ __forceinline__ float half_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x4_t lds_tr16(const LDS_AS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)p);
}

// Which part / row tile / KV head this workgroup serves.  With xcd_map the
// workgroups of one part (its row tiles and KV heads, which read the same pages)
// get ids that differ by multiples of 8, i.e. land on the same XCD and share L2.
__device__ __forceinline__ void map_block(const DecodeParams& p, int& part, int& mt, int& kvh) {
  const int x = blockIdx.x;
  const int G = p.m_tiles * p.h_kv;
  int g;
  if (p.xcd_map) {
    const int k = x >> 3;
    g = k % G;
    part = (k / G) * 8 + (x & 7);
  } else {
    part = x / G;
    g = x % G;
  }
  mt = g % p.m_tiles;
  kvh = g / p.m_tiles;
}

struct SeqRange {
  int L, nb, lo, hi, ord, chunks, base;  // base: first workspace slot of the sequence
  bool ok;
};

// A sequence's length and workspace slots, read with scalar loads (constant
// address space): they are waited for through lgkmcnt, never through vmcnt, so
// they can be fetched ahead without tying a wait to the page transfers.
#define CONST_AS __attribute__((address_space(4)))
struct SeqDesc {
  int L, base, next;  // cache_seqlens[b], num_splits[b], num_splits[b + 1]
};
__device__ __forceinline__ SeqDesc load_seq(const DecodeParams& p, int b) {
  const CONST_AS int32_t* sl = (const CONST_AS int32_t*)p.seqlens;
  const CONST_AS int32_t* ns = (const CONST_AS int32_t*)p.num_splits;
  return SeqDesc{sl[b], ns[b], ns[b + 1]};
}

__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, const SeqDesc& d, int b, int i0, int f0,
                                              int j0, int e0, int ord0) {
  SeqRange r;
  r.L = d.L;
  if (r.L < 0) r.L = 0;
  r.nb = (r.L + kPage - 1) / kPage;
  r.lo = (b == i0) ? f0 : 0;
  r.hi = (b == j0) ? e0 : (r.nb > 1 ? r.nb : 1);
  if (r.hi > r.nb) r.hi = r.nb;
  if (r.lo < 0) r.lo = 0;
  if (r.lo > r.hi) r.lo = r.hi;
  r.ord = (b == i0) ? ord0 : 0;
  r.base = d.base;
  r.chunks = d.next - r.base;
  // metadata that does not belong to these lengths / part count must not make
  // the epilogue write outside the workspace: such a chunk writes nothing
  const long long slot = (long long)r.base + r.ord;
  r.ok = r.ord >= 0 && r.ord < r.chunks && slot >= 0 && slot < (long long)p.batch + p.num_parts;
  return r;
}
__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b, int i0, int f0, int j0, int e0,
                                              int ord0) {
  return seq_range(p, load_seq(p, b), b, i0, f0, j0, e0, ord0);
}

// Block-table entries of pages [base, base + 64) of sequence b, one per lane
// (-1 past the table); a page's id is then read with readlane, so the DMA for a
// page never waits on a dependent global load.  Entries past the sequence's
// last page are read (in bounds of the table) but never used, which lets the
// load start before the sequence length is known.
__device__ __forceinline__ int load_page_ids(const DecodeParams& p, int b, int base, int lane) {
  const int j = base + lane;
  return j < p.max_blocks ? p.block_table[(long long)b * p.max_blocks + j] : -1;
}
__device__ __forceinline__ int page_id(int ids, int k) { return __builtin_amdgcn_readlane(ids, k); }

// Resource descriptor for page `blk` (physical id pid) of a sequence of length
// L: the page's bytes for this layout, clipped to the valid tokens so slots past
// L (and unknown page ids) read as zeros.
__device__ __forceinline__ i32x4_t page_rsrc(const DecodeParams& p, int pid, int blk, int L,
                                             int row_bytes = kRowBytes) {
  int valid = L - blk * kPage;
  if (valid > kPage) valid = kPage;
  const bool ok = pid >= 0 && (long long)pid < p.num_pages;
  const long long page_stride = (long long)kPage * p.h_kv * row_bytes;
  const char* base = (const char*)p.kcache + (ok ? (long long)pid * page_stride : 0);
  return make_rsrc(base, ok ? (uint32_t)(valid * p.h_kv * row_bytes) : 0u);
}

// Per-lane source offsets of a slice DMA: instruction (half th, group g) writes
// LDS bytes [g*2048 + th*1024, +1024) = tokens 8th..8th+7 of chunk group g, and
// lane i supplies token 8th + i/8, chunk 8g + ((i%8) ^ swz(token)).  The byte
// offset is vbase[th] + 128*g, so two registers cover all 18 instructions.
struct SliceDma {
  int vbase[2];
};
__device__ __forceinline__ SliceDma slice_dma_offsets(int tok0, int kvh, int h_kv, int lane) {
  SliceDma d;
#pragma unroll
  for (int th = 0; th < 2; ++th) {
    const int t = 8 * th + (lane >> 3);
    d.vbase[th] = ((tok0 + t) * h_kv + kvh) * kRowBytes + (((lane & 7) ^ swz(t)) << 4);
  }
  return d;
}
// One 1 KB HBM -> LDS transfer: 16 bytes per lane from rsrc + voffset to LDS
// dst + 16 * lane.  Written as inline assembly so the compiler does not track
// it: it would otherwise treat every later LDS read as possibly aliasing the
// transfer in flight and wait for all outstanding loads before it, which
// serialises the page pipeline; the kernels wait for their transfers explicitly
// (wait_vmcnt) before reading the LDS they fill.  The instruction has no
// register result.  M0 holds the LDS base; one wait state separates its write
// from the transfer that reads it.  The immediate offset would move the LDS
// destination as well, so the source offset is all in voffset.
__device__ __forceinline__ void dma16(LDS_AS char* dst, i32x4_t rsrc, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"((unsigned)(size_t)dst), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
template <int G>
__device__ __forceinline__ void dma_group(LDS_AS char* dst, i32x4_t rsrc, const SliceDma& d) {
  dma16(dst + G * kGroupBytes, rsrc, d.vbase[0] + G * 128);
  dma16(dst + G * kGroupBytes + 1024, rsrc, d.vbase[1] + G * 128);
}
// Piece i (0..17) of a slice transfer: chunk group i / 2, token half i % 2.
// Lets a kernel spread a slice's transfers over its compute instead of issuing
// them back to back: a burst of transfers stalls the issuing wave for as long
// as the memory pipeline takes to accept them.
__device__ __forceinline__ void dma_piece(LDS_AS char* dst, i32x4_t rsrc, const SliceDma& d, int i) {
  const int g = i >> 1, th = i & 1;
  dma16(dst + g * kGroupBytes + th * 1024, rsrc, d.vbase[th] + g * 128);
}
template <int... Gs>
__device__ __forceinline__ void dma_groups(LDS_AS char* dst, i32x4_t rsrc, const SliceDma& d,
                                           std::integer_sequence<int, Gs...>) {
  (dma_group<Gs>(dst, rsrc, d), ...);
}
// Move tokens [tok0, tok0 + 16) of one page (KV head kvh) into a 16-token LDS
// slice: 18 instructions (9 chunk groups x 2 token halves).
__device__ __forceinline__ void dma_slice(LDS_AS char* dst, i32x4_t rsrc, const SliceDma& d) {
  dma_groups(dst, rsrc, d, std::make_integer_sequence<int, 9>{});
}

// FP8 cache (656-byte rows, see kF8RowBytes).  A 16-token slice moves as 656
// token-major 16-byte chunks: 10 full transfers and one of 16 lanes; lane i of
// transfer k supplies chunk 64k + i.  Its LDS image is dequantised into the
// bf16 slice layout above before the slice is used, so the scoring and PV code
// is the same for both formats.
constexpr int kF8SliceBytes = kSlice * kF8RowBytes;             // 10496
constexpr int kF8Chunks = kF8RowBytes / 16;                     // 41 per row
constexpr int kF8SliceDma = (kF8SliceBytes + 1023) / 1024;      // 11
constexpr int kF8LastLanes = (kF8SliceBytes - 1024 * (kF8SliceDma - 1)) / 16;  // 16
struct F8Dma {
  int off[kF8SliceDma];
};
__device__ __forceinline__ F8Dma fp8_dma_offsets(int tok0, int kvh, int h_kv, int lane) {
  F8Dma d;
#pragma unroll
  for (int k = 0; k < kF8SliceDma; ++k) {
    const int n = 64 * k + lane;
    const int t = n < kSlice * kF8Chunks ? n / kF8Chunks : 0;  // lanes past the slice never transfer
    d.off[k] = ((tok0 + t) * h_kv + kvh) * kF8RowBytes + 16 * (n - t * kF8Chunks);
  }
  return d;
}
__device__ __forceinline__ void dma_slice_fp8(LDS_AS char* dst, i32x4_t rsrc, const F8Dma& d, int lane) {
#pragma unroll
  for (int k = 0; k < kF8SliceDma - 1; ++k) dma16(dst + 1024 * k, rsrc, d.off[k]);
  if (lane < kF8LastLanes) dma16(dst + 1024 * (kF8SliceDma - 1), rsrc, d.off[kF8SliceDma - 1]);
}
__device__ __forceinline__ unsigned cvt_fp8x2(unsigned v, float scale, bool hi_word) {
  // e4m3 -> bf16 with a power-of-two scale (the instruction uses the scale's
  // exponent), exact
  return hi_word ? __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, scale, true))
                 : __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, scale, false));
}
// FP8 slice image (token-major rows) -> bf16 slice (swizzled).  Lane l takes
// token l%16 and latent group l/16: 128 dims with that group's scale, plus rope
// dims 16(l/16) .. +15 copied as they are.  With the token in the low lane bits
// the 16 lanes of a group read 16 distinct 16-byte bank groups (rows are 656 =
// 144 mod 256 bytes apart) and write 16 distinct ones (the slice swizzle).
__device__ __forceinline__ void dequant_slice(const LDS_AS char* src, LDS_AS char* dst, int lane) {
  const int t = lane & 15, g = lane >> 4;
  const LDS_AS char* row = src + t * kF8RowBytes;
  // every read first, so that one LDS round trip covers them all
  u32x4_t v[8], rope[2];
#pragma unroll
  for (int c = 0; c < 8; ++c) v[c] = *(const LDS_AS u32x4_t*)(row + g * kF8Group + 16 * c);
#pragma unroll
  for (int c = 0; c < 2; ++c) rope[c] = *(const LDS_AS u32x4_t*)(row + kLatent + 16 + 32 * g + 16 * c);
  const float sc = *(const LDS_AS float*)(row + kLatent + 4 * g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4_t lo = {cvt_fp8x2(v[c][0], sc, false), cvt_fp8x2(v[c][0], sc, true), cvt_fp8x2(v[c][1], sc, false),
                        cvt_fp8x2(v[c][1], sc, true)};
    const u32x4_t hi = {cvt_fp8x2(v[c][2], sc, false), cvt_fp8x2(v[c][2], sc, true), cvt_fp8x2(v[c][3], sc, false),
                        cvt_fp8x2(v[c][3], sc, true)};
    *(LDS_AS u32x4_t*)(dst + slice_off(t, 16 * g + 2 * c)) = lo;
    *(LDS_AS u32x4_t*)(dst + slice_off(t, 16 * g + 2 * c + 1)) = hi;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) *(LDS_AS u32x4_t*)(dst + slice_off(t, 64 + 2 * g + c)) = rope[c];
}

// Token-sparse decode.  A wave's 16-token slice of page blk of sequence b is
// rows sp_offs[sp_rowptr[b] + 64 blk + 16 w + t], t < 16 (byte offsets; the
// array is padded by one page, so a last page's reads stay inside it).  The 16
// offsets move into LDS with one 16-lane transfer (4 bytes per lane), counted
// with the page transfers, and each lane then reads the offsets of its two
// tokens: no registers hold a page's offsets while it is in flight.
__device__ __forceinline__ void dma4(LDS_AS char* dst, i32x4_t rsrc, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)dst)), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void stage_offs(LDS_AS char* dst, i32x4_t offs_rsrc, int row0, int blk, int w, int lane) {
  if (lane < kSlice) dma4(dst, offs_rsrc, (row0 + blk * kPage + w * kSlice + lane) * 4);
}
// per-lane transfer offsets of a gathered slice: the swizzle of
// slice_dma_offsets with each token's row read from the staged list; tokens past
// the sequence's kept keys read zeros
__device__ __forceinline__ SliceDma gathered_dma(const LDS_AS char* staged, int valid, int kvh, int lane) {
  SliceDma d;
#pragma unroll
  for (int th = 0; th < 2; ++th) {
    const int t = 8 * th + (lane >> 3);
    uint32_t off = *(const LDS_AS uint32_t*)(staged + 4 * t);
    if (t >= valid) off = kSparseNone;
    d.vbase[th] = (int)(off + (uint32_t)(kvh * kRowBytes) + (uint32_t)(((lane & 7) ^ swz(t)) << 4));
  }
  return d;
}

__device__ __forceinline__ void row_coords(const DecodeParams& p, int b, int kvh, int row, int& s,
                                           long long& qo) {
  s = row / p.group;
  const int h = kvh * p.group + row % p.group;
  qo = ((long long)b * p.s_q + s) * p.h_q + h;  // flat (b, s, h) index
}

// ---------------------------------------------------------------------------
// <= 16 rows: token-split kernel.
// The part's pages form one stream across its sequences: while a page is
// processed the next one of the stream -- possibly the first page of the next
// sequence -- is on its way into the other LDS buffer, and the next sequence's
// length and page ids load while the current one runs, its queries during the
// current one's epilogue.
// LDS: per wave two 16-token transfer slots + merge statistics; with the FP8
// cache the slots hold FP8 images (2 x 10496 B) and a third region holds the
// dequantised bf16 slice the wave computes on.  At a chunk end the waves merge
// their partial outputs through the slot just consumed.
template <bool kFp8>
struct TsLayout {
  static constexpr int kSlot = kFp8 ? kF8SliceBytes : kSliceBytes;
  static constexpr int kWave = kFp8 ? 2 * kF8SliceBytes + kSliceBytes : 2 * kSliceBytes;
  static constexpr int kDma = kFp8 ? kF8SliceDma : kSliceDma;  // transfers per slice issue
  static constexpr int kStat = 4 * kWave;                        // [4 waves][16 rows][m, l]
  static constexpr int kLds = kStat + 4 * 16 * 2 * 4;
};

template <bool kFp8>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
decode_tokensplit(DecodeParams p) {
  using Lay = TsLayout<kFp8>;
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  LDS_AS char* smem = (LDS_AS char*)smem_generic;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, mt, kvh;
  map_block(p, part, mt, kvh);
  const int32_t* md = p.tile_md + (long long)part * kMdInts;
  const int i0 = md[0], f0 = md[1], e0 = md[3], ord0 = md[4];
  const int j0 = min(md[2], p.batch - 1);
  if (i0 >= p.batch || i0 < 0) return;

  LDS_AS char* slices = smem + w * Lay::kWave;                     // transfer slot k at k * Lay::kSlot
  LDS_AS char* bslice = smem + w * Lay::kWave + 2 * kF8SliceBytes;  // FP8 only: dequantised slice
  LDS_AS float* mstat = (LDS_AS float*)(smem + Lay::kStat);         // [4 waves][16 rows][2]

  // lane roles: QK output / PV operand B -> query row (lane & 15)
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int row = mt * 16 + r16;
  const bool row_ok = row < p.rows;
  // per-lane LDS bases inside a slice (see slice_off)
  int kaddr[2], vaddr[4];
#pragma unroll
  for (int k = 0; k < 2; ++k) kaddr[k] = slice_off(r16, 4 * k + grp);
  {
    const int tt = grp * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) vaddr[k] = slice_off(tt, 2 * k + ((lane & 3) >> 1)) + ((lane & 1) << 3);
  }
  SliceDma dma;
  F8Dma f8dma;
  if constexpr (kFp8) f8dma = fp8_dma_offsets(w * kSlice, kvh, p.h_kv, lane);
  else dma = slice_dma_offsets(w * kSlice, kvh, p.h_kv, lane);
  // this wave's slice of page blk of sequence range r, whose id is entry k of the
  // block-table window `ids_` (entries r.lo .. r.lo + 63)
  auto issue = [&](LDS_AS char* dst, int ids_, int k, int blk_, const SeqRange& r) {
    if constexpr (kFp8) dma_slice_fp8(dst, page_rsrc(p, page_id(ids_, k), blk_, r.L, kF8RowBytes), f8dma, lane);
    else dma_slice(dst, page_rsrc(p, page_id(ids_, k), blk_, r.L), dma);
  };

  // queries: B operand of the 16x16x32 QK MFMA, 8 dims per lane per k-step.
  // Rows past the last one (a ragged tile) compute on row 0's query; every row
  // is independent through the softmax and PV, and such rows are never stored,
  // so the loads need no mask and nothing waits for them before first use.
  bf16x8_t qreg[18];
  auto load_q = [&](int bq) {
    int s;
    long long qo;
    row_coords(p, bq, kvh, row_ok ? row : 0, s, qo);
    const bf16x8_t* qp = (const bf16x8_t*)(p.q + qo * kDqk) + grp;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = qp[ks * 4];
  };

  // in-flight DMA only ever targets buffer `buf`; buf ^ 1 is free between pages.
  // Sequence descriptors (lengths, page ids) are loaded two sequences ahead and
  // queries one ahead, so each is complete at the drain that ends the epilogue
  // before the one that uses it.
  int buf = 0;
  int b = i0;
  int ids = load_page_ids(p, b, f0, lane);
  SeqRange sr = seq_range(p, b, i0, f0, j0, e0, ord0);
  load_q(b);
  SeqDesc nd = {};
  int nids = -1;
  if (b < j0) {
    nids = load_page_ids(p, b + 1, 0, lane);
    nd = load_seq(p, b + 1);
  }
  vm_drain();
  SeqRange nr = seq_range(p, nd, b + 1, i0, f0, j0, e0, ord0);
  if (sr.lo != f0) {  // clamped (malformed) metadata
    ids = load_page_ids(p, b, sr.lo, lane);
    vm_drain();
  }
  if (sr.lo < sr.hi) issue(slices, ids, 0, sr.lo, sr);
  for (;;) {
    const bool has_next = b < j0;
    SeqDesc nd2 = {};
    int nids2 = -1;
    if (b + 1 < j0) {
      nids2 = load_page_ids(p, b + 2, 0, lane);
      nd2 = load_seq(p, b + 2);
    }
    int s;
    long long qo;
    row_coords(p, b, kvh, row_ok ? row : 0, s, qo);
    const int nkeys = p.causal ? max(0, sr.L - p.s_q + s + 1) : sr.L;

    f32x4_t O[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) O[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    bool next_started = false;  // first page of the next sequence already requested
    for (int blk = sr.lo; blk < sr.hi; ++blk) {
      if (blk + 1 < sr.hi) {
        const int k = (blk + 1 - sr.lo) & 63;
        if (k == 0) ids = load_page_ids(p, b, blk + 1, lane);
        issue(slices + (buf ^ 1) * Lay::kSlot, ids, k, blk + 1, sr);
        wait_vmcnt<Lay::kDma>();
      } else if (has_next && nr.lo < nr.hi) {
        issue(slices + (buf ^ 1) * Lay::kSlot, nids, 0, nr.lo, nr);
        next_started = true;
        wait_vmcnt<Lay::kDma>();
      } else {
        wait_vmcnt<0>();
      }
      const LDS_AS char* reg = slices + buf * Lay::kSlot;
      if constexpr (kFp8) {
        dequant_slice(reg, bslice, lane);
        reg = bslice;
      }

      // S^T[16 tokens x 16 rows] = K_slice . Q^T ; A-operand row = token r16,
      // chunk 4*ks + grp = group ks/2, position 4*(ks&1) + grp.  Three
      // accumulation chains; K operands are read kAhead k-steps ahead.
      f32x4_t S;
      {
        constexpr int kAhead = 4;
        f32x4_t Sc[3] = {};
        bf16x8_t ka[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
          ka[i] = *(const LDS_AS bf16x8_t*)(reg + kaddr[i & 1] + (i >> 1) * kGroupBytes);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if (ks + kAhead < 18) {
            const int n = ks + kAhead;
            ka[n % (kAhead + 1)] = *(const LDS_AS bf16x8_t*)(reg + kaddr[n & 1] + (n >> 1) * kGroupBytes);
          }
          Sc[ks % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % (kAhead + 1)], qreg[ks], Sc[ks % 3], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ks + kAhead < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        S = Sc[0] + Sc[1] + Sc[2];
      }
      __builtin_amdgcn_sched_barrier(0);
      // online softmax over this wave's 16 tokens: lane holds tokens grp*4 + i of row r16
      const int tok0 = blk * kPage + w * kSlice + grp * 4;
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (tok0 + i < nkeys) ? S[i] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = wave_max16(mx);
      float alpha = 1.f;
      if (mx > m_run + kTau) {
        alpha = __builtin_amdgcn_exp2f(m_run - mx);  // 0 when m_run == -inf
        m_run = mx;
        l_run *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float pr[4];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
        ps += pr[i];
      }
      l_run += wave_sum16(ps);
      u32x2_t pb = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
      const s16x4_t pbs = __builtin_bit_cast(s16x4_t, pb);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 32; ++i) O[i] *= alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
      // O^T[16 dims x 16 rows] += V^T[16 dims x 16 tokens] . P^T, 32 dim tiles;
      // dims 16*dt + (lane&3)*4 = group dt/4, position 2*(dt&3) + (lane&3)/2.
      // Transposed reads run kVAhead tiles ahead of their MFMA.
      {
        constexpr int kVAhead = 8;
        bf16x4_t va[kVAhead + 1];
#pragma unroll
        for (int i = 0; i < kVAhead; ++i) va[i] = lds_tr16(reg + vaddr[i & 3] + (i >> 2) * kGroupBytes);
        __builtin_amdgcn_sched_group_barrier(0x100, kVAhead, 0);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          if (dt + kVAhead < 32) {
            const int n = dt + kVAhead;
            va[n % (kVAhead + 1)] = lds_tr16(reg + vaddr[n & 3] + (n >> 2) * kGroupBytes);
          }
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, va[dt % (kVAhead + 1)]),
                                                            pbs, O[dt], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (dt + kVAhead < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      buf ^= 1;
    }
    // the next sequence's queries load during this epilogue
    if (has_next) load_q(b + 1);

    // ---- merge the four waves' partial softmax states through LDS (the
    // buffer just consumed, buf ^ 1, of every wave), then write
    // the merge goes through a region no transfer targets: the slot just
    // consumed (bf16) or the dequantised slice (FP8)
    const int dbuf = kFp8 ? 2 * kF8SliceBytes : (buf ^ 1) * kSliceBytes;
    wg_barrier();  // every wave is done with its slices
    if (lane < 16) *(LDS_AS f32x2_t*)(mstat + (w * 16 + lane) * 2) = f32x2_t{m_run, l_run};
    wg_barrier();
    // Each wave produces the 64-dim slab 64 w .. 64 w + 63 of each half of the
    // output rows, in the MFMA layout itself (row r16, dims 16 dt + 4 grp .. +3,
    // dim tiles 4 w .. 4 w + 3): its own contribution stays in registers and
    // only the three other waves' values go through LDS.  With M the largest of
    // the four waves' maxima m_v, a row is sum_v 2^(m_v - M) O_v / sum_v
    // 2^(m_v - M) l_v; each wave's weight, divided by that sum, multiplies its
    // O_v as it is summed (a wave that saw no key has m_v = -inf, O_v = 0,
    // l_v = 0 and weight 0).
    const int rr = r16;
    const int rrow = mt * 16 + rr;
    float mv[4], lv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x2_t st = *(const LDS_AS f32x2_t*)(mstat + (v * 16 + rr) * 2);
      mv[v] = st[0];
      lv[v] = st[1];
    }
    const float M = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));
    float cv[4], lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      cv[v] = (mv[v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv[v] - M);
      lsum += cv[v] * lv[v];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) cv[v] *= inv;
    int rs;
    long long ro;
    row_coords(p, b, kvh, rrow < p.rows ? rrow : 0, rs, ro);
    const bool split = sr.chunks > 1;
    const long long slot_row = ((long long)(sr.base + sr.ord) * p.h_kv + kvh) * p.rows + rrow;
    constexpr int kDumpStride = 260;  // floats per row: 256 + 4 pad
    // the merge for wave index W (a compile-time constant: no dynamic indexing of O)
    auto merge = [&](auto W) {
      constexpr int kW = decltype(W)::value;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        LDS_AS float* dump = (LDS_AS float*)(smem + kW * Lay::kWave + dbuf);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
          if (dt / 4 != kW) *(LDS_AS f32x4_t*)(dump + r16 * kDumpStride + dt * 16 + grp * 4) = O[half * 16 + dt];
        wg_barrier();
        // the other waves' 12 reads in flight before the first sum
        f32x4_t xs[3][4];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int v = (kW + 1 + j) & 3;
          const LDS_AS float* src = (const LDS_AS float*)(smem + v * Lay::kWave + dbuf);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            xs[j][k] = *(const LDS_AS f32x4_t*)(src + r16 * kDumpStride + (4 * kW + k) * 16 + grp * 4);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
        f32x4_t acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[k] = cv[kW] * O[half * 16 + 4 * kW + k] + cv[(kW + 1) & 3] * xs[0][k] +
                   cv[(kW + 2) & 3] * xs[1][k] + cv[(kW + 3) & 3] * xs[2][k];
        if (rrow < p.rows && sr.ok) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int d0 = half * 256 + (4 * kW + k) * 16 + grp * 4;
            if (split) {
              *(f32x4_t*)(p.o_acc + slot_row * kDv + d0) = acc[k];
            } else {
              const u32x2_t pk = {pack_bf16(acc[k][0], acc[k][1]), pack_bf16(acc[k][2], acc[k][3])};
              *(u32x2_t*)(p.out + ro * kDv + d0) = pk;
            }
          }
        }
        wg_barrier();
      }
    };
    switch (w) {
      case 0: merge(std::integral_constant<int, 0>{}); break;
      case 1: merge(std::integral_constant<int, 1>{}); break;
      case 2: merge(std::integral_constant<int, 2>{}); break;
      default: merge(std::integral_constant<int, 3>{}); break;
    }
    if (w == 0 && grp == 0 && rrow < p.rows && sr.ok) {
      const float l2 = lsum > 0.f ? M + __builtin_amdgcn_logf(lsum) : -INFINITY;
      if (split) p.lse_acc[slot_row] = l2;
      else p.lse[ro] = l2 * kLn2;
    }
    if (!has_next) break;
    vm_drain();  // the next queries and descriptors (and this epilogue's stores)
    // advance the stream; an empty sequence requested nothing, so its successor
    // starts its own first page now (buffer `buf`, idle)
    ++b;
    sr = nr;
    ids = nids;
    nr = seq_range(p, nd2, b + 1, i0, f0, j0, e0, ord0);
    nids = nids2;
    if (!next_started && sr.lo < sr.hi) issue(slices + buf * Lay::kSlot, ids, 0, sr.lo, sr);
  }
}

// ---------------------------------------------------------------------------
// 64-row tiles: pair-split kernel.
// The 4 waves form a 2 x 2 grid: wave w owns query rows 32*(w&1) .. +31 (its
// queries stay in registers) and tokens 32*(w>>1) .. +31 of every page for
// QK^T.  The two waves of a row group agree on one running max per page through
// LDS, so their P blocks share a reference; P goes to LDS and PV is split by
// output dims (128 per wave, all 64 rows), which reads every V element of the
// page from LDS once per workgroup.
// LDS: two page buffers (bf16 pages, or FP8 pages in their first 82 KB), P
// [64 rows x 64 tokens] bf16, the per-page row maxima of both token groups,
// alpha, the end-of-chunk (m, l) of both token groups, the token-sparse row
// offsets and the FP8 page's scale table.  At a chunk end the page buffers
// stage each wave's output rows.
constexpr int kPsRows = 64;
constexpr int kPsPbuf = 2 * kPageBytes;
constexpr int kPsXmax = kPsPbuf + kPsRows * 128;
constexpr int kPsAbuf = kPsXmax + 2 * kPsRows * 4;
constexpr int kPsSbuf = kPsAbuf + kPsRows * 4;
constexpr int kPsOffs = kPsSbuf + 2 * kPsRows * 2 * 4;  // token-sparse: [2 page slots][4 waves][16] row offsets
// chunk end: per wave, its 128 output dims of the 64 rows as [row][dim] fp32
// (row stride 132 floats) plus the rows' output offsets, inside the page buffers
constexpr int kPsStgStride = 132;
constexpr int kPsStgBytes = kPsRows * kPsStgStride * 4 + kPsRows * 8;
static_assert(4 * kPsStgBytes <= kPsPbuf, "the chunk-end staging must fit in the page buffers");
constexpr int kPsScl = kPsOffs + 2 * 4 * kSlice * 4;    // FP8 pages: [4 groups][64 tokens] fp32 scales of the page
constexpr int kPsLds = kPsScl + 4 * kPage * 4;
// transfer pieces of the next page issued during QK^T (the rest during PV)
#ifndef MLA_QK_DMA
#define MLA_QK_DMA 18
#endif
constexpr int kQkDma = MLA_QK_DMA;
// transfer pieces issued during the softmax (after the QK^T ones); the rest go
// during PV
#ifndef MLA_SM_DMA
#define MLA_SM_DMA 0
#endif
constexpr int kSmDma = MLA_SM_DMA;
constexpr int kPvDma0 = kQkDma + kSmDma;

// P row r holds 64 bf16 tokens as 8 chunks of 16 bytes; chunk c is stored at
// position c ^ ((r >> 1) & 7), which keeps 16 consecutive rows reading the same
// chunk on 16 different bank groups.
__device__ __forceinline__ int pbuf_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// FP8 pages in the 64-row kernel.  A page lives in LDS as its 64 token-major
// 656-byte rows: 41 transfers of 1 KB, wave w issuing transfers w, w + 4, ...
// Rows 656 bytes apart put 16 consecutive tokens on 16 distinct 16-byte bank
// groups, so the K operand reads (16 bytes of one token per lane) and the
// transposed V reads are conflict free without a swizzle.
constexpr int kF8PageBytes = kPage * kF8RowBytes;  // 41984
constexpr int kF8PageDma = kF8PageBytes / 1024;     // 41
constexpr int kF8WaveDma = (kF8PageDma + 3) / 4;    // 11 (waves 1-3 issue 10)
static_assert(kF8PageBytes % 1024 == 0, "an FP8 page is a whole number of transfers");
struct PageDmaF8 {
  int off[kF8WaveDma];
};
__device__ __forceinline__ PageDmaF8 fp8_page_dma_offsets(int w, int kvh, int h_kv, int lane) {
  PageDmaF8 d;
#pragma unroll
  for (int i = 0; i < kF8WaveDma; ++i) {
    const int o = 1024 * (w + 4 * i) + 16 * lane;  // byte of the LDS page image
    const int t = o / kF8RowBytes;                 // its token and byte within the row
    d.off[i] = (t * h_kv + kvh) * kF8RowBytes + (o - t * kF8RowBytes);
  }
  return d;
}
// transfer i of wave w's share of an FP8 page
__device__ __forceinline__ void dma_piece_f8(LDS_AS char* page, i32x4_t rsrc, const PageDmaF8& d, int w, int i) {
  if (w + 4 * i < kF8PageDma) dma16(page + 1024 * (w + 4 * i), rsrc, d.off[i]);
}
// 8 e4m3 codes (two words) -> 8 bf16 times a power-of-two scale (exact)
__device__ __forceinline__ bf16x8_t cvt8_fp8(unsigned w0, unsigned w1, float sc) {
  const u32x4_t r = {cvt_fp8x2(w0, sc, false), cvt_fp8x2(w0, sc, true), cvt_fp8x2(w1, sc, false),
                     cvt_fp8x2(w1, sc, true)};
  return __builtin_bit_cast(bf16x8_t, r);
}
// 8 bf16 values, element j times sc[j] (powers of two: exact while the
// products stay in bf16's normal range)
__device__ __forceinline__ bf16x8_t scale8(bf16x8_t v, const float* sc) {
  const u32x4_t u = __builtin_bit_cast(u32x4_t, v);
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_bf16(__builtin_bit_cast(float, u[i] << 16) * sc[2 * i],
                     __builtin_bit_cast(float, u[i] & 0xffff0000u) * sc[2 * i + 1]);
  return __builtin_bit_cast(bf16x8_t, r);
}
typedef int i32x2_t __attribute__((ext_vector_type(2)));

template <bool kSparse, bool kFp8>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
decode_pairsplit(DecodeParams p) {
  static_assert(!(kSparse && kFp8), "the token-sparse decode reads bf16 rows");
  constexpr int kPg = kFp8 ? kF8PageBytes : kPageBytes;  // LDS bytes of one page
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  LDS_AS char* smem = (LDS_AS char*)smem_generic;
  LDS_AS char* pages = smem;
  LDS_AS char* pbuf = smem + kPsPbuf;
  LDS_AS float* xmax = (LDS_AS float*)(smem + kPsXmax);  // [2 token groups][64 rows]
  LDS_AS float* abuf = (LDS_AS float*)(smem + kPsAbuf);  // [64 rows]
  LDS_AS float* sbuf = (LDS_AS float*)(smem + kPsSbuf);  // [2 token groups][64 rows][2]
  LDS_AS float* scl = (LDS_AS float*)(smem + kPsScl);    // FP8 pages: [4 groups][64 tokens]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, mt, kvh;
  map_block(p, part, mt, kvh);
  const int32_t* md = p.tile_md + (long long)part * kMdInts;
  const int i0 = md[0], f0 = md[1], e0 = md[3], ord0 = md[4];
  const int j0 = min(md[2], p.batch - 1);
  if (i0 >= p.batch || i0 < 0) return;

  const int l32 = lane & 31;
  const int hb = lane >> 5;   // which 8-element half of a k-step this lane holds
  const int g16 = lane >> 4;
  const int k16 = lane & 15;
  const int rg = w & 1;       // row group of this wave in QK
  const int tg = w >> 1;      // token group of this wave in QK
  const int trow = rg * 32 + l32;          // row inside the tile (QK phase)
  const int qrow = mt * kPsRows + trow;
  const bool qrow_ok = qrow < p.rows;

  // K operand of QK: token 32*tg + l32 -> slice 2*tg + l32/16, token l32 & 15;
  // chunk 2*ks + hb -> group ks/4, position 2*(ks&3) + hb.
  int kaddr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) kaddr[k] = (2 * tg + (l32 >> 4)) * kSliceBytes + slice_off(l32 & 15, 2 * k + hb);
  // V^T operand of PV (transposed read) for tokens 16*ks + 8*(g16>>1) + k16/4 (+4):
  // slice ks, token 8*(g16>>1) + k16/4 (+4); dims 128*w + 32*dt + 16*(g16&1) + 4*(k16&3)
  // -> group 2*w + dt/2, position 4*(dt&1) + 2*(g16&1) + (k16&3)/2, byte 8*(k16&1).
  int vaddr[2][2];
#pragma unroll
  for (int p4 = 0; p4 < 2; ++p4)
#pragma unroll
    for (int d1 = 0; d1 < 2; ++d1) {
      const int t = 8 * (g16 >> 1) + (k16 >> 2) + 4 * p4;
      const int pos = 4 * d1 + 2 * (g16 & 1) + ((k16 & 3) >> 1);
      vaddr[p4][d1] = t * 128 + ((pos ^ swz(t)) << 4) + ((k16 & 1) << 3) + 2 * w * kGroupBytes;
    }
  // P^T operand of PV: row 32*rt + l32, tokens 16*ks + 8*hb .. +7 = chunk 2*ks + hb
  int paddr[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) paddr[rt][ks] = pbuf_off(rt * 32 + l32, 2 * ks + hb);
  const SliceDma dma = slice_dma_offsets(w * kSlice, kvh, p.h_kv, lane);
  // FP8 pages: the K operand row of this lane's token; the transposed V read of
  // lanes 2k, 2k+1 of a 16-lane group addresses token k of the group's 8 at
  // bytes +0 / +8, so that lane i receives dim i of 8 consecutive tokens
  // (16 tokens per k-step: 8 * hb + k16 / 2; dims 128 w + 32 dt + 16 (g16 & 1) + k16)
  int frow = 0, vaddr8 = 0;
  PageDmaF8 fdma = {};
  if constexpr (kFp8) {
    frow = (32 * tg + l32) * kF8RowBytes;
    vaddr8 = (8 * hb + (k16 >> 1)) * kF8RowBytes + 128 * w + 16 * (g16 & 1) + 8 * (k16 & 1);
    fdma = fp8_page_dma_offsets(w, kvh, p.h_kv, lane);
  }
  i32x4_t offs_rsrc = {};
  if constexpr (kSparse) offs_rsrc = make_rsrc(p.sp_offs, 0xffffffffu);  // the row-offset list

  for (int b = i0; b <= j0; ++b) {
    const SeqRange sr = seq_range(p, b, i0, f0, j0, e0, ord0);
    int s;
    long long qo;
    row_coords(p, b, kvh, qrow_ok ? qrow : 0, s, qo);
    const int nkeys = p.causal ? max(0, sr.L - p.s_q + s + 1) : sr.L;

    // rows past the last one compute on row 0's query and are never stored
    // (FP8 pages: k-steps 2j, 2j+1 of the latent take bytes 0-7 / 8-15 of the
    // 16-byte chunk 32 j + 16 hb, i.e. dims 32 j + 16 hb + 8 (ks & 1) .. +7)
    bf16x8_t qreg[36];
    {
      const bf16x8_t* qp = (const bf16x8_t*)(p.q + qo * kDqk);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks)
        qreg[ks] = qp[kFp8 && ks < 32 ? 4 * (ks >> 1) + 2 * hb + (ks & 1) : 2 * ks + hb];
    }
    f32x16_t O[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt][0] = O[dt][1] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;  // l_run covers this wave's token group only

    // token-sparse: the sequence's rows are listed, not paged; the offsets of
    // page blk + 1 are staged one page ahead (LDS slot by page parity)
    i32x4_t grsrc = {};
    if constexpr (kSparse) grsrc = make_rsrc(p.kcache, p.sp_cache_bytes);
    const auto slice_valid = [&](int blk_) { return min(max(sr.L - blk_ * kPage - w * kSlice, 0), kSlice); };
    LDS_AS char* offs_slot[2] = {smem + kPsOffs + w * 64, smem + kPsOffs + (4 + w) * 64};
    int row0 = 0;
    int ids = -1;
    if constexpr (kSparse) {
      row0 = ((const CONST_AS int32_t*)p.sp_rowptr)[b];
      if (sr.lo < sr.hi) {
        stage_offs(offs_slot[0], offs_rsrc, row0, sr.lo, w, lane);
        if (sr.lo + 1 < sr.hi) stage_offs(offs_slot[1], offs_rsrc, row0, sr.lo + 1, w, lane);
        wait_vmcnt<0>();
        dma_slice(pages + w * kSliceBytes, grsrc, gathered_dma(offs_slot[0], slice_valid(sr.lo), kvh, lane));
      }
    } else {
      ids = load_page_ids(p, b, sr.lo, lane);
      if (sr.lo < sr.hi) {
        if constexpr (kFp8) {
          const i32x4_t r = page_rsrc(p, page_id(ids, 0), sr.lo, sr.L, kF8RowBytes);
#pragma unroll
          for (int i = 0; i < kF8WaveDma; ++i) dma_piece_f8(pages, r, fdma, w, i);
        } else {
          dma_slice(pages + w * kSliceBytes, page_rsrc(p, page_id(ids, 0), sr.lo, sr.L), dma);
        }
      }
    }
    for (int blk = sr.lo; blk < sr.hi; ++blk) {
      const int pb = (blk - sr.lo) & 1;
      wait_vmcnt<0>();
      wg_barrier();  // page blk visible; the other buffer, P and xmax are free
      // the next page's slice moves in pieces spread over this page's MFMAs:
      // kQkDma pieces during QK^T, the rest during PV
      const bool has_next = blk + 1 < sr.hi;
      LDS_AS char* npage = pages + (pb ^ 1) * kPg;
      LDS_AS char* ndst = npage + w * kSliceBytes;
      i32x4_t nrsrc = {0, 0, 0, 0};
      SliceDma ndma = dma;
      if (has_next) {
        if constexpr (kSparse) {
          const int ns = (blk + 1 - sr.lo) & 1;
          nrsrc = grsrc;
          ndma = gathered_dma(offs_slot[ns], slice_valid(blk + 1), kvh, lane);
          if (blk + 2 < sr.hi) stage_offs(offs_slot[ns ^ 1], offs_rsrc, row0, blk + 2, w, lane);
        } else {
          const int k = (blk + 1 - sr.lo) & 63;
          if (k == 0) ids = load_page_ids(p, b, blk + 1, lane);
          nrsrc = page_rsrc(p, page_id(ids, k), blk + 1, sr.L, kFp8 ? kF8RowBytes : kRowBytes);
        }
      }
      const LDS_AS char* page = pages + pb * kPg;

      // ---- S^T[32 tokens x 32 rows] = K . Q^T, two accumulation chains,
      // K operands fetched kAhead k-steps ahead.  The loop is instantiated with
      // and without the next page's transfer pieces so that no branch splits it.
      auto qk = [&](auto with_dma) {
        f32x16_t S0 = f32x16_t{}, S1 = f32x16_t{};
        constexpr int kAhead = 4;  // K operands in flight ahead of the MFMA that uses them
        bf16x8_t ka[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
          ka[i] = *(const LDS_AS bf16x8_t*)(page + kaddr[i & 3] + (i >> 2) * kGroupBytes);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          if (ks + kAhead < 36) {
            const int n = ks + kAhead;
            ka[n % (kAhead + 1)] = *(const LDS_AS bf16x8_t*)(page + kaddr[n & 3] + (n >> 2) * kGroupBytes);
          }
          if (ks & 1) S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (kAhead + 1)], qreg[ks], S1, 0, 0, 0);
          else S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (kAhead + 1)], qreg[ks], S0, 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ks + kAhead < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if constexpr (decltype(with_dma)::value) {
#pragma unroll
            for (int i = ks * kQkDma / 36; i < (ks + 1) * kQkDma / 36; ++i) dma_piece(ndst, nrsrc, ndma, i);
          }
        }
        return S0 + S1;
      };
      // FP8 pages: 20 operand reads per lane -- 16 latent chunks of 16 bytes (two
      // k-steps each, dequantised with the token's group scale) and 4 rope
      // k-steps of bf16 -- and the next page's kF8WaveDma transfers spread over them
      auto qk8 = [&](auto with_dma) {
        f32x16_t S0 = f32x16_t{}, S1 = f32x16_t{};
        const LDS_AS char* krow = page + frow;
        const f32x4_t sc = *(const LDS_AS f32x4_t*)(krow + kLatent);  // the token's 4 group scales
        if (rg == 0 && hb == 0) {  // waves 0 and 2 hold every token once: the PV waves' table
#pragma unroll
          for (int g = 0; g < 4; ++g) scl[g * kPage + 32 * tg + l32] = sc[g];
        }
        auto rd = [&](int r) {
          return *(const LDS_AS u32x4_t*)(krow + (r < 16 ? 32 * r + 16 * hb : kLatent + 16 + 32 * (r - 16) + 16 * hb));
        };
        constexpr int kAheadR = 3;  // operand reads in flight ahead of their MFMAs
        u32x4_t kr[kAheadR + 1];
#pragma unroll
        for (int i = 0; i < kAheadR; ++i) kr[i] = rd(i);
#pragma unroll
        for (int r = 0; r < 20; ++r) {
          if (r + kAheadR < 20) kr[(r + kAheadR) % (kAheadR + 1)] = rd(r + kAheadR);
          const u32x4_t c = kr[r % (kAheadR + 1)];
          if (r < 16) {
            const float s8 = sc[r >> 2];
            S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt8_fp8(c[0], c[1], s8), qreg[2 * r], S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt8_fp8(c[2], c[3], s8), qreg[2 * r + 1], S1, 0, 0, 0);
          } else {
            const int ks = 32 + (r - 16);
            if (ks & 1) S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c), qreg[ks], S1, 0, 0, 0);
            else S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c), qreg[ks], S0, 0, 0, 0);
          }
          if constexpr (decltype(with_dma)::value) {
#pragma unroll
            for (int i = r * kF8WaveDma / 20; i < (r + 1) * kF8WaveDma / 20; ++i) dma_piece_f8(npage, nrsrc, fdma, w, i);
          }
        }
        return S0 + S1;
      };
      f32x16_t S;
      if constexpr (kFp8) {
        if (has_next) S = qk8(std::true_type{});
        else S = qk8(std::false_type{});
      } else {
        if (has_next) S = qk(std::true_type{});
        else S = qk(std::false_type{});
      }
      __builtin_amdgcn_sched_barrier(0);
      // lane holds row trow, tokens 32*tg + 8*(r>>2) + 4*hb + (r&3) of the page.
      // Scores stay unscaled (the scale is positive, so the max commutes with
      // it) and keys past a row's last visible one are masked only on a page
      // that some row of the wave does not see whole.
      const int tok0 = blk * kPage + 32 * tg + 4 * hb;
      if (__builtin_amdgcn_ballot_w64((blk + 1) * kPage > nkeys)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tok0 + 8 * (r >> 2) + (r & 3) >= nkeys) S[r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r]);
      mx = half_max(mx) * p.scale_log2;
      if (hb == 0) xmax[tg * kPsRows + trow] = mx;
      wg_barrier();  // both token groups' maxima visible
      mx = fmaxf(mx, xmax[(tg ^ 1) * kPsRows + trow]);
      float alpha = 1.f;
      if (mx > m_run + kTau) {  // identical decision in both waves of the row group
        alpha = __builtin_amdgcn_exp2f(m_run - mx);
        m_run = mx;
        l_run *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], p.scale_log2, -m_use));
        ps += S[r];
        if (!kFp8 && kSmDma > 0 && has_next && r % 4 == 3) {
          for (int i = kQkDma + (r / 4) * kSmDma / 4; i < kQkDma + (r / 4 + 1) * kSmDma / 4; ++i)
            dma_piece(ndst, nrsrc, ndma, i);
        }
      }
      l_run += half_sum(ps);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2_t v = {pack_bf16(S[4 * j], S[4 * j + 1]), pack_bf16(S[4 * j + 2], S[4 * j + 3])};
        *(LDS_AS u32x2_t*)(pbuf + pbuf_off(trow, 4 * tg + j) + hb * 8) = v;
      }
      if (tg == 0 && hb == 0) abuf[trow] = alpha;
      __builtin_amdgcn_sched_barrier(0);
      wg_barrier();  // P and alpha visible

      // ---- O^T[128 dims x 64 rows] += V^T . P^T over the page's 64 tokens
      {
        const float a0 = abuf[l32], a1 = abuf[32 + l32];
        if (__builtin_amdgcn_ballot_w64(a0 != 1.f || a1 != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            O[dt][0] *= a0;
            O[dt][1] *= a1;
          }
        }
      }
      if constexpr (kFp8) {
        // FP8 pages: V^T through the 8-bit transposed read, dequantised without
        // scale; wave w's 128 dims are exactly latent group w, so each token's
        // group-w scale multiplies its P^T entries instead.  The operands of
        // k-step ks + 1 are read and converted while the MFMAs of k-step ks run.
        const LDS_AS float* sclw = scl + w * kPage + 8 * hb;
        bf16x8_t bp[4][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bp[ks][0] = *(const LDS_AS bf16x8_t*)(pbuf + paddr[0][ks]);
          bp[ks][1] = *(const LDS_AS bf16x8_t*)(pbuf + paddr[1][ks]);
        }
        i32x2_t vr[2][4];
        f32x4_t sr[2][2];
        auto read_ops = [&](int ks, int slot) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            vr[slot][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_AS i32x2_t*)(page + 16 * ks * kF8RowBytes + 32 * dt + vaddr8));
          sr[slot][0] = *(const LDS_AS f32x4_t*)(sclw + 16 * ks);
          sr[slot][1] = *(const LDS_AS f32x4_t*)(sclw + 16 * ks + 4);
        };
        bf16x8_t va[2][4], bs[2][2];
        auto convert_ops = [&](int ks, int slot) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) va[slot][dt] = cvt8_fp8((unsigned)vr[slot][dt][0], (unsigned)vr[slot][dt][1], 1.0f);
          const float sv[8] = {sr[slot][0][0], sr[slot][0][1], sr[slot][0][2], sr[slot][0][3],
                               sr[slot][1][0], sr[slot][1][1], sr[slot][1][2], sr[slot][1][3]};
          bs[slot][0] = scale8(bp[ks][0], sv);
          bs[slot][1] = scale8(bp[ks][1], sv);
        };
        read_ops(0, 0);
        convert_ops(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int cur = ks & 1;
          if (ks + 1 < 4) read_ops(ks + 1, cur ^ 1);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            O[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cur][dt], bs[cur][0], O[dt][0], 0, 0, 0);
            O[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cur][dt], bs[cur][1], O[dt][1], 0, 0, 0);
          }
          if (ks + 1 < 4) convert_ops(ks + 1, cur ^ 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // operands of k-step ks (16 tokens): P^T for both row tiles and V^T for the
        // four 32-dim tiles; the next k-step's operands load while this one's
        // MFMAs run
        struct PvOps {
          bf16x8_t bp[2];
          bf16x8_t va[4];
        };
        auto load_ops = [&](int ks) {
          PvOps o;
          o.bp[0] = *(const LDS_AS bf16x8_t*)(pbuf + paddr[0][ks]);
          o.bp[1] = *(const LDS_AS bf16x8_t*)(pbuf + paddr[1][ks]);
          const LDS_AS char* vs = page + ks * kSliceBytes;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int go = (dt >> 1) * kGroupBytes;
            const bf16x4_t v0 = lds_tr16(vs + vaddr[0][dt & 1] + go);
            const bf16x4_t v1 = lds_tr16(vs + vaddr[1][dt & 1] + go);
            o.va[dt] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          return o;
        };
        PvOps ops[2];
        ops[0] = load_ops(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks + 1 < 4) {
            ops[(ks + 1) & 1] = load_ops(ks + 1);
          }
          const PvOps& o = ops[ks & 1];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            O[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.va[dt], o.bp[0], O[dt][0], 0, 0, 0);
            O[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.va[dt], o.bp[1], O[dt][1], 0, 0, 0);
          }
          if (has_next) {
            for (int i = kPvDma0 + ks * (kSliceDma - kPvDma0) / 4; i < kPvDma0 + (ks + 1) * (kSliceDma - kPvDma0) / 4;
                 ++i)
              dma_piece(ndst, nrsrc, ndma, i);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- epilogue: (m, l) of both token groups for every row
    if (hb == 0) {
      sbuf[(tg * kPsRows + trow) * 2 + 0] = m_run;
      sbuf[(tg * kPsRows + trow) * 2 + 1] = l_run;
    }
    wg_barrier();  // ... and every wave is done with the page buffers
    const bool split = sr.chunks > 1;
    const long long slot = (long long)(sr.base + sr.ord) * p.h_kv + kvh;
    // Each wave writes its 128 normalised output dims of the 64 rows into its
    // own region of the page buffers as [row][dim], with every row's output
    // offset (elements; -1 for a row that is not stored), and then stores whole
    // row segments: 512 B of fp32 partial per 32 lanes or 256 B of bf16 output
    // per 16 lanes, instead of 16-byte pieces spread over 32 rows.
    LDS_AS float* stg = (LDS_AS float*)(smem + w * kPsStgBytes);
    LDS_AS long long* roff = (LDS_AS long long*)(smem + w * kPsStgBytes + kPsRows * kPsStgStride * 4);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int rl = rt * 32 + l32;
      const int orow = mt * kPsRows + rl;
      const float mrow = sbuf[rl * 2 + 0];  // same reference in both token groups
      const float lrow = sbuf[rl * 2 + 1] + sbuf[(kPsRows + rl) * 2 + 1];
      const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t v = {O[dt][rt][4 * j], O[dt][rt][4 * j + 1], O[dt][rt][4 * j + 2], O[dt][rt][4 * j + 3]};
          *(LDS_AS f32x4_t*)(stg + rl * kPsStgStride + dt * 32 + 8 * j + 4 * hb) = v * inv;
        }
      if (hb == 0) {
        long long off = -1;
        if (orow < p.rows && sr.ok) {
          int os;
          long long oo;
          row_coords(p, b, kvh, orow, os, oo);
          const long long srow = slot * p.rows + orow;
          off = (split ? srow : oo) * kDv;
          if (w == 0) {
            const float l2 = lrow > 0.f ? mrow + __builtin_amdgcn_logf(lrow) : -INFINITY;
            if (split) p.lse_acc[srow] = l2;
            else p.lse[oo] = l2 * kLn2;
          }
        }
        roff[rl] = off;
      }
    }
    // this wave's own LDS writes are visible to its later reads (in order)
    if (split) {
#pragma unroll 8
      for (int i = 0; i < kPsRows / 2; ++i) {
        const int r = 2 * i + (lane >> 5);
        const long long off = roff[r];
        const f32x4_t v = *(const LDS_AS f32x4_t*)(stg + r * kPsStgStride + 4 * (lane & 31));
        if (off >= 0) *(f32x4_t*)(p.o_acc + off + w * 128 + 4 * (lane & 31)) = v;
      }
    } else {
#pragma unroll 8
      for (int i = 0; i < kPsRows / 4; ++i) {
        const int r = 4 * i + (lane >> 4);
        const long long off = roff[r];
        const LDS_AS float* src = stg + r * kPsStgStride + 8 * (lane & 15);
        const f32x4_t v0 = *(const LDS_AS f32x4_t*)src;
        const f32x4_t v1 = *(const LDS_AS f32x4_t*)(src + 4);
        const u32x4_t pk = {pack_bf16(v0[0], v0[1]), pack_bf16(v0[2], v0[3]), pack_bf16(v1[0], v1[1]),
                            pack_bf16(v1[2], v1[3])};
        if (off >= 0) *(u32x4_t*)(p.out + off + w * 128 + 8 * (lane & 15)) = pk;
      }
    }
    wg_barrier();  // sbuf and page buffers are reused by the next sequence
  }
}

template <auto Kernel>
hipError_t launch_one(int lds, const DecodeParams& p, hipStream_t stream) {
  // allow the kernel more than the default 64 KB of dynamic LDS (once per
  // process and kernel: each kernel is its own instantiation)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int grid = p.num_parts * p.m_tiles * p.h_kv;
  hipLaunchKernelGGL(Kernel, dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (tile_rows_for(p.rows) == 16 && !p.sparse) {
    if (p.kv_fp8) return launch_one<decode_tokensplit<true>>(TsLayout<true>::kLds, p, stream);
    return launch_one<decode_tokensplit<false>>(TsLayout<false>::kLds, p, stream);
  }
  if (p.kv_fp8) return launch_one<decode_pairsplit<false, true>>(kPsLds, p, stream);
  if (p.sparse) return launch_one<decode_pairsplit<true, false>>(kPsLds, p, stream);
  return launch_one<decode_pairsplit<false, false>>(kPsLds, p, stream);
}

}  // namespace mla
