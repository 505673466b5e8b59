// Device helpers shared by the decode kernels (decode.hip: the 16-row and
// 64-row kernels; decode_wide.hip: the 128-row kernel): the LDS page layout and
// its swizzle, the HBM -> LDS page transfers, sequence ranges from the split-KV
// metadata, wave reductions.  Everything here is internal to the library.
#pragma once

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
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float wave_sum16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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

// FP8 (e4m3) cache rows, kF8RowBytes: conversions to bf16 MFMA operands.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned cvt_fp8x2(unsigned v, float scale, bool hi_word) {
  // e4m3 -> bf16 with a power-of-two scale (the instruction uses the scale's
  // exponent), exact
  return hi_word ? __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, scale, true))
                 : __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, scale, false));
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
// MLA_SYNC_DEBUG (a separate reference build of the library, never the
// product path): every transfer waits for itself right after it is issued, so
// no page data is ever in flight while the kernel runs on.  Its results must be
// bit-identical to the pipelined build's; a wait miscounted in the pipeline
// would show up as a difference.
#ifdef MLA_SYNC_DEBUG
#define MLA_DMA_TAIL "\n\ts_waitcnt vmcnt(0)"
#else
#define MLA_DMA_TAIL ""
#endif
__device__ __forceinline__ void dma16(LDS_AS char* dst, i32x4_t rsrc, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" MLA_DMA_TAIL
               :
               : "s"((unsigned)(size_t)dst), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
// Token-sparse decode.  A wave's 16-token slice of page blk of sequence b is
// rows sp_offs[sp_rowptr[b] + 64 blk + 16 w + t], t < 16 (byte offsets; the
// array is padded by one page, so a last page's reads stay inside it).  The 16
// offsets move into LDS with one 16-lane transfer (4 bytes per lane), counted
// with the page transfers, and each lane then reads the offsets of its two
// tokens: no registers hold a page's offsets while it is in flight.
__device__ __forceinline__ void dma4(LDS_AS char* dst, i32x4_t rsrc, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" MLA_DMA_TAIL
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

// P tiles of the half-page kernels: row r holds 32 bf16 tokens as 4 chunks of
// 16 bytes; chunk c sits at position c ^ ((r >> 2) & 3), so the 16 rows a
// quarter wave reads with one 16-byte read fall on 16 distinct bank groups.
__device__ __forceinline__ int wp_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// PV accumulation in AGPRs (the 128-row kernel):
// O^T += V^T . P^T as inline assembly accumulating in AGPRs, while the
// compiler's own MFMAs (QK^T) accumulate the scores in VGPRs next to the
// queries.  O is only ever touched through the statements below (all with the
// AGPR operand class, all updating in place), so it keeps the AGPR file and
// the compiler cannot spill into it.  Wait states the compiler cannot see
// inside the assembly are written out: one before each MFMA (a VALU write of
// an operand), 20 before O is read by VALU instructions (an MFMA result), 4
// after O is written by VALU instructions and before an MFMA accumulates on it.
__device__ __forceinline__ void pv_mfma(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_zero(f32x16_t& acc) { asm volatile("s_nop 3" : "=a"(acc) : "0"(f32x16_t{})); }
__device__ __forceinline__ void acc_settle(f32x16_t& acc) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(acc)); }
// acc *= s in place, one element at a time through a VGPR (the caller settles
// the tuple before and waits 4 states after)
__device__ __forceinline__ void acc_scale(f32x16_t& acc, float s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float e = acc[i];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(s));
    acc[i] = e;
  }
}
// O tuple -> VGPRs (after the MFMA result wait)
__device__ __forceinline__ f32x16_t acc_out(f32x16_t& acc) {
  acc_settle(acc);
  f32x16_t t;
  asm volatile("" : "=v"(t) : "0"(acc));
  return t;
}

__device__ __forceinline__ void row_coords(const DecodeParams& p, int b, int kvh, int row, int& s,
                                           long long& qo) {
  s = row / p.group;
  const int h = kvh * p.group + row % p.group;
  qo = ((long long)b * p.s_q + s) * p.h_q + h;  // flat (b, s, h) index
}

}  // namespace
}  // namespace mla
