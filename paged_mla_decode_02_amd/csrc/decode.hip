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
// This file holds the kernel for <= 16 query rows per KV head and the dispatch
// over all decode kernels (64-row tiles: decode_qkpv.hip; 128-row tiles:
// decode_wide.hip):
//   decode_tokensplit  (<= 16 query rows per KV head, memory-bound shapes):
//     each of the 4 waves owns 16 tokens of every page and an independent online
//     softmax over them; the 4 states merge at the end of a chunk through LDS.
//     It also runs on the FP8 cache (656-byte rows, see kF8RowBytes): pages
//     stay FP8 in LDS and the MFMA operands are dequantised in registers, K
//     with its per-group scale and V without, the V scale folded into P, and
//     on gathered rows (the token-sparse decode).
#include <type_traits>
#include <utility>

#include "decode_common.h"

namespace mla {
namespace {

// FP8 cache (656-byte rows, see kF8RowBytes).  A 16-token slice moves as 656
// token-major 16-byte chunks: 10 full transfers and one of 16 lanes; lane i of
// transfer k supplies chunk 64k + i, so the LDS image is the slice's rows one
// after the other.  The kernels read their MFMA operands from that image and
// dequantise them in registers.
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


// ---------------------------------------------------------------------------
// <= 16 rows: token-split kernel.
// The part's pages form one stream across its sequences: while a page is
// processed the next one of the stream -- possibly the first page of the next
// sequence -- is on its way into the other LDS buffer, and the next sequence's
// length and page ids load while the current one runs, its queries during the
// current one's epilogue.
// LDS: per wave two 16-token transfer slots + merge statistics; with the FP8
// cache the slots hold FP8 images (2 x 10496 B), too small for a wave's partial
// output, so a third region of 18 KB takes the chunk-end merge.  At a chunk end
// the waves merge their partial outputs through the slot just consumed (bf16)
// or that region (FP8).
template <bool kFp8, bool kSparse = false>
struct TsLayout {
  static constexpr int kSlot = kFp8 ? kF8SliceBytes : kSliceBytes;
  static constexpr int kWave = kFp8 ? 2 * kF8SliceBytes + kSliceBytes : 2 * kSliceBytes;
  static constexpr int kDma = kFp8 ? kF8SliceDma : kSliceDma;  // transfers per slice issue
  static constexpr int kStat = 4 * kWave;                        // [4 waves][16 rows][m, l]
  static constexpr int kOffs = kStat + 4 * 16 * 2 * 4;          // token-sparse: [4 waves][2 pages][16] row offsets
  static constexpr int kLds = kOffs + (kSparse ? 4 * 2 * kSlice * 4 : 0);
};

template <bool kFp8, bool kSparse = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
decode_tokensplit(DecodeParams p) {
  static_assert(!(kSparse && kFp8), "the token-sparse decode reads bf16 rows");
  using Lay = TsLayout<kFp8, kSparse>;
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
  // Token-sparse: a sequence's rows are listed, not paged.  The offsets of the
  // slice of page n of a chunk sit in this wave's LDS slot n & 1: staged two
  // pages ahead, each just before the transfer of the page in between, so the
  // wait that covers a slice also covers the offsets staged before its
  // successor's transfer.  A sequence's first page is requested when the
  // sequence starts, not during its predecessor.
  i32x4_t grsrc = {}, offs_rsrc = {};
  if constexpr (kSparse) {
    grsrc = make_rsrc(p.kcache, p.sp_cache_bytes);
    offs_rsrc = make_rsrc(p.sp_offs, 0xffffffffu);
  }
  LDS_AS char* offs_slot = smem + Lay::kOffs + w * 2 * kSlice * 4;
  const auto slice_valid = [&](const SeqRange& r, int blk_) {
    return min(max(r.L - blk_ * kPage - w * kSlice, 0), kSlice);
  };
  int row0 = 0;  // token-sparse: the current sequence's first entry in the offset list
  auto sparse_start = [&](LDS_AS char* dst, int bq, const SeqRange& r) {
    row0 = ((const CONST_AS int32_t*)p.sp_rowptr)[bq];
    stage_offs(offs_slot, offs_rsrc, row0, r.lo, w, lane);
    if (r.lo + 1 < r.hi) stage_offs(offs_slot + kSlice * 4, offs_rsrc, row0, r.lo + 1, w, lane);
    wait_vmcnt<0>();
    dma_slice(dst, grsrc, gathered_dma(offs_slot, slice_valid(r, r.lo), kvh, lane));
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
  if (sr.lo < sr.hi) {
    if constexpr (kSparse) sparse_start(slices, b, sr);
    else issue(slices, ids, 0, sr.lo, sr);
  }
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
      if (kSparse && blk + 1 < sr.hi) {
        const int n0 = blk - sr.lo;
        if (blk + 2 < sr.hi) stage_offs(offs_slot + (n0 & 1) * kSlice * 4, offs_rsrc, row0, blk + 2, w, lane);
        dma_slice(slices + (buf ^ 1) * Lay::kSlot, grsrc,
                  gathered_dma(offs_slot + ((n0 + 1) & 1) * kSlice * 4, slice_valid(sr, blk + 1), kvh, lane));
        wait_vmcnt<Lay::kDma>();
      } else if (blk + 1 < sr.hi) {
        const int k = (blk + 1 - sr.lo) & 63;
        if (k == 0) ids = load_page_ids(p, b, blk + 1, lane);
        issue(slices + (buf ^ 1) * Lay::kSlot, ids, k, blk + 1, sr);
        wait_vmcnt<Lay::kDma>();
      } else if (!kSparse && has_next && nr.lo < nr.hi) {
        issue(slices + (buf ^ 1) * Lay::kSlot, nids, 0, nr.lo, nr);
        next_started = true;
        wait_vmcnt<Lay::kDma>();
      } else {
        wait_vmcnt<0>();
      }
      const LDS_AS char* reg = slices + buf * Lay::kSlot;

      // S^T[16 tokens x 16 rows] = K_slice . Q^T ; A-operand row = token r16,
      // chunk 4*ks + grp = group ks/2, position 4*(ks&1) + grp.  Three
      // accumulation chains; K operands are read kAhead k-steps ahead.
      f32x4_t S;
      if constexpr (kFp8) {
        // FP8 rows, read where they landed (token-major, 656 bytes): a latent
        // k-step is 8 e4m3 codes of token r16, converted with the token's
        // scale of that 128-dim group (exact: powers of two); rope k-steps are
        // bf16 already.  Raw operands are read kAhead k-steps ahead and
        // converted just before their MFMA.
        const LDS_AS char* krow = reg + r16 * kF8RowBytes;
        const f32x4_t ksc = *(const LDS_AS f32x4_t*)(krow + kLatent);
        auto kraw = [&](int n) {
          if (n < 16) {
            const u32x2_t v = *(const LDS_AS u32x2_t*)(krow + 32 * n + 8 * grp);
            return u32x4_t{v[0], v[1], 0u, 0u};
          }
          return *(const LDS_AS u32x4_t*)(krow + kLatent + 16 + 64 * (n - 16) + 16 * grp);
        };
        constexpr int kAhead = 4;
        f32x4_t Sc[3] = {};
        u32x4_t kr[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) kr[i] = kraw(i);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if (ks + kAhead < 18) kr[(ks + kAhead) % (kAhead + 1)] = kraw(ks + kAhead);
          const u32x4_t c = kr[ks % (kAhead + 1)];
          const bf16x8_t ka = ks < 16 ? cvt8_fp8(c[0], c[1], ksc[ks >> 2]) : __builtin_bit_cast(bf16x8_t, c);
          Sc[ks % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[ks], Sc[ks % 3], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100 | 0x002, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        S = Sc[0] + Sc[1] + Sc[2];
      } else {
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
      if constexpr (kFp8) {
        // V^T through the 8-bit transposed read: the 16 lanes of a group
        // address tokens 8 (grp >> 1) + (r16 >> 1) at bytes 16 dt + 8 (r16 & 1),
        // so lane r16 receives dim 16 dt + r16 of those 8 tokens, and keeps the
        // four (4 grp .. 4 grp + 3) its MFMA operand holds.  Codes convert
        // without scale; each token's scale of the tile's 128-dim group
        // multiplies its P^T entry instead (powers of two: exact).
        const LDS_AS char* vbase = reg + (8 * (grp >> 1) + (r16 >> 1)) * kF8RowBytes + 8 * (r16 & 1);
        s16x4_t pg[4];
        {
          f32x4_t tsc[4];  // scales of tokens 4 grp + i, all four groups
#pragma unroll
          for (int i = 0; i < 4; ++i) tsc[i] = *(const LDS_AS f32x4_t*)(reg + (4 * grp + i) * kF8RowBytes + kLatent);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2_t v = {pack_bf16(pr[0] * tsc[0][g], pr[1] * tsc[1][g]), pack_bf16(pr[2] * tsc[2][g], pr[3] * tsc[3][g])};
            pg[g] = __builtin_bit_cast(s16x4_t, v);
          }
        }
        constexpr int kVAhead = 8;
        i32x2_t vr[kVAhead + 1];
#pragma unroll
        for (int i = 0; i < kVAhead; ++i)
          vr[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)(vbase + 16 * i));
        __builtin_amdgcn_sched_group_barrier(0x100, kVAhead, 0);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          if (dt + kVAhead < 32) {
            const int n = dt + kVAhead;
            vr[n % (kVAhead + 1)] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)(vbase + 16 * n));
          }
          const i32x2_t c = vr[dt % (kVAhead + 1)];
          const unsigned word = (unsigned)((grp & 1) ? c[1] : c[0]);
          const u32x2_t vb = {cvt_fp8x2(word, 1.0f, false), cvt_fp8x2(word, 1.0f, true)};
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vb), pg[dt >> 3], O[dt], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100 | 0x002, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
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
    // consumed (bf16) or the merge region (FP8)
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
    if (!next_started && sr.lo < sr.hi) {
      if constexpr (kSparse) sparse_start(slices + buf * Lay::kSlot, b, sr);
      else issue(slices + buf * Lay::kSlot, ids, 0, sr.lo, sr);
    }
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
  if (tile_rows_for(p.rows) == 16) {
    if (p.sparse) return launch_one<decode_tokensplit<false, true>>(TsLayout<false, true>::kLds, p, stream);
    if (p.kv_fp8) return launch_one<decode_tokensplit<true>>(TsLayout<true>::kLds, p, stream);
    return launch_one<decode_tokensplit<false>>(TsLayout<false>::kLds, p, stream);
  }
  if (tile_rows_for(p.rows) == 128 && !p.kv_fp8 && !p.sparse) return launch_decode_wide(p, stream);
  // 64-row tiles (any row count on FP8 pages and gathered rows): the split-wave
  // kernel
  DecodeParams q = p;
  q.m_tiles = tiles64_for(p.rows);
  q.xcd_map = (q.m_tiles * q.h_kv > 1 && q.num_parts % 8 == 0) ? 1 : 0;
  return launch_decode_qkpv(q, stream);
}

}  // namespace mla
