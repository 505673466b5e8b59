// Paged MLA decode, 64-row tiles with two kinds of waves: the kernel for 17 to
// 64 query rows per KV head, and for each 64-row tile of more rows (65 to 128
// on bf16 pages; any number on FP8 pages and gathered rows).  Same method as
// decode.hip and decode_wide.hip -- every latent page read from HBM is
// multiplied against all query rows that share its KV head
// ("OpenSourceWeek Day 1 -- Demystifying DeepSeek's FlashMLA",
// deepseekonline.chat, §II.1), the softmax is computed online with a running
// max and sum and equals the textbook result ("FlashMLA inference
// acceleration" notes, dpshk.com, §2.2) -- with the work of a step split
// between the waves by kind rather than by rows or dims:
//
//   * waves 0 and 1 (score waves) own rows 32w .. 32w+31 of the tile: their
//     queries stay in 144 VGPRs; in step h they compute the scores of half
//     page h + 1 (QK^T) and its online softmax, and publish P(h + 1) and the
//     rows' rescale factors through LDS (both double-buffered);
//   * waves 2 and 3 (value waves) own output dims 256(w-2) .. +255 of all 64
//     rows: O^T is 8 x 2 tiles of 32 x 32 fp32, the whole AGPR file, updated
//     only through the inline-assembly MFMAs of decode_common.h; in step h they
//     run PV of half page h and issue every page transfer (one 16-token slice
//     of each half page per wave, spread between the PV MFMAs);
//   * a step is one barrier plus the longer of the two kinds' work, which run
//     at the same time on their own SIMDs.  The 128-row kernel cannot split
//     its waves this way: 128 rows need all four AGPR files for O and all four
//     VGPR files for the queries;
//   * the latent part of a half page lives in one of four LDS slots and its
//     rope part in one of three: in step h the value waves read slot h, the
//     score waves slot h + 1, half page h + 2 is landing and h + 3 is requested
//     into the slots half pages h - 1 (latent) and h (rope) left.
// Page transfers, the slice swizzle and the chunk bookkeeping are those of
// decode_common.h.  The lazy rescale is that of the other kernels with a
// larger threshold (below).
//
// FP8 pages (656-byte rows, kF8RowBytes; decode_qkpv<true>): a half page's 32
// rows move token-major, latent codes, group scales and rope together, into one
// 20.5 KB slot (21 transfers, the value waves taking alternate ones).  The
// score waves read each lane's K row in 16-byte chunks (two k-steps of 8 latent
// codes, the query registers permuted to match), convert them to bf16 with the
// token's group scale, and copy the half page's scales into an LDS table; the
// value waves read V^T with the 8-bit transposed read and convert it without
// scale, and fold each token's scale for the 128-dim group of an MFMA into the
// P^T entries that multiply it (every scale is a power of two: exact).
//
// Gathered rows (the token-sparse decode, decode_qkpv<false, true>): a slice
// of half page h is the 16 cache rows whose byte offsets the caller lists for
// it; a value wave brings its slice's 16 offsets into LDS (one 16-lane
// transfer) a step before it requests the rows, in the same order as the
// slices, so the step's transfer wait covers them too.
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kQRows = 64;                          // query rows of the tile
constexpr int kQHalf = 32;                          // tokens per step
constexpr int kQLatSlice = 8 * kGroupBytes;         // 16 KB: 16 tokens x 512 latent dims
constexpr int kQLatSlot = 2 * kQLatSlice;           // 32 KB per half page
constexpr int kQRopeSlot = 2 * kGroupBytes;         // 4 KB per half page (2 x 16 tokens x 64 dims)
constexpr int kQLat = 0;                            // 4 latent slots
constexpr int kQRope = kQLat + 4 * kQLatSlot;       // 3 rope slots
constexpr int kQPbuf = kQRope + 3 * kQRopeSlot;     // 2 x P [64 rows][32 tokens] bf16
constexpr int kQPBytes = kQRows * kQHalf * 2;
constexpr int kQAbuf = kQPbuf + 2 * kQPBytes;       // 2 x alpha [64] fp32
constexpr int kQLbuf = kQAbuf + 2 * kQRows * 4;     // 1 / l [64] fp32 at the chunk end
constexpr int kQRbuf = kQLbuf + kQRows * 4;         // output row offsets [64] int at the chunk end
constexpr int kQLds = kQRbuf + kQRows * 4;
constexpr int kQStage = 2 * kQLatSlot;              // per value wave: 64 rows x 256 dims fp32 of O
constexpr int kQDma = 2 * (kLatent / 64 + 1);       // transfers per value wave per half page (18)
static_assert(kQLds <= 160 * 1024, "LDS budget");
// Lazy-rescale threshold, log2 units: the running max moves only when a half
// page's maximum exceeds it by more than 2^64.  Rescaling O costs a value wave
// ~770 VALU instructions on its 256 AGPRs, on the step's critical path; with
// 2^8 (the other kernels' threshold) a workload whose keys include 1 % scaled
// outliers rescaled about a fifth of its steps.  P then stays below 2^64 and
// the sums below 2^64 times the key count: far inside the bf16 / fp32
// exponent range.  On FP8 pages P^T is multiplied by power-of-two group scales
// before PV; those products stay finite while 2^64 times the values of V does,
// which the fp32 sums of O need on either kind of page.
constexpr float kQTau = 64.0f;

// FP8 pages: four slots of 32 token-major 656-byte rows, inside the 128 KB the
// chunk-end staging takes; P, alpha, the group-scale tables, 1 / l and the row
// offsets after it.
constexpr int kQF8Slot = kQHalf * kF8RowBytes;                         // 20992
constexpr int kQF8Dma = (kQF8Slot + 1023) / 1024;                      // 21 transfers per half page
constexpr int kQF8LastLanes = (kQF8Slot - 1024 * (kQF8Dma - 1)) / 16;  // the last one moves 32 x 16 B
// four, as on bf16 pages: five to seven (three to five half pages in flight
// instead of two) measured the same, the FP8 steps being bound by the waves'
// work rather than by the page stream
constexpr int kQF8Slots = 4;
template <bool kFp8>
struct QLay {
  static constexpr int kSlot = kFp8 ? kQF8Slot : kQLatSlot;
  // half-page slots: step h reads slots h (PV) and h + 1 (QK^T) and requests
  // half page h + kSlots - 1 into the slot h - 1 left
  static constexpr int kSlots = kFp8 ? kQF8Slots : 4;
  static constexpr int kPbuf = kFp8 ? (kSlots * kQF8Slot > 2 * kQStage ? kSlots * kQF8Slot : 2 * kQStage) : kQPbuf;
  static constexpr int kAbuf = kPbuf + 2 * kQPBytes;
  static constexpr int kSbuf = kAbuf + 2 * kQRows * 4;  // FP8: 2 x scales [4 groups][32 tokens] fp32
  static constexpr int kLbuf = kSbuf + (kFp8 ? 2 * 4 * kQHalf * 4 : 0);
  static constexpr int kRbuf = kLbuf + kQRows * 4;
  static constexpr int kLds = kRbuf + kQRows * 4;
  // gathered rows: 2 value waves x 2 half pages x 16 staged row offsets
  static constexpr int kObuf = kLds;
  static constexpr int kSparseLds = kObuf + 2 * 2 * kSlice * 4;
  // transfers per value wave wk per half page: 18 (bf16); FP8 transfers wk,
  // wk + 2, .. of the 21
  static constexpr int dmas(int wk) { return kFp8 ? (kQF8Dma + 1 - wk) / 2 : kQDma; }
};
static_assert(QLay<false>::kLds == kQLds && QLay<true>::kLds <= 160 * 1024, "LDS budget");

// PV MFMA i of a step (0..31) is followed by transfer dma_at<n>(i) (of the n a
// value wave issues) of the next half page but two, or by none (-1): the
// transfers spread evenly.
template <int N>
__host__ __device__ constexpr int dma_at(int i) {
  for (int g = 0; g < N; ++g)
    if ((32 * g) / N == i) return g;
  return -1;
}

template <bool kFp8, bool kSparse>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
decode_qkpv(DecodeParams p) {
  static_assert(!(kFp8 && kSparse), "the token-sparse decode reads bf16 rows");
  using L = QLay<kFp8>;
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  LDS_AS char* smem = (LDS_AS char*)smem_generic;
  LDS_AS float* lbuf = (LDS_AS float*)(smem + L::kLbuf);
  LDS_AS int* rbuf = (LDS_AS int*)(smem + L::kRbuf);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = w < 2;
  const int wk = w & 1;  // index among the waves of its kind
  int part, mt, kvh;
  map_block(p, part, mt, kvh);
  const int32_t* md = p.tile_md + (long long)part * kMdInts;
  const int i0 = md[0], f0 = md[1], e0 = md[3], ord0 = md[4];
  const int j0 = min(md[2], p.batch - 1);
  if (i0 >= p.batch || i0 < 0) return;

  const int l32 = lane & 31;
  const int hb = lane >> 5;
  const int g16 = lane >> 4;
  const int k16 = lane & 15;
  const int trow = 32 * wk + l32;  // score waves: tile row of this lane
  const int qrow = mt * kQRows + trow;
  const bool qrow_ok = qrow < p.rows;

  // K operand of QK^T (score waves): token l32 of the half page, 8 dims per
  // k-step, addressed as in the 128-row kernel ((base ^ ((ks & 3) << 5)) +
  // (ks / 4) groups; latent k-steps 0..31, rope k-steps 32..35)
  const int kx = slice_off(l32 & 15, hb);
  const int klat = (l32 >> 4) * kQLatSlice + kx;
  const int krope = (l32 >> 4) * kGroupBytes + kx;
  // V^T operand of PV (value waves, transposed read): k-step ks is slice ks,
  // tokens 8 (g16 >> 1) + k16 / 4 (+4 p4); dims 256 wk + 32 dt + 16 (g16 & 1) +
  // 4 (k16 & 3): chunk group 4 wk + dt / 2, the odd dim tile flipping address
  // bit 6
  int vx;
  {
    const int t = 8 * (g16 >> 1) + (k16 >> 2);
    const int pos = 2 * (g16 & 1) + ((k16 & 3) >> 1);
    vx = t * 128 + ((pos ^ swz(t)) << 4) + ((k16 & 1) << 3) + 4 * wk * kGroupBytes;
  }
  // FP8 pages: the score waves read token l32's row; the value waves' 8-bit
  // transposed V^T read of k-step ks, dim tile dt is at 16 ks rows + 32 dt
  // bytes from vx8 (lanes 2k, 2k + 1 of a 16-lane group address token k of 8
  // at +0 / +8 bytes, so lane i receives dim i of 8 consecutive tokens)
  const int frow = l32 * kF8RowBytes;
  const int vx8 = (8 * hb + (k16 >> 1)) * kF8RowBytes + 256 * wk + 16 * (g16 & 1) + 8 * (k16 & 1);
  // P^T operand of PV: row 32 rt + l32, tokens 16 ks + 8 hb .. +7: px ^ (ks << 5)
  const int px = wp_off(l32, hb);
  // P write of the softmax: row trow, tokens 8 j + 4 hb .. +3: (buffer + pwx) ^ (j << 4)
  const int pwx = wp_off(trow, 0) + 8 * hb;

  // transfers (value waves): slice wk of each half page, i.e. tokens 16 wk ..
  // 16 wk + 15 of the first (d0) or second (d1) half of a page
  const SliceDma d0 = slice_dma_offsets(kSlice * wk, kvh, p.h_kv, lane);
  const SliceDma d1 = slice_dma_offsets(kQHalf + kSlice * wk, kvh, p.h_kv, lane);
  // FP8 pages: transfer j of value wave wk is transfer n = wk + 2 j of a half
  // page's 21; lane l supplies slot bytes 1024 n + 16 l, i.e. byte o - 656 t of
  // row t = o / 656 (f8off: first half of a page; the second lies f8half
  // further)
  constexpr int kF8Mine = (kQF8Dma + 1) / 2;
  int f8off[kF8Mine];
  int f8half = 0;
  if constexpr (kFp8) {
#pragma unroll
    for (int j = 0; j < kF8Mine; ++j) {
      const int o = 1024 * (wk + 2 * j) + 16 * lane;
      const int t = min(o / kF8RowBytes, kQHalf - 1);  // lanes past the slot never transfer
      f8off[j] = (t * p.h_kv + kvh) * kF8RowBytes + (o - t * kF8RowBytes);
    }
    f8half = kQHalf * p.h_kv * kF8RowBytes;
  }
  // gathered rows: the offset list and the cache as buffer resources (offsets
  // past the cache, kSparseNone included, read zeros)
  i32x4_t offs_rsrc = {}, grsrc = {};
  if constexpr (kSparse) {
    offs_rsrc = make_rsrc(p.sp_offs, 0xffffffffu);
    grsrc = make_rsrc(p.kcache, p.sp_cache_bytes);
  }

  for (int b = i0; b <= j0; ++b) {
    const SeqRange sr = seq_range(p, b, i0, f0, j0, e0, ord0);
    int s;
    long long qo;
    row_coords(p, b, kvh, qrow_ok ? qrow : 0, s, qo);
    const int nkeys = p.causal ? max(0, sr.L - p.s_q + s + 1) : sr.L;
    const int h0 = 2 * sr.lo;
    const int h1 = min(2 * sr.hi, (sr.L + kQHalf - 1) / kQHalf);

    // One page loop per kind of wave (the same barriers, step for step), so
    // that the score waves' queries and the value waves' O are never live in
    // the same code.
    int ids = kSparse ? 0 : load_page_ids(p, b, sr.lo, lane);
    auto half_rsrc = [&](int h) {
      const int blk = h >> 1;
      return page_rsrc(p, page_id(ids, (blk - sr.lo) & 63), blk, sr.L, kFp8 ? kF8RowBytes : kRowBytes);
    };
    // gathered rows: row0 indexes the sequence's offset list; gd holds the
    // per-lane sources of the slice being requested
    const int row0 = kSparse ? ((const CONST_AS int32_t*)p.sp_rowptr)[b] : 0;
    SliceDma gd = {};
    LDS_AS char* const obuf = smem + L::kObuf + 2 * wk * kSlice * 4;
    // offsets of slice wk of half page hd into its staging slot (hd % 2): none
    // past the chunk's end, so the list is never read beyond it
    auto stage_half = [&](int hd) {
      if (hd < h1) stage_offs(obuf + (hd & 1) * kSlice * 4, offs_rsrc, row0 + kQHalf * hd, 0, wk, lane);
    };
    // the slice's sources from its staged offsets; keys past the sequence read zeros
    auto gather_half = [&](int hd) {
      const int valid = hd < h1 ? min(max(sr.L - kQHalf * hd - kSlice * wk, 0), kSlice) : 0;
      return gathered_dma(obuf + (hd & 1) * kSlice * 4, valid, kvh, lane);
    };
    // transfer i (0..17) of half page h by a value wave: chunk group i / 2
    // (group 8 is the rope part), token half i % 2
    // (FP8 pages: transfer i of the wave's L::dmas(wk) into slot lat)
    auto dma_piece_h = [&](int h, i32x4_t r, int lat, int rope, int i) {
      if constexpr (kFp8) {
        const int n = wk + 2 * i;
        LDS_AS char* dst = smem + lat * kQF8Slot + 1024 * n;
        const int src = f8off[i] + (h & 1) * f8half;
        if (n < kQF8Dma - 1) dma16(dst, r, src);
        else if (lane < kQF8LastLanes) dma16(dst, r, src);
        (void)rope;
      } else {
        const int g = i >> 1, th = i & 1;
        const int vb = kSparse ? gd.vbase[th] + g * 128
                               : ((h & 1) ? (th ? d1.vbase[1] : d1.vbase[0]) : (th ? d0.vbase[1] : d0.vbase[0])) + g * 128;
        if (g < 8) dma16(smem + kQLat + lat * kQLatSlot + wk * kQLatSlice + g * kGroupBytes + th * 1024, r, vb);
        else dma16(smem + kQRope + rope * kQRopeSlot + wk * kGroupBytes + th * 1024, r, vb);
      }
    };
    constexpr int kMaxDma = kFp8 ? kF8Mine : kQDma;
    auto prologue_dma = [&]() {
      if constexpr (kSparse) {
        // offsets of h0 and h0 + 1, then their rows; h0 + 2's offsets go into
        // h0's staging slot once h0's have been read, before h0 + 1's rows
        stage_half(h0);
        stage_half(h0 + 1);
        wait_vmcnt<0>();
        gd = gather_half(h0);
#pragma unroll
        for (int g = 0; g < kQDma; ++g) dma_piece_h(h0, grsrc, 0, 0, g);
        stage_half(h0 + 2);
        gd = gather_half(h0 + 1);
#pragma unroll
        for (int g = 0; g < kQDma; ++g) dma_piece_h(h0 + 1, grsrc, 1, 1, g);
        return;
      }
#pragma unroll
      for (int k = 0; k < L::kSlots - 2; ++k) {
        const i32x4_t r = h0 + k < h1 ? half_rsrc(h0 + k) : make_rsrc(p.kcache, 0u);
#pragma unroll
        for (int g = 0; g < kMaxDma; ++g)
          if (!kFp8 || g < L::dmas(wk)) dma_piece_h(h0 + k, r, k, k, g);
      }
    };
    // the resource of half page hd's transfers: past the chunk's end an empty
    // buffer range (it reads zeros and touches no memory, so every step has the
    // same transfers in flight)
    auto step_rsrc = [&](int hd) {
      i32x4_t dr = make_rsrc(p.kcache, 0u);
      if (hd < h1) {
        if ((((hd >> 1) - sr.lo) & 63) == 0 && (hd & 1) == 0) {
          // the next 64 pages' ids (once per 64 pages); drained here, so the
          // compiler needs no wait for them that would also wait for the page
          // transfers in flight
          ids = load_page_ids(p, b, hd >> 1, lane);
          vm_drain();
        }
        dr = half_rsrc(hd);
      }
      return dr;
    };
    const bool split = sr.chunks > 1;
    const long long slot_base = ((long long)(sr.base + sr.ord) * p.h_kv + kvh) * p.rows;
    // Step h, for h = h0 - 1 .. h1 - 1: the score waves score and softmax half
    // page h + 1; the value waves run PV of half page h (at h0 - 1: P = 0 and
    // alpha = 1 against half page h0's slot, so that no branch surrounds the PV
    // assembly) and request half page h + 3 (past the chunk's end with an empty
    // buffer range: it reads zeros and touches no memory, so every step has the
    // same transfers in flight).  One barrier per step: half page h + 1 (for
    // the score waves) and P(h), alpha(h) (for the value waves) become visible
    // at it, and every wave is done with step h - 1.  Slots of half page h:
    // latent (h - h0) & 3, rope (h - h0) % 3, counted from h0 - 1.
    if (scorer) {
      // queries (B operand, k-step ks = dims 16 ks + 8 hb .. +7), drained
      // with the page ids before any transfer.  Rows past the last one compute
      // on row 0's query and are never stored.
      bf16x8_t qreg[36];
      {
        const bf16x8_t* qp = (const bf16x8_t*)(p.q + qo * kDqk);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks)  // FP8: latent k-step pairs follow the 16-byte code chunks
          qreg[ks] = qp[kFp8 && ks < 32 ? 4 * (ks >> 1) + 2 * hb + (ks & 1) : 2 * ks + hb];
      }
      vm_drain();
      wg_barrier();  // every wave is done with the previous chunk's output staging in the slots
      float m_run = -INFINITY, l_run = 0.f;  // of row trow (lanes l and l ^ 32 agree)
      // S^T [32 tokens x 32 rows] of one half page (score waves)
      auto qk = [&](int lat_off, int rope_off, f32x16_t& S) {
        constexpr int kAhead = 4;  // K operands in flight ahead of their MFMA
        bf16x8_t ka[kAhead + 1];
        const int lb = lat_off + klat, rb = rope_off + krope;
        auto kread = [&](int n) {
          const int a = n < 32 ? (lb ^ ((n & 3) << 5)) + (n >> 2) * kGroupBytes : rb ^ ((n & 3) << 5);
          return *(const LDS_AS bf16x8_t*)(smem + a);
        };
        S = f32x16_t{};
#pragma unroll
        for (int i = 0; i < kAhead; ++i) ka[i] = kread(i);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          if (ks + kAhead < 36) ka[(ks + kAhead) % (kAhead + 1)] = kread(ks + kAhead);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (kAhead + 1)], qreg[ks], S, 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ks + kAhead < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // FP8 pages: 20 reads per lane from token l32's row -- 16 latent chunks of
      // 16 bytes (k-steps 2r and 2r + 1, converted with the token's group
      // scale) and 4 rope k-steps of bf16; score wave 0 copies the row's four
      // group scales into table tb for the value waves
      auto qk8 = [&](int slot_off, int tb, f32x16_t& S) {
        const LDS_AS char* krow = smem + slot_off + frow;
        const f32x4_t sc = *(const LDS_AS f32x4_t*)(krow + kLatent);
        if (wk == 0 && hb == 0) {
          LDS_AS float* tab = (LDS_AS float*)(smem + L::kSbuf + tb * 4 * kQHalf * 4);
#pragma unroll
          for (int g = 0; g < 4; ++g) tab[g * kQHalf + l32] = sc[g];
        }
        auto rd = [&](int r) {
          return *(const LDS_AS u32x4_t*)(krow + (r < 16 ? 32 * r + 16 * hb : kLatent + 16 + 32 * (r - 16) + 16 * hb));
        };
        constexpr int kAheadR = 3;  // operand reads in flight ahead of their MFMAs
        u32x4_t kr[kAheadR + 1];
        S = f32x16_t{};
#pragma unroll
        for (int i = 0; i < kAheadR; ++i) kr[i] = rd(i);
#pragma unroll
        for (int r = 0; r < 20; ++r) {
          if (r + kAheadR < 20) kr[(r + kAheadR) % (kAheadR + 1)] = rd(r + kAheadR);
          const u32x4_t c = kr[r % (kAheadR + 1)];
          if (r < 16) {
            const float s8 = sc[r >> 2];
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt8_fp8(c[0], c[1], s8), qreg[2 * r], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt8_fp8(c[2], c[3], s8), qreg[2 * r + 1], S, 0, 0, 0);
          } else {
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c), qreg[16 + r], S, 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      };

      // online softmax of half page h from its scores S (score waves): lane
      // holds row trow, tokens 8 (r >> 2) + 4 hb + (r & 3) of the half page.
      // The same steps as the 128-row kernel's (masked maximum, rescale
      // decision, exponentials, sums and bf16 packing), run back to back.
      auto softmax = [&](int h, const f32x16_t& S) {
        // only a half page that reaches past a row's last visible key is masked
        // (a wave-uniform branch: whole half pages skip it)
        const bool partial = __builtin_amdgcn_ballot_w64((h + 1) * kQHalf > nkeys) != 0;
        float sx[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sx[r] = S[r];
        if (__builtin_expect(partial, 0)) {
          const int lim = nkeys - h * kQHalf - 4 * hb;  // visible tokens from this lane's first position
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) sx[r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sx[r]);
        const float m = half_max(mx) * p.scale_log2;
        float alpha = 1.f;
        if (m > m_run + kQTau) {  // the reference moves (at the first visible key O and l are 0: alpha stays 1)
          if (m_run != -INFINITY) alpha = __builtin_amdgcn_exp2f(m_run - m);
          m_run = m;
          l_run *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sx[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[r], p.scale_log2, -m_use));
          psum += sx[r];
        }
        const int pw = L::kPbuf + (h & 1) * kQPBytes + pwx;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2_t v = {pack_bf16(sx[4 * j], sx[4 * j + 1]), pack_bf16(sx[4 * j + 2], sx[4 * j + 3])};
          *(LDS_AS u32x2_t*)(smem + (pw ^ (j << 4))) = v;
        }
        l_run += half_sum(psum);
        if (hb == 0) ((LDS_AS float*)(smem + L::kAbuf + (h & 1) * kQRows * 4))[trow] = alpha;
      };

      if (h0 < h1) {
        const int pw = L::kPbuf + ((h0 - 1) & 1) * kQPBytes + pwx;
#pragma unroll
        for (int j = 0; j < 4; ++j) *(LDS_AS u32x2_t*)(smem + (pw ^ (j << 4))) = u32x2_t{0u, 0u};
        if (hb == 0) ((LDS_AS float*)(smem + L::kAbuf + ((h0 - 1) & 1) * kQRows * 4))[trow] = 1.f;
        if constexpr (kFp8) {  // finite scales for the first step's zero P
          if (wk == 0 && hb == 0) {
            LDS_AS float* tab = (LDS_AS float*)(smem + L::kSbuf + ((h0 - 1) & 1) * 4 * kQHalf * 4);
#pragma unroll
            for (int g = 0; g < 4; ++g) tab[g * kQHalf + l32] = 0.f;
          }
        }
      }
      int lat = L::kSlots - 1, rope = 2;
      for (int h = h0 - 1; h0 < h1 && h < h1; ++h) {
        const int lat1 = kFp8 ? (lat + 1 == L::kSlots ? 0 : lat + 1) : (lat + 1) & 3;
        const int rope1 = rope == 2 ? 0 : rope + 1;
        // half page h + 1 landed (the value waves wait for their transfers before it)
        wg_barrier();
        if (h + 1 < h1) {
          f32x16_t S;
          if constexpr (kFp8) qk8(lat1 * kQF8Slot, (h + 1) & 1, S);
          else qk(kQLat + lat1 * kQLatSlot, kQRope + rope1 * kQRopeSlot, S);
          softmax(h + 1, S);
        }
        lat = lat1;
        rope = rope1;
      }
      // chunk end: publish 1 / l and the row's output offset, write lse
      if (hb == 0) {
        lbuf[trow] = l_run > 0.f ? 1.f / l_run : 0.f;
        rbuf[trow] = (qrow_ok && sr.ok) ? (int)(split ? slot_base + qrow : qo) : -1;
        if (qrow_ok && sr.ok) {
          const float l2 = l_run > 0.f ? m_run + __builtin_amdgcn_logf(l_run) : -INFINITY;
          if (split) p.lse_acc[slot_base + qrow] = l2;
          else p.lse[qo] = l2 * kLn2;
        }
      }
      wg_barrier();  // 1 / l and offsets of every row visible
    } else {
      vm_drain();
      wg_barrier();  // every wave is done with the previous chunk's output staging in the slots
      prologue_dma();
      f32x16_t O[8][2];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc_zero(O[dt][rt]);
      // O^T [256 dims x 64 rows] += V^T . P^T over half page h's 32 tokens (value
      // waves); `between(i)` runs after the i-th of its 32 MFMAs
      auto pv = [&](int h, int lat_off, auto&& between) {
        const LDS_AS float* ab = (const LDS_AS float*)(smem + L::kAbuf + (h & 1) * kQRows * 4);
        const float a0 = ab[l32], a1 = ab[32 + l32];
        const int pb = L::kPbuf + (h & 1) * kQPBytes + px;
        const int vb = lat_off + vx;
        // column c: k-step c / 8 (slice), dim tile c % 8
        auto vread = [&](int c) {
          const int ks = c >> 3, dt = c & 7;
          const int off = ks * kQLatSlice + (dt >> 1) * kGroupBytes;
          const bf16x4_t v0 = lds_tr16(smem + (vb ^ ((dt & 1) << 6)) + off);
          const bf16x4_t v1 = lds_tr16(smem + (vb ^ (16 | ((dt & 1) << 6))) + off + 512);
          return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8_t bp[2], va[3];
        va[0] = vread(0);
        va[1] = vread(1);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) bp[rt] = *(const LDS_AS bf16x8_t*)(smem + pb + rt * 32 * 64);
        if (__builtin_amdgcn_ballot_w64(a0 != 1.f || a1 != 1.f)) {
          acc_settle(O[0][0]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            acc_scale(O[dt][0], a0);
            acc_scale(O[dt][1], a1);
          }
          asm volatile("s_nop 3" ::: "memory");
        }
        // the MFMAs are volatile assembly, which LDS reads do not move across:
        // V^T of column c + 2 is requested after the first MFMA of column c, the
        // P^T operands of k-step 1 after the last k-step-0 MFMA that reads them
#pragma unroll
        for (int c = 0; c < 16; ++c) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            pv_mfma(O[c & 7][rt], va[c % 3], bp[rt]);
            if (rt == 0 && c + 2 < 16) va[(c + 2) % 3] = vread(c + 2);
            if (c == 7) bp[rt] = *(const LDS_AS bf16x8_t*)(smem + (pb ^ 32) + rt * 32 * 64);
            between(2 * c + rt);
            __builtin_amdgcn_sched_barrier(0);  // keep the transfer between these two MFMAs
          }
        }
      };

      // FP8 pages: O^T [256 dims x 64 rows] += V^T . P^T over half page h, V^T
      // through the 8-bit transposed read converted without scale; dim tiles
      // 0..3 lie in scale group 2 wk, 4..7 in 2 wk + 1, and multiply P^T
      // entries scaled by their tokens' scales of that group.  Every operand
      // read is issued first; k-step 1's conversions run between k-step 0's
      // MFMAs.
      auto pv8 = [&](int h, int slot_off, auto&& between) {
        const LDS_AS float* ab = (const LDS_AS float*)(smem + L::kAbuf + (h & 1) * kQRows * 4);
        const float a0 = ab[l32], a1 = ab[32 + l32];
        const int pb = L::kPbuf + (h & 1) * kQPBytes + px;
        const LDS_AS float* tab = (const LDS_AS float*)(smem + L::kSbuf + (h & 1) * 4 * kQHalf * 4) + 8 * hb;
        const LDS_AS char* vb = smem + slot_off + vx8;
        i32x2_t vr[2][8];
        bf16x8_t bp[2][2];
        f32x4_t sr[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            vr[ks][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)(vb + 16 * ks * kF8RowBytes + 32 * dt));
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) bp[ks][rt] = *(const LDS_AS bf16x8_t*)(smem + (pb ^ (ks << 5)) + rt * 32 * 64);
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {  // tokens 16 ks + 8 hb .. +7 of group 2 wk + gi
            sr[ks][2 * gi] = *(const LDS_AS f32x4_t*)(tab + (2 * wk + gi) * kQHalf + 16 * ks);
            sr[ks][2 * gi + 1] = *(const LDS_AS f32x4_t*)(tab + (2 * wk + gi) * kQHalf + 16 * ks + 4);
          }
        }
        if (__builtin_amdgcn_ballot_w64(a0 != 1.f || a1 != 1.f)) {
          acc_settle(O[0][0]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            acc_scale(O[dt][0], a0);
            acc_scale(O[dt][1], a1);
          }
          asm volatile("s_nop 3" ::: "memory");
        }
        bf16x8_t va[2][8], bs[2][2][2];  // [k-step][dim tile], [k-step][group][row tile]
        auto convert_v = [&](int ks, int dt) {
          va[ks][dt] = cvt8_fp8((unsigned)vr[ks][dt][0], (unsigned)vr[ks][dt][1], 1.0f);
        };
        auto convert_p = [&](int ks, int gi, int rt) {
          const float sv[8] = {sr[ks][2 * gi][0],     sr[ks][2 * gi][1],     sr[ks][2 * gi][2],
                               sr[ks][2 * gi][3],     sr[ks][2 * gi + 1][0], sr[ks][2 * gi + 1][1],
                               sr[ks][2 * gi + 1][2], sr[ks][2 * gi + 1][3]};
          bs[ks][gi][rt] = scale8(bp[ks][rt], sv);
        };
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) convert_v(0, dt);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) convert_p(0, q4 >> 1, q4 & 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
              pv_mfma(O[dt][rt], va[ks][dt], bs[ks][dt >> 2][rt]);
              between(16 * ks + 2 * dt + rt);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (ks == 0) {
              convert_v(1, dt);
              if (dt < 4) convert_p(1, dt >> 1, dt & 1);
            }
          }
        }
      };

      int lat = L::kSlots - 1, rope = 2;
      for (int h = h0 - 1; h0 < h1 && h < h1; ++h) {
        const int lat1 = kFp8 ? (lat + 1 == L::kSlots ? 0 : lat + 1) : (lat + 1) & 3;
        const int latd = kFp8 ? (lat == 0 ? L::kSlots - 1 : lat - 1) : (lat + 3) & 3;
        const int rope1 = rope == 2 ? 0 : rope + 1;
        // half page h + 1 landed: only the transfers of h + 2 .. h + kSlots - 2
        // may still be in flight
        if constexpr (kFp8) {
          if (wk == 0) wait_vmcnt<(L::kSlots - 3) * L::dmas(0)>();
          else wait_vmcnt<(L::kSlots - 3) * L::dmas(1)>();
        } else {
          wait_vmcnt<kQDma>();
        }
        wg_barrier();
        const int hd = h + L::kSlots - 1;
        i32x4_t dr;
        if constexpr (kSparse) {
          // h + 3's offsets landed with the wait above; h + 4's go into h + 2's slot
          gd = gather_half(hd);
          stage_half(hd + 1);
          dr = grsrc;
        } else {
          dr = step_rsrc(hd);
        }
        auto between = [&](int i) {
          const int g = dma_at<kMaxDma>(i);
          if (g >= 0 && (!kFp8 || g < L::dmas(wk))) dma_piece_h(hd, dr, latd, rope, g);
        };
        if constexpr (kFp8) pv8(h, (h < h0 ? 0 : lat) * kQF8Slot, between);
        else pv(h, kQLat + (h < h0 ? 0 : lat) * kQLatSlot, between);
        lat = lat1;
        rope = rope1;
      }
      // chunk end: normalise the 256 output dims of all 64 rows and store
      // them through LDS (this wave's two latent slots), so that every store
      // writes one whole 1 KB row segment.  Transfers past the chunk's end
      // (empty ranges) write the slots: they land first.
      wait_vmcnt<0>();
      wg_barrier();  // 1 / l and offsets of every row visible; every wave is done with the slots
      // staging row R (= tile row) holds 256 dims, 16-byte chunk c (dims 4c ..
      // 4c + 3) at position c ^ (R & 7); lane base offsets recomputed per chunk
      // (kept out of loop-invariant hoisting), the rest immediates
      int wb[4], rb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wb[j] = kQLat + wk * kQStage + l32 * 1024 + (((2 * j + hb) ^ (l32 & 7)) << 4);
        asm volatile("" : "+v"(wb[j]));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rb[i] = kQLat + wk * kQStage + ((lane ^ i) << 4);
        asm volatile("" : "+v"(rb[i]));
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float inv = lbuf[32 * rt + l32];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x16_t o = acc_out(O[dt][rt]);
#pragma unroll
          for (int j = 0; j < 4; ++j)  // chunk 8 dt + 2 j + hb
            *(LDS_AS f32x4_t*)(smem + wb[j] + rt * 32 * 1024 + dt * 128) =
                f32x4_t{o[4 * j] * inv, o[4 * j + 1] * inv, o[4 * j + 2] * inv, o[4 * j + 3] * inv};
        }
      }
      // row R: every lane stores chunk `lane`; eight rows read before their stores
      auto store_rows = [&](auto split_tag) {
#pragma unroll
        for (int k0 = 0; k0 < kQRows; k0 += 8) {
          f32x4_t v[8];
          int ro[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            v[i] = *(const LDS_AS f32x4_t*)(smem + rb[(k0 + i) & 7] + (k0 + i) * 1024);
            ro[i] = rbuf[k0 + i];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (ro[i] >= 0) {
              const long long d = (long long)ro[i] * kDv + 256 * wk + 4 * lane;
              if constexpr (decltype(split_tag)::value) {
                *(f32x4_t*)(p.o_acc + d) = v[i];
              } else {
                const u32x2_t pk = {pack_bf16(v[i][0], v[i][1]), pack_bf16(v[i][2], v[i][3])};
                *(u32x2_t*)(p.out + d) = pk;
              }
            }
          }
        }
      };
      if (split) store_rows(std::true_type{});
      else store_rows(std::false_type{});
    }
  }
  // transfers past the last chunk's end (empty ranges) may still be in flight:
  // let them land before the workgroup's LDS is released
  wait_vmcnt<0>();
}

template <bool kFp8, bool kSparse>
hipError_t launch_qkpv(const DecodeParams& p, hipStream_t stream) {
  constexpr int lds = kSparse ? QLay<kFp8>::kSparseLds : QLay<kFp8>::kLds;
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)decode_qkpv<kFp8, kSparse>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int grid = p.num_parts * p.m_tiles * p.h_kv;
  hipLaunchKernelGGL((decode_qkpv<kFp8, kSparse>), dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_qkpv(const DecodeParams& p, hipStream_t stream) {
  if (p.sparse) return launch_qkpv<false, true>(p, stream);
  return p.kv_fp8 ? launch_qkpv<true, false>(p, stream) : launch_qkpv<false, false>(p, stream);
}

}  // namespace mla
