// Paged MLA decode, 128-row tiles: the kernel for more than 64 query rows per
// KV head on bf16 pages (the compute-bound shapes: 128 heads, or 64 heads with
// two query tokens).  Same method as decode.hip -- every latent page read from
// HBM is multiplied against all query rows that share its KV head ("OpenSourceWeek
// Day 1 -- Demystifying DeepSeek's FlashMLA", deepseekonline.chat, §II.1), the
// softmax is computed online with a running max and sum and equals the
// textbook result ("FlashMLA inference acceleration" notes, dpshk.com, §2.2) --
// with a decomposition chosen for gfx950's register files and LDS:
//
//   * a workgroup owns 128 rows; in QK^T wave w owns rows 32w .. 32w+31 whole
//     (its queries stay in 144 VGPRs), so a row's maximum and sum never leave
//     its wave: no exchange between waves before the softmax;
//   * in PV wave w owns output dims 128w .. 128w+127 of all 128 rows: O is 256
//     fp32 accumulators per lane, which fill the AGPR file exactly.  The PV
//     MFMAs are inline assembly accumulating in AGPRs, while the compiler's
//     own MFMAs (QK^T) accumulate the scores in VGPRs next to the queries (one
//     function cannot mix the two accumulator files otherwise); O is only ever
//     touched through that assembly, so the compiler cannot spill into it;
//   * the unit of work is a half page (32 tokens).  Step h scores half page
//     h + 1 (QK^T), then runs PV of half page h while the softmax of half page
//     h + 1 is computed between its MFMAs: the softmax's VALU work overlaps
//     matrix work and one workgroup barrier per step suffices (P and the
//     rescale factors are double-buffered);
//   * the latent part of a half page (512 dims, read by QK^T and PV) lives in
//     one of four slots and its rope part (64 dims, read by QK^T only) in one
//     of three: half page h + 3 is requested during step h, two steps ahead of
//     its use, in the slots half pages h - 1 (latent) and h (rope) just left;
//   * V^T is read from the latent slot with the transposed LDS read
//     (ds_read_b64_tr_b16); each V element is read once per 128 rows;
//   * at a chunk's end each wave's O goes through LDS (the latent slots are
//     free then) so that every store writes whole 512-byte row segments.
// Page transfers, the slice swizzle, the lazy rescale (the running max moves
// only when it grows by more than 2^8) and the chunk bookkeeping are those of
// decode.hip (decode_common.h).
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kWRows = 128;                        // query rows of the tile
constexpr int kHalf = 32;                          // tokens per step
constexpr int kLatSlice = 8 * kGroupBytes;         // 16 KB: 16 tokens x 512 latent dims
constexpr int kLatSlot = 2 * kLatSlice;            // 32 KB per half page
constexpr int kRopeSlot = 2 * kGroupBytes;         // 4 KB per half page (2 x 16 tokens x 64 dims)
constexpr int kWLat = 0;                           // 4 latent slots
constexpr int kWRope = kWLat + 4 * kLatSlot;       // 3 rope slots
constexpr int kWPbuf = kWRope + 3 * kRopeSlot;     // 2 x P [128 rows][32 tokens] bf16
constexpr int kWPBytes = kWRows * kHalf * 2;
constexpr int kWAbuf = kWPbuf + 2 * kWPBytes;      // 2 x alpha [128] fp32
constexpr int kWLbuf = kWAbuf + 2 * kWRows * 4;    // 1 / l [128] fp32 at the chunk end
constexpr int kWRbuf = kWLbuf + kWRows * 4;        // output row offsets [128] int at the chunk end
constexpr int kWLds = kWRbuf + kWRows * 4;
constexpr int kWStage = 32 * 1024;                 // per wave: 64 rows x 128 dims fp32 of O (in the latent slots)
constexpr int kWDma = 9;                           // transfers per wave per half page
static_assert(kWLds <= 160 * 1024, "LDS budget");


__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
decode_wide(DecodeParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  LDS_AS char* smem = (LDS_AS char*)smem_generic;
  LDS_AS float* lbuf = (LDS_AS float*)(smem + kWLbuf);
  LDS_AS int* rbuf = (LDS_AS int*)(smem + kWRbuf);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const int trow = 32 * w + l32;  // tile row of this lane in QK^T and the softmax
  const int qrow = mt * kWRows + trow;
  const bool qrow_ok = qrow < p.rows;

  // LDS addresses.  In every operand below the variable chunk index enters
  // only through the swizzle, as an XOR on bits 4-6 of the byte address that
  // no slot, slice or group base touches, so each operand keeps one base and
  // derives the rest per step (four invariant addresses per operand would take
  // registers the queries need).
  // K operand of QK^T: token l32 of the half page (slice l32 / 16), 8 dims per
  // k-step: chunk 2 ks + hb -> group ks / 4, position 2 (ks & 3) + hb, i.e.
  // (base ^ ((ks & 3) << 5)) + (ks / 4) groups.  Latent k-steps 0..31 read the
  // latent slot, rope k-steps 32..35 the rope slot.
  const int kx = slice_off(l32 & 15, hb);
  const int klat = (l32 >> 4) * kLatSlice + kx;
  const int krope = (l32 >> 4) * kGroupBytes + kx;
  // V^T operand of PV (transposed read): k-step ks is slice ks of the half page,
  // tokens 8 (g16 >> 1) + k16 / 4 (+4 p4); dims 128 w + 32 dt + 16 (g16 & 1) + 4 (k16 & 3).
  // Token + 4 flips swizzle bit 0 (address bit 4) and adds 4 rows of 128
  // bytes; the odd dim tile of a group flips position bit 2 (address bit 6).
  int vx;
  {
    const int t = 8 * (g16 >> 1) + (k16 >> 2);
    const int pos = 2 * (g16 & 1) + ((k16 & 3) >> 1);
    vx = t * 128 + ((pos ^ swz(t)) << 4) + ((k16 & 1) << 3) + 2 * w * kGroupBytes;
  }
  // P^T operand of PV: row 32 rt + l32 (the swizzle depends on l32 only),
  // tokens 16 ks + 8 hb .. +7 = chunk 2 ks + hb: px ^ (ks << 5)
  const int px = wp_off(l32, hb);
  // P write of the softmax: row trow, tokens 8 j + 4 hb .. +3 = chunk j, bytes
  // 8 hb: (buffer + pwx) ^ (j << 4)
  const int pwx = wp_off(trow, 0) + 8 * hb;

  // transfers: wave w moves tokens 16 (w >> 1) + 8 (w & 1) .. +7 of each half
  // page (slice w >> 1, token half w & 1): 8 latent chunk groups and the rope group
  // (selects, not a runtime array index: an indexed private array would live in scratch memory)
  const SliceDma d0 = slice_dma_offsets(kSlice * (w >> 1), kvh, p.h_kv, lane);
  const SliceDma d1 = slice_dma_offsets(kHalf + kSlice * (w >> 1), kvh, p.h_kv, lane);
  const int dma_vb0 = (w & 1) ? d0.vbase[1] : d0.vbase[0];
  const int dma_vb1 = (w & 1) ? d1.vbase[1] : d1.vbase[0];
  const int dma_lat = (w >> 1) * kLatSlice + (w & 1) * 1024;
  const int dma_rope = (w >> 1) * kGroupBytes + (w & 1) * 1024;

  for (int b = i0; b <= j0; ++b) {
    const SeqRange sr = seq_range(p, b, i0, f0, j0, e0, ord0);
    int s;
    long long qo;
    row_coords(p, b, kvh, qrow_ok ? qrow : 0, s, qo);
    const int nkeys = p.causal ? max(0, sr.L - p.s_q + s + 1) : sr.L;
    const int h0 = 2 * sr.lo;
    const int h1 = min(2 * sr.hi, (sr.L + kHalf - 1) / kHalf);

    // queries (B operand, k-step ks = dims 16 ks + 8 hb .. +7) and the chunk's
    // page ids, drained before any transfer so that no compiler wait for them
    // can also wait for a page.  Rows past the last one compute on row 0's
    // query and are never stored.
    bf16x8_t qreg[36];
    {
      const bf16x8_t* qp = (const bf16x8_t*)(p.q + qo * kDqk);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) qreg[ks] = qp[2 * ks + hb];
    }
    int ids = load_page_ids(p, b, sr.lo, lane);
    vm_drain();
    wg_barrier();  // every wave is done with the previous chunk's output staging in the slots

    // half page h lives in latent slot (h - h0) & 3 and rope slot (h - h0) % 3;
    // transfer g < 8 of a wave moves latent chunk group g, transfer 8 the rope group
    auto half_rsrc = [&](int h) {
      const int blk = h >> 1;
      return page_rsrc(p, page_id(ids, (blk - sr.lo) & 63), blk, sr.L);
    };
    auto dma_piece_h = [&](int h, i32x4_t r, int lat, int rope, int g) {
      const int vb = ((h & 1) ? dma_vb1 : dma_vb0) + g * 128;
      if (g < 8) dma16(smem + kWLat + lat * kLatSlot + dma_lat + g * kGroupBytes, r, vb);
      else dma16(smem + kWRope + rope * kRopeSlot + dma_rope, r, vb);
    };
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const i32x4_t r = h0 + k < h1 ? half_rsrc(h0 + k) : make_rsrc(p.kcache, 0u);
#pragma unroll
      for (int g = 0; g < kWDma; ++g) dma_piece_h(h0 + k, r, k, k, g);
    }

    f32x16_t O[4][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc_zero(O[dt][rt]);
    float m_run = -INFINITY, l_run = 0.f;  // of row trow (lanes l and l ^ 32 agree)

    // S^T [32 tokens x 32 rows] of one half page; `between(ks)` runs after MFMA
    // ks (it issues the next transfers: kept in the same basic block as the
    // MFMAs, and the MFMA / LDS-read pattern pinned, so they stay interleaved)
    auto qk = [&](int lat_off, int rope_off, f32x16_t& S, auto&& between) {
      constexpr int kAhead = 4;  // K operands in flight ahead of their MFMA
      bf16x8_t ka[kAhead + 1];
      const int lb = lat_off + klat, rb = rope_off + krope;
      auto kread = [&](int n) {
        const int a = n < 32 ? (lb ^ ((n & 3) << 5)) + (n >> 2) * kGroupBytes : rb ^ ((n & 3) << 5);
        return *(const LDS_AS bf16x8_t*)(smem + a);
      };
      // one accumulation chain: dependent 32x32x16 MFMAs issue back to back at full rate
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
        between(ks);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // online softmax of half page h from its scores S (raw dot products): lane
    // holds row trow, tokens 8 (r >> 2) + 4 hb + (r & 3) of the half page.
    // Written as kSoftSteps pieces placed one after each MFMA of PV.  A wave
    // issues about 16 cycles of VALU work under a 32-cycle MFMA, so each piece
    // stays near that: the masked maximum in two halves, then one scaling FMA
    // and the previous element's exponential (a quarter-rate instruction) per
    // piece, then the sums and bf16 packing two elements at a time.
    constexpr int kSoftSteps = 30;
    float sx[16];
    float alpha = 1.f, m_use = 0.f, psum = 0.f, mx = -INFINITY;
    unsigned pk0 = 0u;
    bool partial = false;
    // With live == false (no half page h: the chunk's last PV step) the
    // pieces still run, on zero scores, so the PV loop has no per-element
    // selects; they then write only P and alpha slots that nothing reads and
    // leave the running maximum and sum alone.
    auto soft_step = [&](int h, const f32x16_t& S, int st, bool live) {
      if (st == 0) {
        // only a half page that reaches past a row's last visible key is
        // masked (a wave-uniform branch: whole half pages skip it)
        partial = __builtin_amdgcn_ballot_w64((h + 1) * kHalf > nkeys) != 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sx[r] = S[r];
        if (__builtin_expect(partial, 0)) {
          const int lim = nkeys - h * kHalf - 4 * hb;  // visible tokens from this lane's first position
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) sx[r] = -INFINITY;
        }
      } else if (st <= 2) {
        if (st == 1) mx = -INFINITY;
#pragma unroll
        for (int r = 8 * (st - 1); r < 8 * st; ++r) mx = fmaxf(mx, sx[r]);
      } else if (st == 3) {
        const float m = half_max(mx) * p.scale_log2;
        alpha = 1.f;
        if (live && m > m_run + kTau) {  // the reference moves (at the first visible key O and l are 0: alpha stays 1)
          if (m_run != -INFINITY) alpha = __builtin_amdgcn_exp2f(m_run - m);
          m_run = m;
          l_run *= alpha;
        }
        m_use = (m_run == -INFINITY) ? 0.f : m_run;
        psum = 0.f;
      } else if (st <= 20) {
        const int j = st - 4;
        if (j < 16) sx[j] = __builtin_fmaf(sx[j], p.scale_log2, -m_use);
        if (j >= 1) sx[j - 1] = __builtin_amdgcn_exp2f(sx[j - 1]);
      } else if (st <= 28) {
        const int q = st - 21;
        psum += sx[2 * q];
        psum += sx[2 * q + 1];
        const unsigned pk = pack_bf16(sx[2 * q], sx[2 * q + 1]);
        if (q & 1) {
          const int pw = kWPbuf + (h & 1) * kWPBytes + pwx;
          *(LDS_AS u32x2_t*)(smem + (pw ^ ((q >> 1) << 4))) = u32x2_t{pk0, pk};
        } else {
          pk0 = pk;
        }
      } else {
        const float ps = half_sum(psum);
        if (live) l_run += ps;
        if (hb == 0) ((LDS_AS float*)(smem + kWAbuf + (h & 1) * kWRows * 4))[trow] = alpha;
      }
    };

    // rescale factors of half page h's rows, read early (they are in LDS since
    // the step's barrier) so that PV does not wait for them
    auto read_alpha = [&](int h, float (&a)[4]) {
      const LDS_AS float* ab = (const LDS_AS float*)(smem + kWAbuf + (h & 1) * kWRows * 4);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = ab[32 * rt + l32];
    };
    // O^T [128 dims x 128 rows] += V^T . P^T over half page h's 32 tokens;
    // `between(i)` runs after the i-th of its 32 MFMAs
    auto pv = [&](int h, int lat_off, const float (&a)[4], auto&& between) {
      if (__builtin_amdgcn_ballot_w64(a[0] != 1.f || a[1] != 1.f || a[2] != 1.f || a[3] != 1.f)) {
        acc_settle(O[0][0]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc_scale(O[dt][rt], a[rt]);
        asm volatile("s_nop 3" ::: "memory");
      }
      // The MFMAs are volatile assembly, which LDS reads do not move across, so
      // the reads are pipelined here by hand: V^T of the next (k-step, dim tile)
      // column is requested after the first MFMA of the current one, and the
      // P^T operand of row tile rt for k-step 1 right after its last k-step-0
      // MFMA; no MFMA waits on a read issued just before it.
      const int pb = kWPbuf + (h & 1) * kWPBytes + px;
      const int vb = lat_off + vx;
      auto vread = [&](int c) {
        const int ks = c >> 2, dt = c & 3;
        const int off = ks * kLatSlice + (dt >> 1) * kGroupBytes;
        const bf16x4_t v0 = lds_tr16(smem + (vb ^ ((dt & 1) << 6)) + off);
        const bf16x4_t v1 = lds_tr16(smem + (vb ^ (16 | ((dt & 1) << 6))) + off + 512);
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t bp[4], va[2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) bp[rt] = *(const LDS_AS bf16x8_t*)(smem + pb + rt * 32 * 64);
      va[0] = vread(0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          pv_mfma(O[c & 3][rt], va[c & 1], bp[rt]);
          if (rt == 0 && c < 7) va[(c + 1) & 1] = vread(c + 1);
          if (c == 3) bp[rt] = *(const LDS_AS bf16x8_t*)(smem + (pb ^ 32) + rt * 32 * 64);
          between(4 * c + rt);
          __builtin_amdgcn_sched_barrier(0);  // keep the piece between these two MFMAs
        }
      }
    };

    if (h0 < h1) {
      wait_vmcnt<kWDma>();
      wg_barrier();  // half page h0 visible
      f32x16_t S;
      // half page h0 + 2's transfers, one per four MFMAs of QK^T(h0)
      const i32x4_t r2 = h0 + 2 < h1 ? half_rsrc(h0 + 2) : make_rsrc(p.kcache, 0u);
      qk(kWLat, kWRope, S, [&](int ks) {
        if ((ks & 3) == 0) dma_piece_h(h0 + 2, r2, 2, 2, ks >> 2);
      });
#pragma unroll
      for (int st = 0; st < kSoftSteps; ++st) soft_step(h0, S, st, true);
    }
    int lat = 0, rope = 0;  // slots of half page h
    for (int h = h0; h < h1; ++h) {
      const int lat1 = (lat + 1) & 3, rope1 = rope == 2 ? 0 : rope + 1;
      const bool nxt = h + 1 < h1;
      // half page h + 1 landed: only the transfers of h + 2 (issued a step
      // ago, or the prologue's) may still be in flight
      if (nxt) wait_vmcnt<kWDma>();
      // half page h + 1 visible, P(h) and alpha(h) visible; every wave is done
      // with step h - 1, so latent slot (h - 1) and rope slot (h) are free
      wg_barrier();
      float a[4];
      read_alpha(h, a);
      f32x16_t S = f32x16_t{};
      if (nxt) {
        // half page h + 3's transfers, one per four MFMAs of QK^T(h + 1).  Past
        // the chunk's end they are issued with an empty buffer range (they read
        // zeros, touch no memory, and fill slots nothing reads any more), so
        // every step has the same transfers in flight and the same waits.
        const int hd = h + 3;
        i32x4_t dr = make_rsrc(p.kcache, 0u);
        if (hd < h1) {
          if ((((hd >> 1) - sr.lo) & 63) == 0 && (hd & 1) == 0) {
            // the next 64 pages' ids (once per 64 pages); drained here, so the
            // compiler needs no wait for them -- which would also wait for
            // the page transfers in flight -- on the common path
            ids = load_page_ids(p, b, hd >> 1, lane);
            vm_drain();
          }
          dr = half_rsrc(hd);
        }
        const int latd = (lat + 3) & 3;
        qk(kWLat + lat1 * kLatSlot, kWRope + rope1 * kRopeSlot, S, [&](int ks) {
          if ((ks & 3) == 0) dma_piece_h(hd, dr, latd, rope, ks >> 2);
        });
      }
      // PV(h), with the softmax of half page h + 1 between its MFMAs
      pv(h, kWLat + lat * kLatSlot, a, [&](int i) {
        if (i < kSoftSteps) soft_step(h + 1, S, i, nxt);
      });
      lat = lat1;
      rope = rope1;
    }

    // ---- chunk end: the row owner publishes 1 / l and its row's output offset
    // and writes lse; every wave normalises its 128 output dims of all 128 rows
    // and stores them through its own 32 KB of the latent slots, 64 rows at a
    // time, so that each store writes two whole 512-byte row segments rather
    // than 32-byte pieces of 32 rows
    const bool split = sr.chunks > 1;
    const long long slot_base = ((long long)(sr.base + sr.ord) * p.h_kv + kvh) * p.rows;
    if (hb == 0) {
      lbuf[trow] = l_run > 0.f ? 1.f / l_run : 0.f;
      rbuf[trow] = (qrow_ok && sr.ok) ? (int)(split ? slot_base + qrow : qo) : -1;
      if (qrow_ok && sr.ok) {
        const float l2 = l_run > 0.f ? m_run + __builtin_amdgcn_logf(l_run) : -INFINITY;
        if (split) p.lse_acc[slot_base + qrow] = l2;
        else p.lse[qo] = l2 * kLn2;
      }
    }
    // transfers past the chunk's end (empty ranges) write the slots: they land
    // before the slots hold output
    wait_vmcnt<0>();
    wg_barrier();  // 1 / l and offsets of every row visible; every wave is done with the slots
    // Lane base offsets, recomputed per chunk (kept out of loop-invariant
    // hoisting, which would hold one register per address across the page
    // loop); everything else is an immediate offset.  Staging row R = 32 r2 +
    // l32 holds tile row 64 half + R; its 16-byte chunk c (dims 4c .. 4c + 3 of
    // the wave's 128) sits at position c ^ (R & 7): the 8 rows (or 8 chunks)
    // one LDS pass serves fall on distinct banks.
    int wb[4], rb[4], ob = kWRbuf + 4 * hb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wb[j] = kWLat + w * kWStage + l32 * 512 + (((2 * j + hb) ^ (l32 & 7)) << 4);
      rb[j] = kWLat + w * kWStage + hb * 512 + ((l32 ^ ((2 * j + hb) & 7)) << 4);
      asm volatile("" : "+v"(wb[j]), "+v"(rb[j]));
    }
    asm volatile("" : "+v"(ob));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const int rt = 2 * half + r2;
        const float inv = lbuf[32 * rt + l32];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const f32x16_t o = acc_out(O[dt][rt]);
#pragma unroll
          for (int j = 0; j < 4; ++j)  // chunk 8 dt + 2 j + hb
            *(LDS_AS f32x4_t*)(smem + wb[j] + r2 * 32 * 512 + dt * 128) =
                f32x4_t{o[4 * j] * inv, o[4 * j + 1] * inv, o[4 * j + 2] * inv, o[4 * j + 3] * inv};
        }
      }
      // lanes 0-31 store staging row 2k, lanes 32-63 row 2k + 1: chunk l32
      // each; eight rows' data and offsets are read before their stores
      auto store_half = [&](auto split_tag) {
#pragma unroll
        for (int k0 = 0; k0 < 32; k0 += 8) {
          f32x4_t v[8];
          int ro[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            v[i] = *(const LDS_AS f32x4_t*)(smem + rb[(k0 + i) & 3] + (k0 + i) * 1024);
            ro[i] = *(const LDS_AS int*)(smem + ob + 4 * (64 * half + 2 * (k0 + i)));
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (ro[i] >= 0) {
              const long long d = (long long)ro[i] * kDv + 128 * w + 4 * l32;
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
      if (split) store_half(std::true_type{});
      else store_half(std::false_type{});
    }
  }
  // transfers past the last chunk's end (empty ranges) may still be in flight:
  // let them land before the workgroup's LDS is released
  wait_vmcnt<0>();
}

}  // namespace

hipError_t launch_decode_wide(const DecodeParams& p, hipStream_t stream) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)decode_wide, hipFuncAttributeMaxDynamicSharedMemorySize, kWLds);
  if (attr != hipSuccess) return attr;
  const int grid = p.num_parts * p.m_tiles * p.h_kv;
  hipLaunchKernelGGL(decode_wide, dim3(grid), dim3(kThreads), kWLds, stream, p);
  return hipGetLastError();
}

}  // namespace mla
