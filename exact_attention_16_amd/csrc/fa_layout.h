// Index math of the gfx950 attention-forward kernels: work decomposition,
// LDS tile layouts (XOR-swizzled 16-byte chunks), the DMA, MFMA-operand and
// transposed-read lane mappings, and global offsets.
//
// Everything here is plain integer arithmetic usable from device code and
// from host code: the host-side layout checker compiles this header with an
// ordinary C++ compiler and enumerates every access the kernels make.
//
// Notation follows the pages: a work-group owns one block of query rows
// (a "Q tile", Br rows) of one (batch, head) and streams key/value blocks
// ("KV tiles", Bc keys) past it, one work-group per (Q tile, batch*head)
// (hotdry.top, "FlashAttention的Triton性能考古学", section "FlashAttention
// v2：循环重构与寄存器积累": the loop order and the grid).
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

constexpr int kRowsPerWave = 32;  // query rows owned by one wave (one MFMA column block)

// A kernel configuration: head dimension D, NW waves (64 lanes) per
// work-group, BN keys per KV tile, RPW query rows per wave (one or two
// 32-row MFMA column blocks), ES bytes per K/V element. One K or V tile in
// LDS holds BN rows (keys) of D elements, row-major, each row split in
// 16-byte chunks whose order is XOR-swizzled per row.
template <int D_, int NW_, int BN_, int RPW_ = kRowsPerWave, int ES_ = 2> struct Cfg {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int BN = BN_;
  static constexpr int RPW = RPW_;
  static constexpr int ES = ES_;                         // bytes per K/V element
  static constexpr int threads = 64 * NW;
  static constexpr int BM = RPW * NW;                    // query rows per work-group
  static constexpr int rowBytes = D * ES;
  static constexpr int chunks = rowBytes / 16;           // 16-byte chunks per row
  static constexpr int tileBytes = BN * rowBytes;        // one K or V tile
  static constexpr int dmaPerWave = tileBytes / 1024 / NW;  // 1-KiB DMA issues per wave
  static constexpr int rowsPerBlock = 64 / chunks;       // rows filled by one DMA issue
  static constexpr int dmaRowsK = NW * rowsPerBlock;     // source rows between K issues
  static constexpr int dmaRowsV = rowsPerBlock;          // source rows between V issues
  static_assert(tileBytes % (1024 * NW) == 0, "tile must split into whole DMA issues");
  static_assert(BN % 32 == 0, "KV tile must be whole 32-key MFMA blocks");
  static_assert(RPW % kRowsPerWave == 0, "a wave owns whole 32-row blocks");
};

// Two of the kernels' shapes: four waves (128 query rows), each running a
// tile start to end, for grids too small to fill the chip with 256-row
// tiles; eight waves (256 rows) in two groups that alternate MFMA and
// softmax phases (ping-pong). The ping-pong kernel uses 128-key tiles at
// D=64 so that an MFMA phase (32 MFMAs) balances a softmax phase.
template <int D> using Cfg4 = Cfg<D, 4, 64>;
template <int D> using Cfg8 = Cfg<D, 8, (D == 64 ? 128 : 96)>;

// ------------------------------------------------------- work decomposition
// One work-group per (Q tile, batch*head). Work-group ids are dealt to the 8
// XCDs round-robin (XCD = id mod 8), each XCD with its own L2. When B*H is a
// multiple of 8, XCD x takes heads x, x+8, x+16, ... (local heads 0, 1, ...),
// so every head's K/V stays in one L2:
//  * Not causal: all tiles cost the same; the XCD takes its heads one at a
//    time, all Q tiles of a head together.
//  * Causal: Q tile t needs keys [0, (t+1)*BM), so work grows with t. The
//    XCD takes its heads in groups of hg, and within a group the Q tiles in
//    turn over the group's heads, heaviest first (longest-processing-time
//    order), so the short tiles fill the tail. The launcher picks hg:
//    kHeadGroup for sequences of one length, and for a variable-length
//    batch the heads one sequence puts on an XCD, so that sequences of
//    different lengths are not mixed. (Measured on the long causal
//    workload, 4 heads per XCD: groups of 1 took 3% longer than 4. On the
//    variable-length batch, 32 heads per XCD: groups of 4 took 12% and of
//    32 took 15% longer than groups of 2, one sequence.)
// Otherwise ids go to heads in turn, Q tile order outermost (heaviest first
// when causal).
constexpr int kHeadGroup = 4;
FA_HD void block_to_tile(int bid, int BH, int nqt, bool causal, int* qt, int* bh,
                         int hg = kHeadGroup) {
  int ord;
  if ((BH & 7) == 0) {
    const int x = bid & 7, k = bid >> 3;  // XCD, and this id's rank on it
    int lh;                               // local head on the XCD
    if (!causal) {
      lh = k / nqt;
      ord = k - lh * nqt;
    } else {
      const int hx = BH >> 3;                  // heads on this XCD
      const int g = k / (hg * nqt);            // head group
      const int h0 = g * hg;
      const int gn = hx - h0 < hg ? hx - h0 : hg;  // heads in it
      const int r = k - h0 * nqt;              // rank within the group
      ord = r / gn;
      lh = h0 + (r - ord * gn);
    }
    *bh = x + 8 * lh;
  } else {
    ord = bid / BH;
    *bh = bid - ord * BH;
  }
  *qt = causal ? (nqt - 1 - ord) : ord;
}

// ceil(S / BM) for S >= 0, without forming S + BM - 1 (which overflows int
// for S near INT_MAX)
FA_HD int num_q_tiles(int S, int BM) { return S / BM + (S % BM != 0); }

// Variable lengths: a launch sized for the longest sequence gives every
// shorter one query tiles that lie wholly past its end (work-groups that only
// start and return). For batches of at most kCompactMaxSeqs sequences the
// launch runs only the tiles within each sequence. The lengths are on the
// device, so the launch takes the bound below and each work-group finds its
// item from the offsets (RowState::locate). With offsets that never
// decrease, sequence b has L_b <= its token count query rows, the counts sum
// to at most totq, and the sum of ceil(L_b / BM) is at most
// floor((totq + B*(BM-1)) / BM); never more than the B * nqt of the full grid.
constexpr int kCompactMaxSeqs = 256;  // one pass of a 64-lane scan, 4 per lane
FA_HD long long varlen_cap(int totq, int B, int nqt, int BM) {
  const long long full = (long long)B * nqt;
  const long long cap = ((long long)totq + (long long)B * (BM - 1)) / BM;
  return cap < full ? cap : full;
}
// Item order of a compacted launch. With H a multiple of 8, work-group id
// runs on XCD x = id mod 8 and takes rank k = id / 8 there, over the m = H/8
// heads x, x+8, ... of each sequence (the heads one sequence puts on an XCD);
// otherwise x = 0, k = id, over all m = H heads. Ranks run over the
// sequences in order, m * nt_b ranks for sequence b with nt_b query tiles.
// Within a sequence (rank r): causal, heaviest tile first with the m heads
// in turn; else one head at a time. Returns the tile and the head index j
// among the m (head x + 8j, or j).
FA_HD void varlen_tile(int r, int m, int nt, bool causal, int* qt, int* j) {
  if (causal) {
    const int ord = r / m;
    *j = r - ord * m;
    *qt = nt - 1 - ord;
  } else {
    *j = r / nt;
    *qt = r - *j * nt;
  }
}

// Work item of a persistent work-group b (of G, a multiple of 8) at round k:
// a snake over the ranks of its XCD (see pp_persistent); -1 past the last.
FA_HD int persistent_item(int b, int G, int k, int total) {
  const int x = b & 7, c = b >> 3, cg = G >> 3;
  const int r = k * cg + ((k & 1) ? cg - 1 - c : c);
  const long long id = 8LL * r + x;
  return id < total ? (int)id : -1;
}

// Causal masks are aligned bottom-right: with Lq queries and Lk keys, query i
// sees keys j <= i + (Lk - Lq). With Lq == Lk that is j <= i.
FA_HD int clamp_keys(int e, int Lk) { return e < 0 ? 0 : (e < Lk ? e : Lk); }

// Exclusive upper bound of the keys a work-group's Q tile can see.
FA_HD int tile_kv_end(int qt, int Lq, int Lk, bool causal, int BM) {
  return causal ? clamp_keys((qt + 1) * BM + (Lk - Lq), Lk) : Lk;
}

// Exclusive upper bound of the keys visible to any row of one wave.
FA_HD int wave_kv_end(int q0w, int Lq, int Lk, bool causal) {
  return causal ? clamp_keys(q0w + kRowsPerWave + (Lk - Lq), Lk) : Lk;
}

// Leading KV tiles of BN keys that need no index compares for a wave whose
// first row is q0w: tiles whose last key that row sees (causal) and that end
// before the last key.
FA_HD int unmasked_tiles(int q0w, int Lq, int Lk, bool causal, int BN) {
  const int r = Lk / BN;
  const int e = q0w + (Lk - Lq) + 1;  // keys visible to row q0w
  const int d = e < 0 ? 0 : e / BN;
  return causal ? (d < r ? d : r) : r;
}

// --------------------------------------------------------- LDS swizzles
// Byte offset of logical 16-byte chunk c of row r = r*rowBytes + (c ^ g(r))*16.
//
// K tile (rows = keys): the S^T MFMA operand read has 16 lanes of one
// 64-bank cycle read rows {0..15} (+ a multiple of 16) at one chunk, and 8
// lanes of one 32-bank cycle rows {0..3, 8..11}; g is a bijection of the
// row bits those lanes vary, so either bank model sees no conflict.
//   D=128 (256-byte rows): g = row bits (b0, b1, b3, b2)  [swap of b2, b3]
//   D=64  (128-byte rows, two per 256 bytes): g = (b0^b1, b0^b2, b3)
template <int D> FA_HD int gk(int r);
template <> FA_HD int gk<128>(int r) { return (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1); }
template <> FA_HD int gk<64>(int r) {
  return ((r ^ (r >> 1)) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r >> 3) & 1) << 2);
}
// V tile (rows = keys): the transposed read has the 32 lanes of one cycle
// read 4 consecutive rows x 64 bytes; g moves each of the 4 rows to its own
// 64-byte quarter of the bank space.
//   D=128: g = 4*(r mod 4);  D=64: g = 4*((r/2) mod 2)
template <int D> FA_HD int gv(int r);
template <> FA_HD int gv<128>(int r) { return 4 * (r & 3); }
template <> FA_HD int gv<64>(int r) { return 4 * ((r >> 1) & 1); }

template <int D> FA_HD uint32_t k_off(int r, int c) {
  return (uint32_t)(r * D * 2 + ((c ^ gk<D>(r)) << 4));
}
template <int D> FA_HD uint32_t v_off(int r, int c) {
  return (uint32_t)(r * D * 2 + ((c ^ gv<D>(r)) << 4));
}

// ------------------------------------------------ global -> LDS DMA (16 B)
// A buffer load with the LDS bit writes lane p's 16 bytes to LDS base + 16*p,
// so each DMA issue fills one 1-KiB block of the tile. Lane p fetches the
// logical chunk that belongs at its LDS slot; dma_src_* return that chunk's
// byte offset within the (contiguous) global tile.
// Source rows are rs bytes apart (rowBytes for dense rows, more for strided
// layouts).
// K: issue i of wave w fills block i*NW + w, so successive issues are NW
// blocks (a multiple of 16 rows) apart and gk, which reads row bits 0..3,
// repeats: the source offset of issue i is issue 0's plus i*dmaRowsK*rs.
// V: issue i of wave w fills block w*dmaPerWave + i; gv reads row bits 0..1
// only, so issue i is issue 0's plus i*dmaRowsV*rs.
template <class C> FA_HD int dma_block_k(int w, int i) { return i * C::NW + w; }
template <class C> FA_HD int dma_block_v(int w, int i) { return w * C::dmaPerWave + i; }
template <class C> FA_HD void dma_slot(int block, int lane, int* r, int* pc) {
  const int idx = block * 64 + lane;
  *r = idx / C::chunks;
  *pc = idx % C::chunks;
}
template <class C> FA_HD uint32_t dma_src_k(int w, int i, int lane, uint32_t rs = C::rowBytes) {
  int r, pc;
  dma_slot<C>(dma_block_k<C>(w, i), lane, &r, &pc);
  return (uint32_t)r * rs + (uint32_t)((pc ^ gk<C::D>(r)) << 4);
}
template <class C> FA_HD uint32_t dma_src_v(int w, int i, int lane, uint32_t rs = C::rowBytes) {
  int r, pc;
  dma_slot<C>(dma_block_v<C>(w, i), lane, &r, &pc);
  return (uint32_t)r * rs + (uint32_t)((pc ^ gv<C::D>(r)) << 4);
}
template <class C> FA_HD uint32_t dma_lds_k(int w, int i) { return (uint32_t)dma_block_k<C>(w, i) * 1024u; }
template <class C> FA_HD uint32_t dma_lds_v(int w, int i) { return (uint32_t)dma_block_v<C>(w, i) * 1024u; }

// ------------------------------------------------ MFMA lane mappings (32x32)
// v_mfma_f32_32x32x16_{f16,bf16}: operand A row i / operand B column j is
// supplied by lanes i and i+32 (8 consecutive k each, k-half = lane/32);
// accumulator element r of lane l is (row 8*(r/4) + 4*(l/32) + r%4,
// column l%32).
//
// The kernels compute S^T = K Q^T (rows = keys, columns = query rows) so
// that a lane owns one query row, and feed K rows in the order row_perm32
// (swap of bits 2 and 3) so that accumulator elements 0..7 of a lane are 8
// consecutive keys and 8..15 the next 8 of its k-half. Those 8 consecutive
// keys are exactly the k-run the P.V MFMA needs from that lane, so P goes
// from the S accumulator to the P.V operand without leaving the lane.
FA_HD int row_perm32(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Key (within a 32-key block) held in accumulator element r by k-half hh.
FA_HD int acc_key32(int r, int hh) { return 16 * (r >> 3) + 8 * hh + (r & 7); }

// S^T operand A of contraction step j (d = 16j..16j+15) for 32-key block kb:
// lane reads K row 32*kb + row_perm32(lane%32), chunk 2j + lane/32.
// gk depends only on row bits 0..3, so kb adds exactly kb*32*rowBytes; and
// (2j + hh) ^ g = 2(j ^ g/2) + ((hh ^ g) & 1) with the row base a multiple
// of 128, so step j's offset is step 0's XOR (j << 5).
template <int D> FA_HD uint32_t k_read_off(int kb, int j, int lane) {
  return k_off<D>(32 * kb + row_perm32(lane & 31), 2 * j + (lane >> 5));
}

// O^T operand A (V^T) of d-block jd and 16-key chunk kc, read with
// ds_read_b64_tr_b16 in two halves rd = 0, 1 (keys 16kc + 8h + 4rd + 0..3).
// The instruction works on groups of 16 lanes: source lane s of a group
// reads 4 consecutive 16-bit elements, and result lane i receives element
// i%4 of source lanes i/4, i/4+4, i/4+8, i/4+12. Source lane s = 4e + q of
// group (h = lane/32, g2 = lane/16 % 2) reads key row 16kc + 8h + 4rd + e at
// d = 32jd + 16g2 + 8(q%2) + 4(q/2) .. +3, so result lane i = 4q' + c' holds
// V[16kc + 8h + 4rd + e][32jd + row_perm32(16g2 + i)] for e = 0..3: the
// MFMA row of lane l is d = 32jd + row_perm32(l%32) with keys 8h + 4rd + e.
// gv depends only on row bits 0..1, so kc and rd add kc*16*rowBytes and
// rd*4*rowBytes; gv only flips chunk bits 2..3, where jd sits, so block jd's
// offset is block 0's XOR (jd << 6).
template <int D> FA_HD uint32_t v_tr_off(int jd, int kc, int rd, int lane) {
  const int i = lane & 15, g2 = (lane >> 4) & 1, h = lane >> 5;
  const int row = 16 * kc + 8 * h + 4 * rd + (i >> 2);
  const int c = 4 * jd + 2 * g2 + (i & 1);
  return v_off<D>(row, c) + 8 * ((i >> 1) & 1);
}

// ------------------------------------------ global byte offsets (per head)
// Q operand fragment j of a lane: row qrow, d = 16*j + 8*hh + 0..7.
template <int D> FA_HD uint32_t q_frag_off(int qrow, int j, int hh, uint32_t rs = D * 2) {
  return (uint32_t)qrow * rs + (uint32_t)((16 * j + 8 * hh) * 2);
}
// O store of a lane: row qrow, d = 32*jd + 16*g + 8*hh + 0..7 (accumulator
// elements 8*g .. 8*g+7 of d-block jd).
template <int D> FA_HD uint32_t o_frag_off(int qrow, int jd, int g, int hh, uint32_t rs = D * 2) {
  return (uint32_t)qrow * rs + (uint32_t)((32 * jd + 16 * g + 8 * hh) * 2);
}

// ------------------------------------- ping-pong schedule (eight waves)
// Waves 0-3 (group A) and 4-7 (group B) share the four SIMDs one each (wave
// w and w+4 land on the same SIMD). Each wave runs steps j = 0..ntiles: an
// MFMA phase (O += P(j-1) V(j-1), S(j) = K(j) Q^T), then the softmax phase of
// S(j). Group B runs half a step behind group A, so that on each SIMD one wave
// multiplies while the other exponentiates. KV tile t lives in LDS stage
// t mod kStages for both K and V. DMA pair i carries K(i+2) and V(i+1); each
// wave issues its share of it in step i (group A before its MFMA phase, group
// B after the softmax phase of step i-1). Work-group barriers divide time in
// slots, and at the end of every slot each wave waits for all its DMA but the
// latest pair. Two forms:
//  * two barriers per step: slot t of a wave runs its phase t - group (phase
//    2j: MFMA phase of step j, 2j+1: its softmax phase), so the phases of the
//    two groups are pinned to each other. Pair i is issued in slot 2i and has
//    landed by the end of slot 2i+2: K(j) and V(j-1), both of pair j-2, are
//    in place from slot 2j-1 on. Pair i overwrites K(i-1) and V(i-2), both
//    last read (by group B) in slot 2i-1.
//  * one barrier per step: slot e holds group A's step e and group B's
//    softmax phase of step e-1 and MFMA phase of step e; within a slot the
//    phases alternate without being pinned. Pair i is issued in slot i and
//    has landed by the end of slot i+1: K(j) and V(j-1) are in place from
//    slot j on. Pair i overwrites K(i-1) and V(i-2), last read in slot i-1.
// At D = 128 the second barrier costs more than the drift it prevents; at
// D = 64 the softmax phase is as long as the MFMA phase and the pinned form
// keeps the two groups from exponentiating at the same time.
constexpr int kStages = 3;
template <int D> constexpr bool pp_one_barrier = (D == 128);
// barriers after the prologue's
FA_HD int pp_slots(int ntiles, bool one_barrier) {
  return one_barrier ? ntiles + 1 : 2 * ntiles + 3;
}

}  // namespace fa
