// Index math of the gfx950 attention-forward kernel: work decomposition,
// LDS layouts (with XOR swizzles), MFMA operand / accumulator lane mappings
// and global offsets.
//
// Everything here is plain integer arithmetic usable from device code and
// from host code (the host-side layout checker compiles this header with a
// normal C++ compiler and enumerates every access the kernel makes).
//
// Notation follows the pages: a work-group owns one block of query rows
// ("Q tile", Br/BM rows) of one (batch, head) and streams key/value blocks
// ("KV tiles", Bc/BN keys) past it (hotdry.top, "FlashAttention的Triton性能
// 考古学", sections on the v2 loop order and the (cdiv(S, Bc), B*N_h) grid).
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

// ---------------------------------------------------------------- tile sizes
constexpr int kWaves = 4;                   // waves (64 lanes) per work-group
constexpr int kThreads = 64 * kWaves;       // 256
constexpr int kRowsPerWave = 32;            // query rows owned by one wave
constexpr int kBM = kRowsPerWave * kWaves;  // 128 query rows per work-group

// Keys per KV tile. D=128 uses 64 keys (K and V^T tiles of 16 KiB each);
// D=64 uses 128 keys (same 16 KiB) so that the per-tile overhead (row-max
// exchange, rescale test, barrier) is amortised over more scores.
template <int D> struct TileCfg;
template <> struct TileCfg<64> { static constexpr int BN = 128; };
template <> struct TileCfg<128> { static constexpr int BN = 64; };

template <int D> struct Lds {
  static constexpr int BN = TileCfg<D>::BN;
  static constexpr int kRowBytes = D * 2;           // K tile row (one key)
  static constexpr int vRowBytes = BN * 2;          // V^T tile row (one d)
  static constexpr int kBytes = BN * D * 2;         // K tile
  static constexpr int vBytes = BN * D * 2;         // V^T tile
  static constexpr int stageBytes = kBytes + vBytes;
  static constexpr int totalBytes = 2 * stageBytes; // double buffered
  // global -> LDS staging work per thread
  static constexpr int kChunks = BN * D / 8;        // 16-byte chunks of K
  static constexpr int kChunksPerThread = kChunks / kThreads;
  static constexpr int vUnits = (BN / 4) * (D / 8); // 4 keys x 8 d units of V
  static constexpr int vUnitsPerThread = vUnits / kThreads;
  static_assert(kChunks % kThreads == 0, "K staging must divide evenly");
  static_assert(vUnits % kThreads == 0, "V staging must divide evenly");
};

// ------------------------------------------------------- work decomposition
// One work-group per (Q tile, batch*head). Under a causal mask Q tile t needs
// keys [0, (t+1)*BM), so work grows with t; tiles are issued heaviest first
// (longest-processing-time order) so that the short ones fill the tail.
// Consecutive work-group ids take consecutive heads, so with B*H a multiple
// of 8 every Q tile of a head lands on the same XCD (ids are dealt to the 8
// XCDs round-robin) and its K/V stay in that XCD's L2.
FA_HD void block_to_tile(int bid, int BH, int nqt, bool causal, int* qt, int* bh) {
  const int ord = bid / BH;
  *bh = bid - ord * BH;
  *qt = causal ? (nqt - 1 - ord) : ord;
}

FA_HD int num_q_tiles(int S) { return (S + kBM - 1) / kBM; }

// Exclusive upper bound of the keys a work-group's Q tile can see.
FA_HD int tile_kv_end(int qt, int S, bool causal) {
  const int e = causal ? (qt + 1) * kBM : S;
  return e < S ? e : S;
}

// Exclusive upper bound of the keys visible to any row of one wave.
FA_HD int wave_kv_end(int q0w, int S, bool causal) {
  const int e = causal ? q0w + kRowsPerWave : S;
  return e < S ? e : S;
}

// ------------------------------------------------------------- LDS swizzle
// Byte offset of 16-byte chunk c of row r, in a buffer of rows of row_bytes
// (128 or 256). The chunk index is XOR-ed with a function g of the row bits
// b0..b5, chosen for the kernel's access patterns:
//  * operand reads: a wave reads rows 32*blk + row_perm32(lane%32) at one
//    chunk; 16 lanes (one 64-bank cycle) cover rows with b0..b3 free, 8
//    lanes (one 32-bank cycle) rows with b0, b1, b3 free -> g is a bijection
//    of those bits, so reads are conflict-free under either bank model;
//  * V^T staging writes: rows 8*dc + dd with dc (bits b3..b5) varying across
//    lanes -> g also varies with b3..b5 (writes at most 2-way).
// 256-byte rows (16 chunks): g = (b0^b3, b1^b4, b3^b5, b2^b4^b5).
// 128-byte rows (8 chunks, 2 rows per 256-byte line): g = (b0^b1^b5,
// b0^b2^b4, b3).
FA_HD int swz_g256(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
  const int b4 = (r >> 4) & 1, b5 = (r >> 5) & 1;
  return (b0 ^ b3) | ((b1 ^ b4) << 1) | ((b3 ^ b5) << 2) | ((b2 ^ b4 ^ b5) << 3);
}
FA_HD int swz_g128(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
  const int b4 = (r >> 4) & 1, b5 = (r >> 5) & 1;
  return (b0 ^ b1 ^ b5) | ((b0 ^ b2 ^ b4) << 1) | (b3 << 2);
}
FA_HD uint32_t swz(int r, int c, int row_bytes) {
  return row_bytes == 256 ? (uint32_t)(r * 256 + ((c ^ swz_g256(r)) << 4))
                          : (uint32_t)(r * 128 + ((c ^ swz_g128(r)) << 4));
}

// ------------------------------------------------ MFMA lane mappings (32x32)
// v_mfma_f32_32x32x16_{f16,bf16}: operand A row i / operand B column j is
// supplied by lanes i and i+32 (8 consecutive k each, k-half = lane/32);
// accumulator element r of lane l is (row 8*(r/4) + 4*(l/32) + r%4,
// column l%32).
//
// The kernel computes S^T = K Q^T (rows = keys, columns = query rows) so that
// a lane ends up owning one query row, and loads K rows in the order
// row_perm32 (swap of bits 2 and 3) so that accumulator elements 0..7 of a
// lane are 8 consecutive keys and 8..15 the next 8 of its k-half. Those 8
// consecutive keys are exactly the k-run the P.V MFMA needs from that lane,
// so P goes from the S accumulator to the P.V operand without leaving the
// lane.
FA_HD int row_perm32(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Key (within a 32-key block) held in accumulator element r by k-half hh.
FA_HD int acc_key32(int r, int hh) { return 16 * (r >> 3) + 8 * hh + (r & 7); }

// ---------------------------------------------- LDS offsets used by the kernel
// K tile: row = key (0..BN-1), 8-element chunk ch (0..D/8-1).
template <int D> FA_HD uint32_t k_lds(int key, int ch) { return swz(key, ch, Lds<D>::kRowBytes); }
// V^T tile: row = d (0..D-1), 8-key chunk kc8 (0..BN/8-1); byte offset within
// the chunk for 4-key quarter q4 (0 or 1) is 8*q4.
template <int D> FA_HD uint32_t vt_lds(int d, int kc8) {
  return (uint32_t)Lds<D>::kBytes + swz(d, kc8, Lds<D>::vRowBytes);
}

// K staging: chunk index idx -> (key, ch); consecutive threads take
// consecutive 16-byte chunks of the contiguous K tile (coalesced).
template <int D> FA_HD void k_stage_map(int idx, int* key, int* ch) {
  *key = idx / (D / 8);
  *ch = idx % (D / 8);
}
// V staging: unit u -> (kg, dc): keys 4*kg..4*kg+3, d = 8*dc..8*dc+7;
// consecutive threads take consecutive d-chunks of the same 4 rows.
template <int D> FA_HD void v_stage_map(int u, int* kg, int* dc) {
  *kg = u / (D / 8);
  *dc = u % (D / 8);
}

// LDS byte offsets of the kernel's accesses, per lane (lane = 0..63):
// S^T MFMA operand A: K row 32*kb + row_perm32(lane%32), d-chunk 2*j + lane/32.
template <int D> FA_HD uint32_t k_read_off(int kb, int j, int lane) {
  return k_lds<D>(32 * kb + row_perm32(lane & 31), 2 * j + (lane >> 5));
}
// O^T MFMA operand A: V^T row 32*jd + row_perm32(lane%32), keys 16*kc + 8*(lane/32) + 0..7.
template <int D> FA_HD uint32_t vt_read_off(int jd, int kc, int lane) {
  return vt_lds<D>(32 * jd + row_perm32(lane & 31), 2 * kc + (lane >> 5));
}
// K staging store of chunk idx.
template <int D> FA_HD uint32_t k_write_off(int idx) {
  int key, ch;
  k_stage_map<D>(idx, &key, &ch);
  return k_lds<D>(key, ch);
}
// V^T staging store of unit u, row 8*dc + dd: keys 4*kg..4*kg+3 as 8 bytes.
// V[key][d] lands at vt_lds(d, key/8) + 2*(key%8).
template <int D> FA_HD uint32_t vt_write_off(int u, int dd) {
  int kg, dc;
  v_stage_map<D>(u, &kg, &dc);
  return vt_lds<D>(8 * dc + dd, kg >> 1) + 8 * (kg & 1);
}

// ------------------------------------------ global element offsets (per head)
// Q operand fragment j of a lane: row qrow (clamped), d = 16*j + 8*hh + 0..7.
template <int D> FA_HD size_t q_frag_off(int qrow_c, int j, int hh) {
  return (size_t)qrow_c * D + 16 * j + 8 * hh;
}
// 8-element chunk ch of global row `row` of K or V.
template <int D> FA_HD size_t kv_chunk_off(int row, int ch) { return (size_t)row * D + 8 * ch; }
// O store of a lane: row qrow, d = 32*jd + 16*g + 8*hh + 0..7 (accumulator
// elements 8*g .. 8*g+7 of d-block jd).
template <int D> FA_HD size_t o_frag_off(int qrow, int jd, int g, int hh) {
  return (size_t)qrow * D + 32 * jd + 16 * g + 8 * hh;
}

// Global row of key `key` of the tile starting at kv0, clamped into [0, S).
// Rows past the end are masked before use, so any in-range row will do.
FA_HD int kv_row(int kv0, int key, int S) {
  const int r = kv0 + key;
  return r < S ? r : S - 1;
}

}  // namespace fa
