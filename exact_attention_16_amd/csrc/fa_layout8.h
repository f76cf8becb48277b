// Index math of the 8-bit (E4M3) attention-forward kernel: LDS tile
// swizzles, the DMA source offsets, the MFMA operand and transposed-read
// lane mappings and the global offsets of Q and O. The work decomposition,
// the causal alignment and the ping-pong schedule are those of fa_layout.h.
//
// Plain integer arithmetic usable from device and host code (the host-side
// layout checker enumerates every access with these functions).
#pragma once
#include "fa_layout.h"

namespace fa {

// Eight waves of 32 query rows (256 rows), head dimension 128 of one-byte
// elements: 128-byte rows, eight 16-byte chunks per row. 128-key tiles
// (16 KiB per K or V tile), and 64-key tiles for the interleaved kernel.
using CfgF8 = Cfg<128, 8, 128, kRowsPerWave, 1>;
using CfgF8i = Cfg<128, 8, 64, kRowsPerWave, 1>;
// Head dimension 64: 64-byte rows, four chunks; 128-key tiles (8 KiB).
using CfgF8h = Cfg<64, 8, 128, kRowsPerWave, 1>;

// ------------------------------------------------ MFMA lane mappings
// v_mfma_f32_32x32x64_f8f6f4 (both operands E4M3): operand A row i / operand
// B column j is supplied by lanes i and i+32, 32 consecutive k each (k-half
// = lane/32, bytes 0..31 of the lane's eight registers); accumulator
// element r of lane l is (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
//
// S^T = K Q^T: a KV tile is two 64-key chunks c, each computed as two
// 32-row MFMA blocks b (block kb = 2c + b). MFMA row r of block kb reads key
// 64c + 32*((r/4) % 2) + 16b + 4*(r/8) + r%4. With that order accumulator
// element r of k-half hh holds key 64c + 32hh + 16b + r: the 32 values a
// lane holds for chunk c are 32 consecutive keys, exactly the k-run the P.V
// MFMA takes from that lane for chunk c, so P goes from the S accumulators
// to the P.V operand without leaving the lane.
FA_HD int k8_key(int kb, int r) {
  return 64 * (kb >> 1) + 32 * ((r >> 2) & 1) + 16 * (kb & 1) + 4 * (r >> 3) + (r & 3);
}
// key (within the tile) of accumulator element r of k-half hh in block kb
FA_HD int acc_key8(int kb, int r, int hh) { return 64 * (kb >> 1) + 32 * hh + 16 * (kb & 1) + r; }

// --------------------------------------------------------- LDS swizzles
// Byte offset of logical 16-byte chunk c of row r = r*D + (c ^ g(r))*16.
//
// D = 128:
// K: the 16 lanes of one 64-bank cycle of an operand read take MFMA rows
// 0..15 (or 16..31) at one chunk, i.e. keys {0..7, 32..39} (+8, +16 or +48);
// even and odd rows fall in different halves of the bank space, so g must
// map key bits 1, 2, 5 one-to-one onto the eight chunk positions for either
// value of bit 0. Under a 32-bank model the 8 lanes of a cycle take keys
// {0..3, 32..35} (+4, ...), so g must also be one-to-one in bits 0, 1, 5 for
// either value of bit 2. g = (b0 ^ b2, b1, b5) is both.
template <int D> FA_HD int gk8(int r);
template <> FA_HD int gk8<128>(int r) { return ((r ^ (r >> 2)) & 1) | (r & 2) | (((r >> 5) & 1) << 2); }
// V: the 32 lanes of one cycle of a transposed read take 8 consecutive keys
// at two neighbouring chunks (2jd, 2jd+1); g = 2*(key bits 1..2) sends the
// four keys of each parity to four different chunk pairs.
template <int D> FA_HD int gv8(int r);
template <> FA_HD int gv8<128>(int r) { return 2 * ((r >> 1) & 3); }
// D = 64 (four rows per 256 bytes, four chunks per row):
// K: the 16 lanes of a 64-bank cycle take keys {0..7, 32..39}: row bits 0-1
// pick the quarter of the bank space, so g must be one-to-one in bits 2 and
// 5 for each value of bits 0-1; the 8 lanes of a 32-bank cycle take keys
// {0..3, 32..35}: bit 0 picks the half, so g must be one-to-one in bits 1
// and 5 for each value of bit 0. g = (b1 ^ b2, b5) is both.
template <> FA_HD int gk8<64>(int r) { return ((r ^ (r >> 1)) >> 1 & 1) | (((r >> 5) & 1) << 1); }
// V: the 32 lanes of a transposed-read cycle take 8 consecutive keys at two
// neighbouring chunks; rows r and r+4 share a quarter of the bank space, so
// g = 2*(key bit 2) moves the second of them to the other chunk pair.
template <> FA_HD int gv8<64>(int r) { return 2 * ((r >> 2) & 1); }

template <int D = 128> FA_HD uint32_t k8_off(int r, int c) {
  return (uint32_t)(r * D + ((c ^ gk8<D>(r)) << 4));
}
template <int D = 128> FA_HD uint32_t v8_off(int r, int c) {
  return (uint32_t)(r * D + ((c ^ gv8<D>(r)) << 4));
}

// ------------------------------------------------ global -> LDS DMA (16 B)
// As for 16-bit tiles (fa_layout.h): issue i of wave w fills one 1-KiB block
// (8 rows at D = 128, 16 at D = 64). K issues are NW blocks (64 or 128 rows)
// apart and gk8 reads row bits 0, 1, 2 and 5 only; V issues are one block
// apart and gv8 reads row bits 1, 2 only: issue i's source offset is issue
// 0's plus i rows strides.
template <class C = CfgF8>
FA_HD uint32_t dma_src_k8(int w, int i, int lane, uint32_t rs = C::rowBytes) {
  int r, pc;
  dma_slot<C>(dma_block_k<C>(w, i), lane, &r, &pc);
  return (uint32_t)r * rs + (uint32_t)((pc ^ gk8<C::D>(r)) << 4);
}
template <class C = CfgF8>
FA_HD uint32_t dma_src_v8(int w, int i, int lane, uint32_t rs = C::rowBytes) {
  int r, pc;
  dma_slot<C>(dma_block_v<C>(w, i), lane, &r, &pc);
  return (uint32_t)r * rs + (uint32_t)((pc ^ gv8<C::D>(r)) << 4);
}

// ------------------------------------------------ LDS operand reads
// S^T operand A of block kb, contraction step j (d = 64j .. 64j+63): lane
// reads key k8_key(kb, lane%32) at d = 64j + 32hh .. +31, as two 16-byte
// reads x = 0, 1 (chunks 4j + 2hh + x). Step j and read x flip chunk bits 2
// and 0 only, so their offsets are step 0's XOR (j << 6 | x << 4); block kb
// adds (64c + 16b) rows, which leaves key bits 0, 1, 2, 5 unchanged.
template <int D = 128> FA_HD uint32_t k8_read_off(int kb, int j, int x, int lane) {
  return k8_off<D>(k8_key(kb, lane & 31), 4 * j + 2 * (lane >> 5) + x);
}
FA_HD uint32_t k8_block_rows(int kb) { return (uint32_t)(64 * (kb >> 1) + 16 * (kb & 1)); }

// O^T operand A (V^T) of d-block jd (d = 32jd .. 32jd+31) and 64-key chunk
// c, read with ds_read_b64_tr_b8 in four parts t (keys 64c + 32hh + 8t +
// 0..7). The instruction works on groups of 16 lanes: result lane i,
// element e (byte) is byte i%8 of source lane 2e + i/8. Source lane s of
// group g (hh = g/2) reads key 64c + 32hh + 8t + s/2 at d = 32jd + 16(g%2) +
// 8(s%2) .. +7, so result lane i holds V[64c + 32hh + 8t + e][32jd + 16(g%2)
// + i] for e = 0..7: MFMA row l%32 is d = 32jd + l%32 with keys 32hh + 8t + e
// of the chunk, the same keys P supplies. jd flips chunk bits 1..2 (offset
// XOR jd << 5); c and t add 64c + 8t rows, which leaves key bits 1..2 alone.
template <int D = 128> FA_HD uint32_t v8_tr_off(int jd, int c, int t, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int row = 64 * c + 32 * (g >> 1) + 8 * t + (s >> 1);
  return v8_off<D>(row, 2 * jd + (g & 1)) + 8 * (s & 1);
}

// ------------------------------------------ global byte offsets (per head)
// Q operand B fragment of step j, half x: row qrow, d = 64j + 32hh + 16x .. +15.
FA_HD uint32_t q8_frag_off(int qrow, int j, int hh, int x, uint32_t rs = 128) {
  return (uint32_t)qrow * rs + (uint32_t)(64 * j + 32 * hh + 16 * x);
}
// O store (16-bit output): accumulator elements 4u .. 4u+3 of d-block jd are
// d = 32jd + 8u + 4hh + 0..3, eight bytes at row qrow.
FA_HD uint32_t o8_frag_off(int qrow, int jd, int u, int hh, uint32_t rs = 256) {
  return (uint32_t)qrow * rs + (uint32_t)((32 * jd + 8 * u + 4 * hh) * 2);
}

}  // namespace fa
