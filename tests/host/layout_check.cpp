// Host-side checker of the attention kernel's index math (fa_layout.h).
//
// Enumerates, for every lane of every wave, each LDS and global access the
// kernel makes, and checks:
//  * the global->LDS DMA of a K or V tile writes every LDS byte of the tile
//    exactly once, and each 16-byte slot receives the logical chunk the
//    swizzle assigns to it (elements are tagged with their (row, d) origin);
//  * each S^T operand read (16 bytes) returns K[32kb + row_perm32(i)][16j + 8hh + e];
//  * each pair of transposed V reads, passed through the lane permutation of
//    ds_read_b64_tr_b16 (within 16 lanes: result lane i, element e = element
//    i%4 of source lane 4e + i/4), returns V[16kc + 8h + 4rd + e][32jd +
//    row_perm32(lane%32)] -- the operand the P.V MFMA expects;
//  * the offsets the kernel turns into immediates really are additive
//    (k_read_off in kb, v_tr_off in kc and rd);
//  * all LDS offsets stay inside the tile and are aligned; global offsets of
//    in-range rows stay inside the head and out-of-range rows start at or
//    past the end (so the buffer range check drops or zero-fills them whole);
//  * the work decomposition visits each (Q tile, head) once, every key a row
//    can see lies in a tile its wave computes, and O is written exactly once;
//    a compacted variable-length launch visits each query tile within the
//    sequences once;
//  * the worst LDS bank-conflict degree of every pattern, under a 64-bank
//    model (256 bytes per cycle) and a 32-bank model (128 bytes per cycle);
//  * the eight-wave ping-pong schedule: replaying both wave groups' slots
//    (DMA issues, waits for all but the latest pair, LDS reads) in the order
//    the kernel code runs them, every read of a stage finds the tile it
//    expects, landed and published by a barrier, and no DMA overwrites a
//    stage that a wave of either group still has to read.
// All of it for every kernel configuration (four and eight waves, 16-bit),
// and the same checks for the 8-bit kernel's layouts (fa_layout8.h): its
// K operand reads, its transposed V reads through ds_read_b64_tr_b8 (within
// 16 lanes: result lane i, byte e = byte i%8 of source lane 2e + i/8), the
// accumulator-to-P key order, and its global Q loads and O stores.
//
// Prints a summary and "OK"; exits non-zero on any error.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "../../exact_attention_16_amd/csrc/fa_layout8.h"

using namespace fa;

static int g_err = 0;
#define CHECK(cond, ...)                                     \
  do {                                                       \
    if (!(cond)) {                                           \
      if (g_err < 20) {                                      \
        std::printf("ERROR %s:%d: ", __FILE__, __LINE__);    \
        std::printf(__VA_ARGS__);                            \
        std::printf("\n");                                   \
      }                                                      \
      ++g_err;                                               \
    }                                                        \
  } while (0)

// Worst conflict degree of one wave-wide access of `bytes` per lane.
static int conflict_degree(const std::vector<uint32_t>& addr, int bytes, int banks) {
  const int lanes_per_cycle = banks * 4 / bytes;
  int worst = 1;
  for (int g0 = 0; g0 < 64; g0 += lanes_per_cycle) {
    std::map<int, std::set<uint32_t>> words;  // bank -> distinct dword addresses
    for (int l = g0; l < g0 + lanes_per_cycle && l < 64; ++l)
      for (int w = 0; w < bytes / 4; ++w) {
        const uint32_t a = addr[l] / 4 + w;
        words[a % banks].insert(a);
      }
    for (auto& kv : words) worst = std::max(worst, (int)kv.second.size());
  }
  return worst;
}

// tag of element (row, d) of a tile
static long tag_of(int row, int d, int D) { return (long)row * D + d; }

// Simulate the DMA of one tile; returns per-byte-pair tags (one per element).
template <class C>
static std::vector<long> dma_tile(bool is_k, int* worst64) {
  constexpr int D = C::D;
  std::vector<long> tag(C::tileBytes / 2, -1);
  *worst64 = 1;
  for (int w = 0; w < C::NW; ++w)
    for (int i = 0; i < C::dmaPerWave; ++i) {
      std::vector<uint32_t> addr(64);
      for (int p = 0; p < 64; ++p) {
        const uint32_t dst = (is_k ? dma_lds_k<C>(w, i) : dma_lds_v<C>(w, i)) + 16 * p;
        const uint32_t src = is_k ? dma_src_k<C>(w, i, p) : dma_src_v<C>(w, i, p);
        // the kernel forms issue i's source offset as issue 0's plus a stride
        for (uint32_t rs = C::rowBytes; rs <= C::rowBytes + 48; rs += 16)
          CHECK((is_k ? dma_src_k<C>(w, i, p, rs) : dma_src_v<C>(w, i, p, rs)) ==
                    (is_k ? dma_src_k<C>(w, 0, p, rs) + i * (uint32_t)C::dmaRowsK * rs
                          : dma_src_v<C>(w, 0, p, rs) + i * (uint32_t)C::dmaRowsV * rs),
                "DMA source stride w=%d i=%d p=%d rs=%u", w, i, p, rs);
        addr[p] = dst;
        CHECK(dst % 16 == 0 && dst + 16 <= (uint32_t)C::tileBytes, "DMA dst %u", dst);
        CHECK(src % 16 == 0 && src + 16 <= (uint32_t)C::tileBytes, "DMA src %u", src);
        const int row = src / C::rowBytes, d0 = (src % C::rowBytes) / 2;
        // the slot must be where the swizzle puts that logical chunk
        const uint32_t expect = is_k ? k_off<D>(row, d0 / 8) : v_off<D>(row, d0 / 8);
        CHECK(expect == dst, "DMA slot mismatch w=%d i=%d p=%d", w, i, p);
        for (int e = 0; e < 8; ++e) {
          const uint32_t el = dst / 2 + e;
          CHECK(tag[el] == -1, "LDS element %u written twice", el);
          tag[el] = tag_of(row, d0 + e, D);
        }
      }
      *worst64 = std::max(*worst64, conflict_degree(addr, 16, 64));
    }
  for (size_t e = 0; e < tag.size(); ++e) CHECK(tag[e] != -1, "LDS element %zu never written", e);
  return tag;
}

template <class C>
static void check_lds() {
  constexpr int D = C::D;
  constexpr int BN = C::BN;
  constexpr uint32_t RB = C::rowBytes;
  int kw, vw;
  const std::vector<long> ktag = dma_tile<C>(true, &kw);
  const std::vector<long> vtag = dma_tile<C>(false, &vw);

  // ---- S^T operand reads
  int kr[2] = {1, 1};
  for (int kb = 0; kb < BN / 32; ++kb)
    for (int j = 0; j < D / 16; ++j) {
      std::vector<uint32_t> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t off = k_read_off<D>(kb, j, lane);
        CHECK(off == k_read_off<D>(0, j, lane) + (uint32_t)(kb * 32 * RB),
              "k_read_off not additive in kb");
        CHECK(off == (k_read_off<D>(0, 0, lane) ^ (uint32_t)(j << 5)) +
                         (uint32_t)(kb * 32 * RB),
              "k_read_off is not step 0 XOR (j << 5)");
        addr[lane] = off;
        CHECK(off % 16 == 0 && off + 16 <= (uint32_t)C::tileBytes, "K read off %u", off);
        const int key = 32 * kb + row_perm32(lane & 31);
        for (int e = 0; e < 8; ++e)
          CHECK(ktag[off / 2 + e] == tag_of(key, 16 * j + 8 * (lane >> 5) + e, D),
                "K read kb=%d j=%d lane=%d e=%d", kb, j, lane, e);
      }
      kr[0] = std::max(kr[0], conflict_degree(addr, 16, 64));
      kr[1] = std::max(kr[1], conflict_degree(addr, 16, 32));
    }

  // ---- V^T operand: pairs of transposed reads
  int vr[2] = {1, 1};
  for (int jd = 0; jd < D / 32; ++jd)
    for (int kc = 0; kc < BN / 16; ++kc)
      for (int rd = 0; rd < 2; ++rd) {
        std::vector<uint32_t> addr(64);
        long src[64][4];
        for (int lane = 0; lane < 64; ++lane) {
          const uint32_t off = v_tr_off<D>(jd, kc, rd, lane);
          CHECK(off == v_tr_off<D>(jd, 0, 0, lane) + (uint32_t)(kc * 16 * RB) +
                           (uint32_t)(rd * 4 * RB),
                "v_tr_off not additive in kc/rd");
          CHECK(off == (v_tr_off<D>(0, 0, 0, lane) ^ (uint32_t)(jd << 6)) +
                           (uint32_t)(kc * 16 * RB) + (uint32_t)(rd * 4 * RB),
                "v_tr_off is not block 0 XOR (jd << 6)");
          addr[lane] = off;
          CHECK(off % 8 == 0 && off + 8 <= (uint32_t)C::tileBytes, "V read off %u", off);
          for (int e = 0; e < 4; ++e) src[lane][e] = vtag[off / 2 + e];
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g0 = lane & ~15, i = lane & 15;
          const int d = 32 * jd + row_perm32(lane & 31);
          for (int e = 0; e < 4; ++e) {
            const long got = src[g0 + 4 * e + i / 4][i % 4];
            const int key = 16 * kc + 8 * (lane >> 5) + 4 * rd + e;
            CHECK(got == tag_of(key, d, D), "V^T read jd=%d kc=%d rd=%d lane=%d e=%d", jd, kc,
                  rd, lane, e);
          }
        }
        vr[0] = std::max(vr[0], conflict_degree(addr, 8, 64));
        vr[1] = std::max(vr[1], conflict_degree(addr, 8, 32));
      }

  // ---- accumulator -> P operand key mapping
  for (int hh = 0; hh < 2; ++hh)
    for (int r = 0; r < 16; ++r) {
      const int rho = 8 * (r / 4) + 4 * hh + (r % 4);
      CHECK(row_perm32(rho) == acc_key32(r, hh), "acc key r=%d hh=%d", r, hh);
      CHECK(acc_key32(r, hh) == 16 * (r / 8) + 8 * hh + (r % 8), "P operand key");
    }
  for (int r = 0; r < 32; ++r) CHECK(row_perm32(row_perm32(r)) == r, "perm involution");

  std::printf("D=%d waves=%d BN=%d tile=%d B: conflict degree (64 banks / 32 banks): K operand "
              "read %d/%d, V^T transposed read %d/%d; DMA writes %d/%d (64 banks)\n",
              D, C::NW, BN, C::tileBytes, kr[0], kr[1], vr[0], vr[1], kw, vw);
  CHECK(kr[0] == 1 && kr[1] == 1, "K operand reads conflict");
  CHECK(vr[0] == 1, "V^T reads conflict (64 banks)");
  CHECK(kw == 1 && vw == 1, "DMA writes conflict");
}

// Replays every global access of one kernel configuration for B*H heads
// with Sq query rows and Sk key rows each (per-sequence lengths of a
// variable-length batch are the same per work-group), rows `rs` bytes apart
// in every tensor, and checks: the work-group map is a bijection; every key a
// row sees lies in a tile its wave computes; tiles taken as mask-free hold
// only keys every row of the wave sees; in-range rows stay inside their
// buffer descriptors and rows past the end fall wholly outside; every O
// element and lse entry is written exactly once.
template <class C>
static void check_global(int B, int H, int Sq, int Sk, bool causal, uint32_t rs = C::rowBytes) {
  constexpr int D = C::D;
  const int BH = B * H;
  const int nqt = num_q_tiles(Sq, C::BM);
  const long grid = (long)nqt * BH;
  constexpr int BN = C::BN;
  const int off = Sk - Sq;
  const uint32_t q_bytes = (uint32_t)Sq * rs;
  std::vector<char> seen(grid, 0);
  const size_t head_elems = (size_t)Sq * D;
  const bool track = head_elems * (size_t)BH <= ((size_t)1 << 26);
  std::vector<char> owritten(track ? head_elems * BH : 0, 0);
  std::vector<char> lwritten(track ? (size_t)Sq * BH : 0, 0);
  for (long bid = 0; bid < grid; ++bid) {
    int qt, bh;
    block_to_tile((int)bid, BH, nqt, causal, &qt, &bh);
    CHECK(qt >= 0 && qt < nqt && bh >= 0 && bh < BH, "tile map bid=%ld", bid);
    const long cell = (long)qt * BH + bh;
    CHECK(!seen[cell], "tile visited twice");
    seen[cell] = 1;
    if (qt * C::BM >= Sq) continue;  // the work-group returns at once
    const int kv_end = tile_kv_end(qt, Sq, Sk, causal, C::BM);
    const int ntiles = (kv_end + BN - 1) / BN;
    CHECK(ntiles >= 0 && (ntiles == 0 || (ntiles - 1) * BN < Sk), "tile count");
    // DMA sources: tile-relative offsets; rows past the end start at or past
    // the descriptor's range (Sk - kv0) * rs
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t range = (uint32_t)(Sk - t * BN) * rs;
      for (int w = 0; w < C::NW; ++w)
        for (int i = 0; i < C::dmaPerWave; ++i)
          for (int p = 0; p < 64; ++p)
            for (int kv = 0; kv < 2; ++kv) {
              const uint32_t o = kv ? dma_src_v<C>(w, i, p, rs) : dma_src_k<C>(w, i, p, rs);
              const int row = o / rs;
              CHECK(o % rs + 16 <= (uint32_t)C::rowBytes, "DMA chunk leaves its row");
              if (t * BN + row < Sk)
                CHECK(o + 16 <= range, "DMA in-range row crosses the end");
              else
                CHECK(o >= range, "DMA row past Sk not wholly out of range");
            }
    }
    for (int wave = 0; wave < C::NW; ++wave) {
      for (int sub = 0; sub < C::RPW / kRowsPerWave; ++sub) {
      const int q0w = qt * C::BM + wave * C::RPW + sub * kRowsPerWave;
      const bool live = q0w < Sq;
      const int nw = live ? (wave_kv_end(q0w, Sq, Sk, causal) + BN - 1) / BN : 0;
      CHECK(nw <= ntiles, "wave computes a tile the work-group does not load");
      if (live) {
        const int unm = unmasked_tiles(q0w, Sq, Sk, causal, BN);
        CHECK(unm <= nw, "mask-free tiles beyond the wave's tiles");
        for (int r = q0w; r < q0w + kRowsPerWave && r < Sq; ++r) {
          const int last = causal ? r + off : Sk - 1;  // last key row r sees
          if (unm > 0)
            CHECK(unm * BN - 1 <= last && unm * BN <= Sk, "tile %d taken as mask-free for row %d",
                  unm - 1, r);
        }
      }
      for (int lane = 0; lane < 64; ++lane) {
        const int qrow = q0w + (lane & 31), hh = lane >> 5;
        if (qrow < Sq) {
          // every key this row can see lies in a computed tile
          const int last_key = causal ? (qrow + off < Sk ? qrow + off : Sk - 1) : Sk - 1;
          if (last_key >= 0)
            CHECK(live && last_key < nw * BN, "row %d key %d not covered", qrow, last_key);
        }
        for (int j = 0; j < D / 16; ++j) {
          const uint32_t o = q_frag_off<D>(qrow, j, hh, rs);
          if (qrow < Sq)
            CHECK(o + 16 <= q_bytes, "Q load out of bounds");
          else
            CHECK(o >= q_bytes, "Q row past Sq not wholly out of range");
        }
        if (!live) continue;
        for (int jd = 0; jd < D / 32; ++jd)
          for (int g = 0; g < 2; ++g) {
            const uint32_t o = o_frag_off<D>(qrow, jd, g, hh, rs);
            if (qrow >= Sq) {
              CHECK(o >= q_bytes, "O store past Sq not wholly out of range");
              continue;
            }
            CHECK(o + 16 <= q_bytes && o % rs + 16 <= (uint32_t)C::rowBytes,
                  "O store out of bounds");
            if (track)
              for (int e = 0; e < 8; ++e) {
                const size_t pe = (size_t)bh * head_elems + (size_t)(o / rs) * D + (o % rs) / 2 + e;
                CHECK(!owritten[pe], "O element written twice");
                owritten[pe] = 1;
              }
          }
        if (hh == 0) {
          if (qrow < Sq) {
            CHECK((uint32_t)qrow * 4u + 4u <= (uint32_t)Sq * 4u, "lse store");
            if (track) {
              CHECK(!lwritten[(size_t)bh * Sq + qrow], "lse written twice");
              lwritten[(size_t)bh * Sq + qrow] = 1;
            }
          } else {
            CHECK((uint32_t)qrow * 4u >= (uint32_t)Sq * 4u, "lse past Sq in range");
          }
        }
      }
      }
    }
  }
  for (long c = 0; c < grid; ++c) CHECK(seen[c], "tile never visited");
  if (track) {
    for (size_t p = 0; p < owritten.size(); ++p) CHECK(owritten[p], "O element not written");
    for (size_t p = 0; p < lwritten.size(); ++p) CHECK(lwritten[p], "lse not written");
  }
}

template <class C> static void check_global(int B, int H, int S, bool causal) {
  check_global<C>(B, H, S, S, causal);
}

// Query/key length pairs (as in a variable-length batch), with padded rows.
template <class C> static void check_lengths() {
  const int lens[] = {0, 1, 31, 32, 33, 95, 96, 97, 200, 255, 256, 257, 513};
  for (int lq : lens)
    for (int lk : lens)
      for (int causal = 0; causal < 2; ++causal) {
        if (lq == 0) continue;
        check_global<C>(1, 2, lq, lk, causal != 0);
        check_global<C>(1, 1, lq, lk, causal != 0, C::rowBytes + 48);
      }
}

// ------------------------------------------------ 8-bit kernel (fa_layout8.h)
template <class C> static std::vector<long> dma_tile8(bool is_k, int* worst64) {
  std::vector<long> tag(C::tileBytes, -1);  // one tag per byte (element)
  *worst64 = 1;
  for (int w = 0; w < C::NW; ++w)
    for (int i = 0; i < C::dmaPerWave; ++i) {
      std::vector<uint32_t> addr(64);
      for (int p = 0; p < 64; ++p) {
        const uint32_t dst = (is_k ? dma_lds_k<C>(w, i) : dma_lds_v<C>(w, i)) + 16 * p;
        const uint32_t src = is_k ? dma_src_k8<C>(w, i, p) : dma_src_v8<C>(w, i, p);
        for (uint32_t rs = C::rowBytes; rs <= C::rowBytes + 64; rs += 16)
          CHECK((is_k ? dma_src_k8<C>(w, i, p, rs) : dma_src_v8<C>(w, i, p, rs)) ==
                    (is_k ? dma_src_k8<C>(w, 0, p, rs) + i * (uint32_t)C::dmaRowsK * rs
                          : dma_src_v8<C>(w, 0, p, rs) + i * (uint32_t)C::dmaRowsV * rs),
                "8-bit DMA source stride w=%d i=%d p=%d rs=%u", w, i, p, rs);
        addr[p] = dst;
        CHECK(dst % 16 == 0 && dst + 16 <= (uint32_t)C::tileBytes, "DMA dst %u", dst);
        CHECK(src % 16 == 0 && src + 16 <= (uint32_t)C::tileBytes, "DMA src %u", src);
        const int row = src / C::rowBytes, d0 = src % C::rowBytes;
        const uint32_t expect = is_k ? k8_off<C::D>(row, d0 / 16) : v8_off<C::D>(row, d0 / 16);
        CHECK(expect == dst, "8-bit DMA slot mismatch w=%d i=%d p=%d", w, i, p);
        for (int e = 0; e < 16; ++e) {
          CHECK(tag[dst + e] == -1, "LDS byte %u written twice", dst + e);
          tag[dst + e] = tag_of(row, d0 + e, C::D);
        }
      }
      *worst64 = std::max(*worst64, conflict_degree(addr, 16, 64));
    }
  for (size_t e = 0; e < tag.size(); ++e) CHECK(tag[e] != -1, "LDS byte %zu never written", e);
  return tag;
}

template <class C> static void check_lds8() {
  constexpr int D = C::D;
  int kw, vw;
  const std::vector<long> ktag = dma_tile8<C>(true, &kw);
  const std::vector<long> vtag = dma_tile8<C>(false, &vw);

  // ---- S^T operand reads: block kb, step j, half x
  int kr[2] = {1, 1};
  for (int kb = 0; kb < C::BN / 32; ++kb)
    for (int j = 0; j < D / 64; ++j)
      for (int x = 0; x < 2; ++x) {
        std::vector<uint32_t> addr(64);
        for (int lane = 0; lane < 64; ++lane) {
          const uint32_t off = k8_read_off<D>(kb, j, x, lane);
          CHECK(off == (k8_read_off<D>(0, 0, 0, lane) ^ (uint32_t)(j << 6 | x << 4)) +
                           k8_block_rows(kb) * (uint32_t)C::rowBytes,
                "k8_read_off is not step 0 XOR (j << 6 | x << 4) plus the block's rows");
          addr[lane] = off;
          CHECK(off % 16 == 0 && off + 16 <= (uint32_t)C::tileBytes, "K8 read off %u", off);
          const int key = k8_key(kb, lane & 31);
          for (int e = 0; e < 16; ++e)
            CHECK(ktag[off + e] == tag_of(key, 64 * j + 32 * (lane >> 5) + 16 * x + e, D),
                  "K8 read kb=%d j=%d x=%d lane=%d e=%d", kb, j, x, lane, e);
        }
        kr[0] = std::max(kr[0], conflict_degree(addr, 16, 64));
        kr[1] = std::max(kr[1], conflict_degree(addr, 16, 32));
      }

  // ---- V^T operand: four transposed 8-byte reads per (jd, chunk)
  int vr[2] = {1, 1};
  for (int jd = 0; jd < D / 32; ++jd)
    for (int c = 0; c < C::BN / 64; ++c)
      for (int t = 0; t < 4; ++t) {
        std::vector<uint32_t> addr(64);
        long src[64][8];
        for (int lane = 0; lane < 64; ++lane) {
          const uint32_t off = v8_tr_off<D>(jd, c, t, lane);
          CHECK(off == (v8_tr_off<D>(0, 0, 0, lane) ^ (uint32_t)(jd << 5)) +
                           (uint32_t)((64 * c + 8 * t) * C::rowBytes),
                "v8_tr_off is not block 0 XOR (jd << 5) plus 64c + 8t rows");
          addr[lane] = off;
          CHECK(off % 8 == 0 && off + 8 <= (uint32_t)C::tileBytes, "V8 read off %u", off);
          for (int b = 0; b < 8; ++b) src[lane][b] = vtag[off + b];
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g0 = lane & ~15, i = lane & 15;
          const int d = 32 * jd + (lane & 31);
          for (int e = 0; e < 8; ++e) {
            const long got = src[g0 + 2 * e + i / 8][i % 8];
            const int key = 64 * c + 32 * (lane >> 5) + 8 * t + e;
            CHECK(got == tag_of(key, d, D), "V8^T read jd=%d c=%d t=%d lane=%d e=%d", jd, c, t,
                  lane, e);
          }
        }
        vr[0] = std::max(vr[0], conflict_degree(addr, 8, 64));
        vr[1] = std::max(vr[1], conflict_degree(addr, 8, 32));
      }

  // ---- accumulator -> P operand key order
  for (int kb = 0; kb < C::BN / 32; ++kb)
    for (int hh = 0; hh < 2; ++hh)
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r / 4) + 4 * hh + (r % 4);  // MFMA row of element r
        CHECK(k8_key(kb, row) == acc_key8(kb, r, hh), "8-bit acc key kb=%d r=%d hh=%d", kb, r, hh);
      }
  for (int c = 0; c < C::BN / 64; ++c)
    for (int hh = 0; hh < 2; ++hh)
      for (int e = 0; e < 32; ++e)  // byte e of the lane's P operand of chunk c
        CHECK(acc_key8(2 * c + e / 16, e % 16, hh) == 64 * c + 32 * hh + e, "8-bit P key order");
  std::set<int> keys;
  for (int kb = 0; kb < C::BN / 32; ++kb)
    for (int r = 0; r < 32; ++r) keys.insert(k8_key(kb, r));
  CHECK((int)keys.size() == C::BN && *keys.begin() == 0 && *keys.rbegin() == C::BN - 1,
        "8-bit K rows are not a permutation of the tile");

  std::printf("8-bit D=%d waves=%d BN=%d tile=%d B: conflict degree (64 banks / 32 banks): K "
              "operand read %d/%d, V^T transposed read %d/%d; DMA writes %d/%d (64 banks)\n",
              D, C::NW, C::BN, C::tileBytes, kr[0], kr[1], vr[0], vr[1], kw, vw);
  CHECK(kr[0] == 1 && kr[1] == 1, "8-bit K operand reads conflict");
  CHECK(vr[0] == 1, "8-bit V^T reads conflict (64 banks)");
  CHECK(kw == 1 && vw == 1, "8-bit DMA writes conflict");
}

// Global accesses of the 8-bit kernel for B*H heads of Sq x Sk: rows rs
// bytes apart in q, k, v and rso bytes apart in o (16-bit output).
template <class C>
static void check_global8(int B, int H, int Sq, int Sk, bool causal, uint32_t rs = C::rowBytes,
                          uint32_t rso = 2 * C::D) {
  const int BH = B * H, nqt = num_q_tiles(Sq, C::BM), BN = C::BN;
  const long grid = (long)nqt * BH;
  const uint32_t q_bytes = (uint32_t)Sq * rs, o_bytes = (uint32_t)Sq * rso;
  const size_t head_elems = (size_t)Sq * C::D;
  const bool track = head_elems * (size_t)BH <= ((size_t)1 << 26);
  std::vector<char> seen(grid, 0), owritten(track ? head_elems * BH : 0, 0);
  for (long bid = 0; bid < grid; ++bid) {
    int qt, bh;
    block_to_tile((int)bid, BH, nqt, causal, &qt, &bh);
    const long cell = (long)qt * BH + bh;
    CHECK(qt >= 0 && qt < nqt && bh >= 0 && bh < BH && !seen[cell], "8-bit tile map bid=%ld", bid);
    seen[cell] = 1;
    if (qt * C::BM >= Sq) continue;
    const int ntiles = (tile_kv_end(qt, Sq, Sk, causal, C::BM) + BN - 1) / BN;
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t range = (uint32_t)(Sk - t * BN) * rs;
      for (int w = 0; w < C::NW; ++w)
        for (int i = 0; i < C::dmaPerWave; ++i)
          for (int p = 0; p < 64; ++p)
            for (int kv = 0; kv < 2; ++kv) {
              const uint32_t o = kv ? dma_src_v8<C>(w, i, p, rs) : dma_src_k8<C>(w, i, p, rs);
              const int row = o / rs;
              CHECK(o % rs + 16 <= (uint32_t)C::rowBytes, "8-bit DMA chunk leaves its row");
              if (t * BN + row < Sk)
                CHECK(o + 16 <= range, "8-bit DMA in-range row crosses the end");
              else
                CHECK(o >= range, "8-bit DMA row past Sk not wholly out of range");
            }
    }
    for (int wave = 0; wave < C::NW; ++wave) {
      const int q0w = qt * C::BM + wave * C::RPW;
      const bool live = q0w < Sq;
      const int nw = live ? (wave_kv_end(q0w, Sq, Sk, causal) + BN - 1) / BN : 0;
      CHECK(nw <= ntiles, "8-bit wave computes a tile the work-group does not load");
      for (int lane = 0; lane < 64; ++lane) {
        const int qrow = q0w + (lane & 31), hh = lane >> 5;
        for (int j = 0; j < C::D / 64; ++j)
          for (int x = 0; x < 2; ++x) {
            const uint32_t o = q8_frag_off(qrow, j, hh, x, rs);
            if (qrow < Sq)
              CHECK(o + 16 <= q_bytes && o % rs + 16 <= (uint32_t)C::rowBytes, "Q8 load out of bounds");
            else
              CHECK(o >= q_bytes, "Q8 row past Sq not wholly out of range");
          }
        if (!live) continue;
        for (int jd = 0; jd < C::D / 32; ++jd)
          for (int u = 0; u < 4; ++u) {
            const uint32_t o = o8_frag_off(qrow, jd, u, hh, rso);
            if (qrow >= Sq) {
              CHECK(o >= o_bytes, "O8 store past Sq not wholly out of range");
              continue;
            }
            CHECK(o + 8 <= o_bytes && o % rso + 8 <= (uint32_t)C::D * 2, "O8 store out of bounds");
            // accumulator elements 4u + e of d-block jd are d = 32jd + 8u + 4hh + e
            CHECK((o % rso) / 2 == (uint32_t)(32 * jd + 8 * u + 4 * hh), "O8 column");
            if (track)
              for (int e = 0; e < 4; ++e) {
                const size_t pe = (size_t)bh * head_elems + (size_t)(o / rso) * C::D + (o % rso) / 2 + e;
                CHECK(!owritten[pe], "O8 element written twice");
                owritten[pe] = 1;
              }
          }
      }
    }
  }
  for (long c = 0; c < grid; ++c) CHECK(seen[c], "8-bit tile never visited");
  if (track)
    for (size_t p = 0; p < owritten.size(); ++p) CHECK(owritten[p], "O8 element not written");
}

// The work-group map for every head-group size a launch can pick: a
// bijection of ids onto (Q tile, head), every head on XCD head mod 8 when
// B*H is a multiple of 8, and causal tiles of a group in descending order.
static void check_tile_map() {
  const int bhs[] = {1, 3, 8, 16, 24, 64, 256, 640}, nqts[] = {1, 3, 32};
  const int hgs[] = {1, 2, 3, 4, 8};
  for (int BH : bhs)
    for (int nqt : nqts)
      for (int hg : hgs)
        for (int causal = 0; causal < 2; ++causal) {
          std::vector<char> seen((size_t)BH * nqt, 0);
          std::vector<int> last_qt(BH, 1 << 30);
          for (int bid = 0; bid < BH * nqt; ++bid) {
            int qt, bh;
            block_to_tile(bid, BH, nqt, causal != 0, &qt, &bh, hg);
            CHECK(qt >= 0 && qt < nqt && bh >= 0 && bh < BH, "tile map range");
            if (!(qt >= 0 && qt < nqt && bh >= 0 && bh < BH)) continue;
            CHECK(!seen[(size_t)qt * BH + bh], "tile map not one-to-one BH=%d nqt=%d hg=%d", BH, nqt, hg);
            seen[(size_t)qt * BH + bh] = 1;
            if (BH % 8 == 0) CHECK(bh % 8 == bid % 8, "head off its XCD");
            if (causal) {  // each head's tiles come heaviest first
              CHECK(qt < last_qt[bh], "causal tiles of a head out of order");
              last_qt[bh] = qt;
            }
          }
        }
}

// The compacted variable-length launch (varlen_cap, varlen_tile): for
// offset arrays that never decrease, the bound covers every query tile within
// the sequences, and ids below it map one-to-one onto those tiles (the rest
// onto nothing), each head on XCD head mod 8 when H is a multiple of 8, a
// sequence's causal tiles heaviest first. The sequence search is done twice:
// a plain walk over the sequences, and the kernel's lane-parallel form
// (varlen_find: four sequences per lane, an inclusive sum over 64 lanes, the
// first lane whose sum exceeds the rank, a walk of that lane's four).
static bool find_plain(const std::vector<int>& cnt, int k, int* g, int* r) {
  for (int b = 0; b < (int)cnt.size(); ++b) {
    if (k < cnt[b]) {
      *g = b;
      *r = k;
      return true;
    }
    k -= cnt[b];
  }
  return false;
}
static bool find_lanes(const std::vector<int>& cnt, int k, int* g, int* r) {
  const int B = (int)cnt.size();
  int tot[64], incl[64];
  for (int l = 0; l < 64; ++l) {
    tot[l] = 0;
    for (int i = 0; i < 4; ++i)
      if (4 * l + i < B) tot[l] += cnt[4 * l + i];
  }
  for (int l = 0; l < 64; ++l) incl[l] = tot[l] + (l ? incl[l - 1] : 0);
  int L = -1;
  for (int l = 0; l < 64 && L < 0; ++l)
    if (k < incl[l]) L = l;
  if (L < 0) return false;
  int rr = k - (incl[L] - tot[L]);
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * L + i < B ? cnt[4 * L + i] : 0;
    if (rr < c) {
      *g = 4 * L + i;
      *r = rr;
      return true;
    }
    rr -= c;
  }
  return false;
}
static void check_varlen_map() {
  unsigned seed = 12345u;
  auto rnd = [&](int n) {
    seed = seed * 1103515245u + 12345u;
    return (int)((seed >> 8) % (unsigned)n);
  };
  const int Hs[] = {1, 3, 8, 16, 24};
  const int Bs[] = {1, 2, 7, 63, 64, 65, 200, kCompactMaxSeqs};
  const int BMs[] = {64, 128, 256};
  long checked = 0;
  for (int H : Hs)
    for (int B : Bs)
      for (int BM : BMs)
        for (int causal = 0; causal < 2; ++causal)
          for (int rep = 0; rep < 3; ++rep) {
            // lengths: a mix of empty, short and long sequences; Sq is the
            // longest (rep 2: some sequences past a stated maximum)
            std::vector<int> len(B);
            int Sq = 1, totq = 0;
            for (int b = 0; b < B; ++b) {
              const int kind = rnd(4);
              len[b] = kind == 0 ? 0 : kind == 1 ? 1 + rnd(BM) : 1 + rnd(20 * BM);
              totq += len[b];
              Sq = std::max(Sq, len[b]);
            }
            if (rep == 2) Sq = std::max(1, Sq / 2);
            const int nqt = num_q_tiles(Sq, BM);
            const bool xcd = H % 8 == 0;
            const int m = xcd ? H / 8 : H;
            std::vector<int> nt(B), cnt(B);
            long need = 0;
            for (int b = 0; b < B; ++b) {
              nt[b] = num_q_tiles(std::min(len[b], Sq), BM);
              cnt[b] = m * nt[b];
              need += nt[b];
            }
            const long long cap = varlen_cap(totq, B, nqt, BM);
            CHECK(need <= cap, "varlen bound %lld below the %ld tiles", cap, need);
            const long long items = cap * H;
            std::map<long long, int> seen;  // (b, h, qt) -> id
            std::vector<int> last_qt((size_t)B * H, 1 << 30);
            for (long long id = 0; id < items; ++id) {
              const int k = xcd ? (int)(id >> 3) : (int)id;
              int g, r, g2, r2;
              const bool any = find_plain(cnt, k, &g, &r);
              const bool any2 = find_lanes(cnt, k, &g2, &r2);
              CHECK(any == any2 && (!any || (g == g2 && r == r2)), "lane search differs");
              if (!any) continue;
              int qt, j;
              varlen_tile(r, m, nt[g], causal != 0, &qt, &j);
              const int h = xcd ? (int)(id & 7) + 8 * j : j;
              CHECK(qt >= 0 && qt < nt[g] && h >= 0 && h < H, "varlen tile out of range");
              if (!(qt >= 0 && qt < nt[g] && h >= 0 && h < H)) continue;
              const long long key = ((long long)g * H + h) * nqt + qt;
              CHECK(!seen.count(key), "varlen tile twice B=%d H=%d BM=%d", B, H, BM);
              seen[key] = (int)id;
              if (xcd) CHECK(h % 8 == id % 8, "varlen head off its XCD");
              if (causal) {
                CHECK(qt < last_qt[(size_t)g * H + h], "varlen causal tiles out of order");
                last_qt[(size_t)g * H + h] = qt;
              }
              ++checked;
            }
            CHECK((long)seen.size() == need * H, "varlen tiles missed: %zu of %ld", seen.size(),
                  need * H);
          }
  std::printf("varlen compacted map: %ld work items checked\n", checked);
}

// ------------------------------------------------ ping-pong schedule replay
// One DMA share (one wave's issues) of a tile into a stage.
struct Share {
  int issue_slot;  // slot in which it was issued
  int land_slot;   // end of this slot: the issuing wave has waited for it
                   // (-1: before slot 0; kNotLanded: not yet)
};
constexpr int kNotLanded = -1000;
struct Stage {
  int tile = -2;  // tile the stage holds (-1: zeros of an empty range)
  std::vector<Share> shares;
};

// Replays the slots of both groups of the eight-wave kernel for a work-group
// with `ntiles` KV tiles and waves that compute `nw` of them, mirroring the
// kernel's code order (with one or two barriers per step), and checks every
// read and every overwrite.
static void check_pingpong(int ntiles, int nw, bool one_barrier) {
  const int NS = kStages;
  Stage kst[3], vst[3];
  // pending DMA per group: (array, stage index) of each share of the latest
  // pairs not yet waited for, in issue order; a wait for all but the latest
  // pair lands everything older.
  struct Pend { Stage* st; size_t share; int pair; };
  std::vector<Pend> pend[2];
  int last_pair[2] = {-100, -100};
  // reads in each slot, for the overwrite check: (array, stage, tile)
  std::map<int, std::vector<std::pair<Stage*, int>>> reads;

  auto issue = [&](int g, Stage* st, int tile, int slot, int pair) {
    if (st->shares.size() == 2) {  // both groups' shares of the old content
      // no read of the old content may happen in or after this slot
      for (auto& kv : reads)
        if (kv.first >= slot)
          for (auto& r : kv.second)
            CHECK(!(r.first == st && r.second == st->tile), "stage overwritten while read");
      st->shares.clear();
      st->tile = tile;
    } else if (st->shares.empty()) {
      st->tile = tile;
    } else {
      CHECK(st->tile == tile, "the two groups DMA different tiles into one stage");
    }
    st->shares.push_back({slot, kNotLanded});
    pend[g].push_back({st, st->shares.size() - 1, pair});
  };
  auto wait_all_but_latest = [&](int g, int slot) {
    std::vector<Pend> keep;
    for (auto& p : pend[g]) {
      if (p.pair == last_pair[g]) keep.push_back(p);
      else p.st->shares[p.share].land_slot = slot;
    }
    pend[g] = keep;
  };
  auto wait_all = [&](int g, int slot) {
    for (auto& p : pend[g]) p.st->shares[p.share].land_slot = slot;
    pend[g].clear();
  };
  auto read = [&](Stage* st, int tile, int slot) {
    CHECK(st->tile == tile, "slot %d reads tile %d but the stage holds %d", slot, tile, st->tile);
    CHECK(st->shares.size() == 2, "slot %d reads a stage only one group has filled", slot);
    for (auto& sh : st->shares)
      CHECK(sh.land_slot != kNotLanded && sh.land_slot < slot, "slot %d reads tile %d before it landed",
            slot, tile);
    reads[slot].push_back({st, tile});
  };
  auto dma_pair = [&](int g, int i, int slot) {
    last_pair[g] = i;
    issue(g, &kst[(i + 2) % NS], i + 2 < ntiles ? i + 2 : -1, slot, i);
    issue(g, &vst[(i + 1) % NS], i + 1 < ntiles ? i + 1 : -1, slot, i);
  };

  // prologue (both groups): K(0), then K(1) and V(0); before the first
  // barrier each group waits for all but its last 2*DPW loads, so K(0) has
  // landed and K(1), V(0) (a pair of their own, id -1) are in flight until the
  // first wait for all but the latest pair. K stage 2 and V stages 1, 2 are
  // first written by DMA pairs 0 and 1.
  for (int g = 0; g < 2; ++g) {
    issue(g, &kst[0], 0, -1, -2);
    wait_all(g, -1);
    last_pair[g] = -1;
    issue(g, &kst[1], ntiles > 1 ? 1 : -1, -1, -1);
    issue(g, &vst[0], 0, -1, -1);
  }
  auto step_reads = [&](int j, int t) {
    if (j >= 1 && j - 1 < nw) read(&vst[(j + 2) % NS], j - 1, t);
    if (j < nw) read(&kst[j % NS], j, t);
  };
  int nslots;
  if (one_barrier) {
    // slot t: A issues pair t, then its MFMA phase of step t; B runs its
    // softmax phase of step t-1 (no LDS access), issues pair t (pair 0 before
    // its loop), then its MFMA phase of step t.
    nslots = ntiles + 1;
    for (int t = 0; t < nslots; ++t) {
      for (int g = 0; g < 2; ++g) {
        dma_pair(g, t, t);
        step_reads(t, t);
      }
      for (int g = 0; g < 2; ++g) wait_all_but_latest(g, t);
    }
  } else {
    // Both groups advance slot by slot; the slot numbers of each group's
    // code follow the kernel: A runs step j in (2j, 2j+1), B in (2j+1, 2j+2).
    nslots = 2 * ntiles + 3;
    for (int t = 0; t < nslots; ++t) {
      for (int g = 0; g < 2; ++g) {
        const int local = t - g;  // B's slot 0 is its lone DMA slot
        if (g == 1 && t == 0) {
          dma_pair(1, 0, t);
        } else if (g == 0 && t == nslots - 1) {
          // A's lone last slot
        } else {
          const int j = local / 2;
          if (local % 2 == 0) {  // MFMA phase of step j
            if (g == 0) dma_pair(0, j, t);
            step_reads(j, t);
          } else {  // softmax phase of step j
            if (g == 1) dma_pair(1, j + 1, t);
          }
        }
      }
      for (int g = 0; g < 2; ++g) wait_all_but_latest(g, t);
    }
  }
  for (int g = 0; g < 2; ++g) wait_all(g, nslots);
  CHECK(pp_slots(ntiles, one_barrier) == nslots, "slot count");
  // every tile was read by both groups
  int nread = 0;
  for (auto& kv : reads) nread += (int)kv.second.size();
  CHECK(nread == 2 * 2 * nw, "read count %d for %d wave tiles", nread, nw);
}

// Interleaved eight-wave schedule (fa_interleave.h): DMA pair j (K(j+2),
// V(j+1)) is issued at the start of iteration j, before the barrier, so it
// may run while slower waves are still in iteration j-1; after the barrier
// of iteration j every pair up to j-1 has landed. Iteration j reads K(j+1)
// (at the last tile too: S(j+1) is computed and dropped) and V(j); the
// prologue reads K(0).
static void check_il_schedule(int ntiles) {
  const int NS = kStages;
  // the prologue loads K(0), K(1), V(0); K stage 2 and V stages 1, 2 hold
  // nothing until DMA pairs 0 and 1 (tile -2: never written)
  int ktile[3] = {0, ntiles > 1 ? 1 : -1, -2}, vtile[3] = {0, -2, -2};
  int kpair[3] = {-1, -1, -1}, vpair[3] = {-1, -1, -1};  // pair that wrote the stage (-1: prologue)
  int kread[3] = {-1, -2, -2}, vread[3] = {-2, -2, -2};  // last iteration reading the stage
  for (int j = 0; j < ntiles; ++j) {
    const int sk = (j + 2) % NS, sv = (j + 1) % NS;
    CHECK(kread[sk] <= j - 2, "il: K stage %d refilled at %d while read at %d", sk, j, kread[sk]);
    CHECK(vread[sv] <= j - 2, "il: V stage %d refilled at %d while read at %d", sv, j, vread[sv]);
    ktile[sk] = j + 2 < ntiles ? j + 2 : -1;
    vtile[sv] = j + 1 < ntiles ? j + 1 : -1;
    kpair[sk] = j;
    vpair[sv] = j;
    const int rk = (j + 1) % NS, rv = j % NS;
    CHECK(kpair[rk] <= j - 1, "il: K stage %d read at %d before its DMA landed", rk, j);
    if (j + 1 < ntiles) CHECK(ktile[rk] == j + 1, "il: K(%d) not resident at %d", j + 1, j);
    CHECK(vtile[rv] == j && vpair[rv] <= j - 1, "il: V(%d) not resident at %d", j, j);
    kread[rk] = j;
    vread[rv] = j;
  }
}

// The two-stage schedule of the four-waves-per-SIMD kernel (and of each
// group of the key-split kernel, over its own tiles): step j reads K(j) and
// V(j) from stage j % 2; at its top it issues the DMA of tile j+1 into the
// other stage, whose last reader was step j-1 (every wave has passed the
// barrier that ends step j-1); the wait before the barrier that ends step j
// lands that DMA.
static void check_two_stage(int ntiles) {
  int tile[2] = {0, -2};       // tile held by the stage (the prologue loads tile 0)
  int landed[2] = {1, 1};      // whether its DMA has landed
  int last_read[2] = {-1, -2}; // step that last read the stage
  for (int j = 0; j < ntiles; ++j) {
    const int cur = j % 2, oth = 1 - cur;
    if (j + 1 < ntiles) {
      CHECK(last_read[oth] <= j - 1, "two-stage: stage %d overwritten while read at %d", oth, j);
      tile[oth] = j + 1;
      landed[oth] = 0;
    }
    CHECK(tile[cur] == j && landed[cur], "two-stage: tile %d not resident at step %d", j, j);
    last_read[cur] = j;
    landed[oth] = 1;  // the wait before the barrier ending step j
  }
}

// the key-split kernel's per-group configuration (two waves, 64 rows,
// 64-key tiles) and the four-waves-per-SIMD kernel's (eight waves, 256 rows,
// 64-key tiles)
using CfgSplitG = Cfg<64, 2, 64>;
using CfgOcc = Cfg<64, 8, 64>;

int main() {
  check_lds<Cfg4<64>>();
  check_lds<Cfg4<128>>();
  check_lds<Cfg8<64>>();
  check_lds<Cfg8<128>>();
  check_lds<CfgSplitG>();
  check_lds<CfgOcc>();
  check_tile_map();
  check_varlen_map();
  std::printf("work-group map: every head-group size: checked\n");
  // persistent work-groups: every item exactly once, ids rising per group
  for (int G : {8, 16, 256, 264})
    for (int total : {1, 7, 8, 100, 256, 1000, 1024, 8192}) {
      std::vector<int> cnt(total, 0);
      for (int b = 0; b < G; ++b) {
        int last = -1;
        for (int k = 0;; ++k) {
          const int id = persistent_item(b, G, k, total);
          if (id < 0) break;
          CHECK(id > last && id % 8 == b % 8, "persistent ids must rise and stay on the XCD");
          last = id;
          ++cnt[id];
        }
        // nothing valid comes after the first id past the end
        for (int k = 0; k < 4 * (total / G + 2); ++k) {
          const int r = k * (G / 8) + ((k & 1) ? G / 8 - 1 - b / 8 : b / 8);
          if (8LL * r + b % 8 >= total) {
            for (int k2 = k + 1; k2 < k + 4; ++k2)
              CHECK(persistent_item(b, G, k2, total) < 0, "persistent item after the end");
            break;
          }
        }
      }
      for (int id = 0; id < total; ++id) CHECK(cnt[id] == 1, "persistent item %d run %d times", id, cnt[id]);
    }
  std::printf("persistent work-group order: checked\n");
  for (int ntiles = 1; ntiles <= 12; ++ntiles)
    for (int nw = 0; nw <= ntiles; ++nw)
      for (int one = 0; one < 2; ++one) check_pingpong(ntiles, nw, one != 0);
  CHECK(pp_one_barrier<128> && !pp_one_barrier<64>, "schedule form per head size");
  std::printf("ping-pong schedules (one and two barriers per step): ntiles 1..12, every wave tile count: checked\n");
  const int shapes[][3] = {{1, 1, 1}, {1, 1, 7}, {1, 1, 64}, {1, 1, 127}, {1, 1, 128},
                           {1, 1, 129}, {1, 2, 200}, {2, 3, 255}, {2, 3, 300}, {1, 1, 1000},
                           {1, 16, 1024}, {1, 1, 4097}};
  for (auto& s : shapes)
    for (int causal = 0; causal < 2; ++causal) {
      check_global<Cfg4<64>>(s[0], s[1], s[2], causal);
      check_global<Cfg4<128>>(s[0], s[1], s[2], causal);
      check_global<Cfg8<64>>(s[0], s[1], s[2], causal);
      check_global<Cfg8<128>>(s[0], s[1], s[2], causal);
      check_global<CfgSplitG>(s[0], s[1], s[2], causal);
      check_global<CfgOcc>(s[0], s[1], s[2], causal);
    }
  check_lengths<Cfg4<64>>();
  check_lengths<Cfg4<128>>();
  check_lengths<Cfg8<64>>();
  check_lengths<Cfg8<128>>();
  check_lengths<CfgSplitG>();
  check_lengths<CfgOcc>();
  std::printf("query/key length pairs (bottom-right causal), padded rows: checked\n");
  // full-size shapes (O coverage tracked up to 64M elements)
  check_global<Cfg4<64>>(1, 16, 1024, true);
  check_global<Cfg8<64>>(10, 64, 1024, false);
  check_global<CfgOcc>(10, 64, 1024, false);
  check_global<CfgSplitG>(1, 16, 1024, true);
  check_global<Cfg8<128>>(2, 16, 8192, true);
  check_global<Cfg8<128>>(1, 8, 16384, true);
  check_global<Cfg4<128>>(1, 1, 65536, true);
  check_global<Cfg8<128>>(1, 1, 65536, true);
  // interleaved eight-wave work-group (the 8-bit kernel's body)
  for (int ntiles = 1; ntiles <= 40; ++ntiles) check_il_schedule(ntiles);
  std::printf("interleaved schedule: ntiles 1..40: checked\n");
  for (int ntiles = 1; ntiles <= 40; ++ntiles) check_two_stage(ntiles);
  std::printf("two-stage schedule: ntiles 1..40: checked\n");
  // 8-bit kernels (ping-pong with 128-key tiles, interleaved with 64-key tiles)
  check_lds8<CfgF8>();
  check_lds8<CfgF8i>();
  check_lds8<CfgF8h>();
  for (auto& s : shapes)
    for (int causal = 0; causal < 2; ++causal) {
      check_global8<CfgF8>(s[0], s[1], s[2], s[2], causal);
      check_global8<CfgF8i>(s[0], s[1], s[2], s[2], causal);
      check_global8<CfgF8h>(s[0], s[1], s[2], s[2], causal);
    }
  {
    const int lens[] = {1, 31, 64, 127, 128, 129, 255, 256, 257, 513};
    for (int lq : lens)
      for (int lk : lens)
        for (int causal = 0; causal < 2; ++causal) {
          check_global8<CfgF8>(1, 2, lq, lk, causal != 0, 128 + 32, 256 + 64);
          check_global8<CfgF8i>(1, 2, lq, lk, causal != 0, 128 + 32, 256 + 64);
          check_global8<CfgF8h>(1, 2, lq, lk, causal != 0, 64 + 48, 128 + 16);
        }
  }
  check_global8<CfgF8>(2, 16, 8192, 8192, true);
  check_global8<CfgF8i>(2, 16, 8192, 8192, true);
  check_global8<CfgF8h>(10, 64, 1024, 1024, false);
  std::printf("8-bit kernel: shapes, length pairs, full size: checked\n");
  if (g_err) {
    std::printf("FAILED with %d errors\n", g_err);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
