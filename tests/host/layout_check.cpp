// Host-side checker of the attention kernel's index math (fa_layout.h).
//
// Enumerates, for every lane of every wave, every LDS access the kernel makes
// per KV tile and every global access for a list of problem shapes, and
// checks: bounds and alignment; that the staging stores cover each LDS byte
// of a stage exactly once; that each operand read returns the element the
// MFMA lane mapping expects (tracked by tagging every stored element); that
// the work decomposition visits each (Q tile, head) once; and the worst LDS
// bank-conflict degree of each access pattern under a 64-bank (16 lanes per
// 16-byte access cycle) and a 32-bank (8 lanes per cycle) model.
//
// Prints one line per finding and "OK" at the end; exits non-zero on error.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "../../exact_attention_16_amd/csrc/fa_layout.h"

using namespace fa;

static int g_err = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      if (g_err < 20) {                           \
        std::printf("ERROR %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                 \
        std::printf("\n");                        \
      }                                           \
      ++g_err;                                    \
    }                                             \
  } while (0)

// Conflict degree of one wave-wide access of `bytes` per lane.
static int conflict_degree(const std::vector<uint32_t>& addr, int bytes, int banks) {
  const int lanes_per_cycle = banks * 4 / bytes;  // bytes per cycle / bytes per lane
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

template <int D>
static void check_lds() {
  using L = Lds<D>;
  constexpr int BN = L::BN;
  // tag[byte] = element id stored there (key*D + d for K; 1<<24 | key*D + d for V)
  std::vector<long> tag(L::stageBytes, -1);
  // ---- K staging
  int kw_worst[2] = {1, 1};
  for (int wave = 0; wave < kWaves; ++wave)
    for (int n = 0; n < L::kChunksPerThread; ++n) {
      std::vector<uint32_t> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int idx = wave * 64 + lane + n * kThreads;
        int key, ch;
        k_stage_map<D>(idx, &key, &ch);
        const uint32_t off = k_write_off<D>(idx);
        addr[lane] = off;
        CHECK(off % 16 == 0 && off + 16 <= (uint32_t)L::kBytes, "K write off %u", off);
        for (int e = 0; e < 8; ++e)
          for (int b = 0; b < 2; ++b) {
            const uint32_t p = off + 2 * e + b;
            if (p >= (uint32_t)L::stageBytes) continue;
            CHECK(tag[p] == -1, "K byte %u written twice", p);
            tag[p] = (long)key * D + 8 * ch + e;
          }
      }
      kw_worst[0] = std::max(kw_worst[0], conflict_degree(addr, 16, 64));
      kw_worst[1] = std::max(kw_worst[1], conflict_degree(addr, 16, 32));
    }
  // ---- V^T staging (8-byte stores of 4 keys of one d)
  int vw_worst[2] = {1, 1};
  for (int wave = 0; wave < kWaves; ++wave)
    for (int n = 0; n < L::vUnitsPerThread; ++n)
      for (int dd = 0; dd < 8; ++dd) {
        std::vector<uint32_t> addr(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int u = wave * 64 + lane + n * kThreads;
          int kg, dc;
          v_stage_map<D>(u, &kg, &dc);
          const uint32_t off = vt_write_off<D>(u, dd);
          addr[lane] = off;
          CHECK(off % 8 == 0 && off >= (uint32_t)L::kBytes && off + 8 <= (uint32_t)L::stageBytes,
                "V write off %u", off);
          for (int q4 = 0; q4 < 4; ++q4)
            for (int b = 0; b < 2; ++b) {
              const uint32_t p = off + 2 * q4 + b;
              if (p >= (uint32_t)L::stageBytes) continue;
              CHECK(tag[p] == -1, "V byte %u written twice", p);
              tag[p] = (1L << 24) | ((long)(4 * kg + q4) * D + 8 * dc + dd);
            }
        }
        vw_worst[0] = std::max(vw_worst[0], conflict_degree(addr, 8, 64));
        vw_worst[1] = std::max(vw_worst[1], conflict_degree(addr, 8, 32));
      }
  for (int p = 0; p < L::stageBytes; ++p) CHECK(tag[p] != -1, "LDS byte %d never written", p);

  // ---- S^T operand reads: lane must get K[key = 32kb + row_perm32(i)][d = 16j + 8hh + e]
  int kr_worst[2] = {1, 1};
  for (int kb = 0; kb < BN / 32; ++kb)
    for (int j = 0; j < D / 16; ++j) {
      std::vector<uint32_t> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t off = k_read_off<D>(kb, j, lane);
        addr[lane] = off;
        CHECK(off % 16 == 0 && off + 16 <= (uint32_t)L::kBytes, "K read off %u", off);
        const int key = 32 * kb + row_perm32(lane & 31);
        for (int e = 0; e < 8; ++e)
          CHECK(tag[off + 2 * e] == (long)key * D + 16 * j + 8 * (lane >> 5) + e,
                "K read kb=%d j=%d lane=%d e=%d got %ld", kb, j, lane, e, tag[off + 2 * e]);
      }
      kr_worst[0] = std::max(kr_worst[0], conflict_degree(addr, 16, 64));
      kr_worst[1] = std::max(kr_worst[1], conflict_degree(addr, 16, 32));
    }
  // ---- O^T operand reads: lane must get V[key = 16kc + 8hh + e][d = 32jd + row_perm32(i)]
  int vr_worst[2] = {1, 1};
  for (int jd = 0; jd < D / 32; ++jd)
    for (int kc = 0; kc < BN / 16; ++kc) {
      std::vector<uint32_t> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t off = vt_read_off<D>(jd, kc, lane);
        addr[lane] = off;
        CHECK(off % 16 == 0 && off >= (uint32_t)L::kBytes && off + 16 <= (uint32_t)L::stageBytes,
              "V read off %u", off);
        const int d = 32 * jd + row_perm32(lane & 31);
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * kc + 8 * (lane >> 5) + e;
          CHECK(tag[off + 2 * e] == ((1L << 24) | ((long)key * D + d)),
                "V read jd=%d kc=%d lane=%d e=%d", jd, kc, lane, e);
        }
      }
      vr_worst[0] = std::max(vr_worst[0], conflict_degree(addr, 16, 64));
      vr_worst[1] = std::max(vr_worst[1], conflict_degree(addr, 16, 32));
    }
  // ---- accumulator -> P operand: element r of lane half hh is key acc_key32(r, hh);
  // MFMA row rho = 8(r/4) + 4hh + r%4 of S^T was supplied by K row row_perm32(rho).
  for (int hh = 0; hh < 2; ++hh)
    for (int r = 0; r < 16; ++r) {
      const int rho = 8 * (r / 4) + 4 * hh + (r % 4);
      CHECK(row_perm32(rho) == acc_key32(r, hh), "acc key r=%d hh=%d", r, hh);
      // P operand of the 16-key chunk g = r/8 takes elements 8g..8g+7 = keys 16g + 8hh + e
      CHECK(acc_key32(r, hh) == 16 * (r / 8) + 8 * hh + (r % 8), "P operand key");
    }
  for (int r = 0; r < 32; ++r) CHECK(row_perm32(row_perm32(r)) == r, "perm involution");

  std::printf("D=%d BN=%d stage=%d B: conflict degree (64 banks / 32 banks): "
              "K read %d/%d, V^T read %d/%d, K write %d/%d, V^T write %d/%d\n",
              D, BN, L::stageBytes, kr_worst[0], kr_worst[1], vr_worst[0], vr_worst[1],
              kw_worst[0], kw_worst[1], vw_worst[0], vw_worst[1]);
  CHECK(kr_worst[0] == 1 && kr_worst[1] == 1, "K operand reads conflict");
  CHECK(vr_worst[0] == 1 && vr_worst[1] == 1, "V^T operand reads conflict");
  CHECK(kw_worst[0] == 1, "K staging writes conflict");
  CHECK(vw_worst[0] <= 2, "V^T staging writes conflict more than 2-way");
}

template <int D>
static void check_global(int B, int H, int S, bool causal) {
  const int BH = B * H;
  const int nqt = num_q_tiles(S);
  const long grid = (long)nqt * BH;
  constexpr int BN = TileCfg<D>::BN;
  std::vector<char> seen(grid, 0);
  const size_t head_elems = (size_t)S * D;
  std::vector<char> owritten(std::min<size_t>(head_elems * (size_t)BH, (size_t)1 << 26), 0);
  const bool track = head_elems * (size_t)BH <= owritten.size();
  for (long bid = 0; bid < grid; ++bid) {
    int qt, bh;
    block_to_tile((int)bid, BH, nqt, causal, &qt, &bh);
    CHECK(qt >= 0 && qt < nqt && bh >= 0 && bh < BH, "tile map bid=%ld", bid);
    const long cell = (long)qt * BH + bh;
    CHECK(!seen[cell], "tile visited twice");
    seen[cell] = 1;
    const int kv_end = tile_kv_end(qt, S, causal);
    const int ntiles = (kv_end + BN - 1) / BN;
    CHECK(ntiles >= 1 && (ntiles - 1) * BN < S, "tile count");
    for (int t = 0; t < ntiles; ++t)
      for (int tid = 0; tid < kThreads; ++tid) {
        for (int n = 0; n < Lds<D>::kChunksPerThread; ++n) {
          int key, ch;
          k_stage_map<D>(tid + n * kThreads, &key, &ch);
          const size_t off = kv_chunk_off<D>(kv_row(t * BN, key, S), ch);
          CHECK(off + 8 <= head_elems, "K load out of bounds");
        }
        for (int n = 0; n < Lds<D>::vUnitsPerThread; ++n) {
          int kg, dc;
          v_stage_map<D>(tid + n * kThreads, &kg, &dc);
          for (int q4 = 0; q4 < 4; ++q4) {
            const size_t off = kv_chunk_off<D>(kv_row(t * BN, 4 * kg + q4, S), dc);
            CHECK(off + 8 <= head_elems, "V load out of bounds");
          }
        }
      }
    for (int wave = 0; wave < kWaves; ++wave) {
      const int q0w = qt * kBM + wave * kRowsPerWave;
      const int wkv = wave_kv_end(q0w, S, causal);
      if (q0w < S) {
        // every key a row of this wave can see lies in a visited tile
        const int need = causal ? std::min(S, q0w + kRowsPerWave) : S;
        CHECK(wkv == need && wkv <= ntiles * BN, "wave key range");
        CHECK(0 < wkv, "wave must see tile 0");
      }
      for (int lane = 0; lane < 64; ++lane) {
        const int qrow = q0w + (lane & 31), hh = lane >> 5;
        const int qrow_c = qrow < S ? qrow : S - 1;
        for (int j = 0; j < D / 16; ++j)
          CHECK(q_frag_off<D>(qrow_c, j, hh) + 8 <= head_elems, "Q load out of bounds");
        if (q0w < S && qrow < S)
          for (int jd = 0; jd < D / 32; ++jd)
            for (int g = 0; g < 2; ++g) {
              const size_t off = o_frag_off<D>(qrow, jd, g, hh);
              CHECK(off + 8 <= head_elems, "O store out of bounds");
              if (track)
                for (int e = 0; e < 8; ++e) {
                  const size_t p = (size_t)bh * head_elems + off + e;
                  CHECK(!owritten[p], "O element written twice");
                  owritten[p] = 1;
                }
            }
      }
    }
  }
  for (long c = 0; c < grid; ++c) CHECK(seen[c], "tile never visited");
  if (track)
    for (size_t p = 0; p < head_elems * (size_t)BH; ++p) CHECK(owritten[p], "O element not written");
}

int main() {
  check_lds<64>();
  check_lds<128>();
  const int shapes[][3] = {{1, 1, 1}, {1, 1, 7}, {1, 1, 64}, {1, 1, 127}, {1, 1, 128},
                           {1, 1, 129}, {1, 2, 200}, {2, 3, 255}, {1, 1, 1000},
                           {1, 16, 1024}, {1, 1, 4097}};
  for (auto& s : shapes)
    for (int causal = 0; causal < 2; ++causal) {
      check_global<64>(s[0], s[1], s[2], causal);
      check_global<128>(s[0], s[1], s[2], causal);
    }
  // full-size shapes: decomposition and bounds only (O coverage tracked up to 64M elements)
  check_global<64>(1, 16, 1024, true);
  check_global<64>(10, 64, 1024, false);
  check_global<128>(2, 16, 8192, true);
  check_global<128>(1, 8, 16384, true);
  if (g_err) {
    std::printf("FAILED with %d errors\n", g_err);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
