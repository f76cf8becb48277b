// Host-side argument checks of the attention-forward library (fa_validate.h),
// built with an ordinary C++ compiler and run under AddressSanitizer and
// UndefinedBehaviorSanitizer (signed overflow, shifts, out-of-bounds): the
// directed cases below, then a fuzz over extreme sizes and strides. Every
// call must return a defined status; an accepted problem must fit the limits
// the kernels rely on (recomputed here in 128-bit arithmetic).
#include <climits>
#include <cstdio>
#include <random>

#include "../../exact_attention_16_amd/csrc/fa_validate.h"

using namespace fa;

static int g_err = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      ++g_err;                                  \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                 \
      std::printf("\n");                        \
    }                                           \
  } while (0)

// fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
static const uintptr_t kBase = 0x100000000000ull, kGap = 1ull << 44;
static void* ptr(int i) { return (void*)(kBase + (uintptr_t)i * kGap); }

static bool valid_status(int r) { return r <= 0 && r >= -9; }

// An accepted strided problem: every tensor's last element within 2^40
// elements of its base, each (sequence, head) under 2^31 bytes.
static void check_accepted(const Problem& P, int B, int H, int Sq, int Sk, int D) {
  const __int128 lastq = (__int128)(B - 1) * P.qb + (__int128)(H - 1) * P.qh + (__int128)(Sq - 1) * P.qs + D;
  const __int128 lasto = (__int128)(B - 1) * P.ob + (__int128)(H - 1) * P.oh + (__int128)(Sq - 1) * P.os + D;
  const __int128 lastk = Sk > 0 ? (__int128)(B - 1) * P.kb + (__int128)(H - 1) * P.kh + (__int128)(Sk - 1) * P.ks + D : 0;
  CHECK(lastq <= ((__int128)1 << 40) && lasto <= ((__int128)1 << 40), "accepted span too large");
  CHECK(lastk >= 0 && lastk < ((__int128)1 << 63), "accepted key span overflows");
  CHECK((__int128)Sq * P.qs * 2 < ((__int128)1 << 31) && (__int128)Sk * P.ks * 2 < ((__int128)1 << 31),
        "accepted head over 32-bit offsets");
  CHECK(P.qs >= D && P.ks >= D && P.vs >= D && P.os >= D, "row stride below D");
}

int main() {
  Problem P;
  bool empty;
  // ---- directed cases
  CHECK(make_dense(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), 2, 16, 8192, 128, 1,
                   0.088f, FA_BF16, &empty) == FA_OK && !empty, "dense long workload");
  CHECK(make_dense(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), INT_MAX, INT_MAX, INT_MAX,
                   128, 1, 0.1f, FA_F16, &empty) == FA_ERR_DIM, "huge dense sizes");
  CHECK(make_dense(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), 1, 1 << 20, 1 << 20, 128,
                   0, 0.1f, FA_F16, &empty) == FA_ERR_DIM, "dense H*S*D over 2^40");
  {
    long long st[14];
    dense_strides(st, 3, 100, 64);
    st[1] = 1LL << 62;  // q head stride: (H - 1) * 2^62 overflows 64 bits
    CHECK(make_fixed(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), 2, 3, 100, 100, 64, 1,
                     0.125f, FA_F16, st, &empty) == FA_ERR_DIM, "2^62 head stride");
    st[1] = LLONG_MAX;
    CHECK(make_fixed(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), 2, 3, 100, 100, 64, 1,
                     0.125f, FA_F16, st, &empty) == FA_ERR_DIM, "LLONG_MAX stride");
    st[1] = LLONG_MIN;
    CHECK(make_fixed(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), 2, 3, 100, 100, 64, 1,
                     0.125f, FA_F16, st, &empty) == FA_ERR_LAYOUT, "LLONG_MIN stride");
  }
  CHECK(make_kt(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), INT_MAX, INT_MAX, 1 << 20, 128,
                0, 0.1f, FA_BF16, &empty) == FA_ERR_DIM, "huge transposed-K sizes");
  CHECK(make_fp8(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), INT_MAX, INT_MAX, 1 << 20, 128,
                 0, 0.1f, 1.f, 1.f, 1.f, &empty) == FA_ERR_DIM, "huge 8-bit sizes");
  {
    const long long st[9] = {1LL << 62, 1LL << 62, 64, 128, 64, 128, 64, 128, 50};
    CHECK(make_varlen(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), (const int*)ptr(5),
                      (const int*)ptr(6), 4, 3, 20, 30, 50, 60, 64, 1, 0.125f, FA_F16, st,
                      &empty) == FA_ERR_DIM, "varlen 2^62 strides");
  }
  // ---- fuzz: sizes and strides from a set of extremes and random values
  std::mt19937_64 rng(20261202);
  const long long llx[] = {0, 1, 8, 64, 128, 1LL << 20, 1LL << 31, 1LL << 40, (1LL << 40) + 8,
                           1LL << 41, 1LL << 62, LLONG_MAX, -8, LLONG_MIN};
  const int ix[] = {0, 1, 2, 7, 64, 100, 129, 1 << 16, 1 << 20, 1 << 30, INT_MAX, -1, INT_MIN};
  auto pick_i = [&]() -> int {
    return (rng() & 1) ? ix[rng() % (sizeof ix / sizeof ix[0])] : (int)(rng() % 4096);
  };
  auto pick_ll = [&]() -> long long {
    const int m = (int)(rng() % 3);
    if (m == 0) return llx[rng() % (sizeof llx / sizeof llx[0])];
    if (m == 1) return (long long)(rng() % 65536) * 8;
    return (long long)(rng() >> (rng() % 64));
  };
  long long accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    const bool near = it % 3 == 0;  // a valid layout with a few strides replaced
    const int B = near ? 1 + (int)(rng() % 4) : pick_i(), H = near ? 1 + (int)(rng() % 8) : pick_i();
    const int Sq = near ? 1 + (int)(rng() % 3000) : pick_i(), Sk = near ? (int)(rng() % 3000) : pick_i();
    const int D = (rng() & 1) ? 64 : 128;
    long long st[14];
    if (near) {
      const long long qh = (long long)Sq * D, kh = (long long)(Sk > 0 ? Sk : 1) * D;
      const long long d[14] = {H * qh, qh, D, H * kh, kh, D, H * kh, kh, D, H * qh, qh, D,
                               (long long)H * Sq, Sq};
      for (int i = 0; i < 14; ++i) st[i] = d[i];
      for (int n = (int)(rng() % 3); n > 0; --n) st[rng() % 14] = pick_ll();
    } else {
      for (long long& x : st) x = pick_ll();
    }
    int r = make_fixed(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), B, H, Sq, Sk, D,
                       (int)(rng() % 2), 0.1f, (int)(rng() % 2), st, &empty);
    CHECK(valid_status(r), "make_fixed status %d", r);
    if (r == FA_OK && !empty) {
      ++accepted;
      check_accepted(P, B, H, Sq, Sk, D);
    }
    r = make_dense(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), B, H, Sq, D, 1, 0.1f,
                   FA_BF16, &empty);
    CHECK(valid_status(r), "make_dense status %d", r);
    if (r == FA_OK && !empty) check_accepted(P, B, H, Sq, Sq, D);
    r = make_kt(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), B, H, Sq, D, 0, 0.1f, FA_F16,
                &empty);
    CHECK(valid_status(r), "make_kt status %d", r);
    r = make_fp8(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), B, H, Sq, D, 1, 0.1f, 0.5f,
                 2.f, 1.f, &empty);
    CHECK(valid_status(r), "make_fp8 status %d", r);
    const long long vst[9] = {st[0], st[1], st[2], st[3], st[4], st[5], st[6], st[7], st[8]};
    r = make_varlen(&P, ptr(0), ptr(1), ptr(2), ptr(3), (float*)ptr(4), (const int*)ptr(5),
                    (const int*)ptr(6), B, H, Sq, Sk, pick_i(), pick_i(), D, 1, 0.1f, FA_BF16, vst,
                    &empty);
    CHECK(valid_status(r), "make_varlen status %d", r);
  }
  std::printf("fuzz: 200000 iterations, %lld strided problems accepted\n", accepted);
  CHECK(accepted > 0, "the fuzz never produced an accepted problem");
  if (g_err) {
    std::printf("FAILED with %d errors\n", g_err);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
