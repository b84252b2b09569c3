// Host-only driver of the C-ABI layer (ssd_api.cpp) for sanitizer builds:
// every kernel launcher and the two HIP runtime calls the layer makes are
// replaced by stubs, so the argument checks, fan-out arithmetic, workspace
// carving and error reporting run on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer. Device pointers are fake, 256-byte aligned
// addresses that the host layer never dereferences. Exits non-zero on the
// first unexpected status.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ssd_internal.hpp"

namespace ssd {
static int g_launches = 0;
hipError_t launch_stats_chunks(const StatsArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_cache(const CacheArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_lookup(const LookupArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_sample(const SampleArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_greedy(const GreedyArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_cache_stats(const CacheStatsArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_tree_stats(const TreeArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_tree_round(const TreeArgs&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_round_chunks(const RoundArgs&, int, hipStream_t, hipEvent_t, hipEvent_t) { ++g_launches; return hipSuccess; }
hipError_t launch_round_resid(const RoundResidArgs&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_rows_resid(const RoundResidArgs&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_round(const RoundArgs&, const RoundResidArgs&, int, hipStream_t, void* const*) {
  g_launches += 3;
  return hipSuccess;
}
}  // namespace ssd

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

static int g_fail = 0;
#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, ssd_last_error()); \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

static void* fake(uintptr_t i) { return reinterpret_cast<void*>((i + 1) << 12); }

// The launchers' magic-number division (make_fastdiv), evaluated as the
// kernels do, against integer division: every divisor up to 4096 with
// dividends near multiples of it and at the ends of [0, 2^31), powers of two
// and a spread of large divisors.
static void check_fastdiv() {
  auto fd = [](uint32_t n, ssd::FastDiv f) {
    return uint32_t(((uint64_t(n) * f.m >> 32) + n) >> f.s);
  };
  auto chk = [&](uint32_t n, uint32_t d, ssd::FastDiv f) {
    if (fd(n, f) != n / d) {
      std::fprintf(stderr, "FAIL fastdiv n=%u d=%u\n", n, d);
      ++g_fail;
    }
  };
  const uint32_t top = 0x7FFFFFFFu;
  uint64_t x = 0x9E3779B97F4A7C15ull;   // xorshift dividends
  auto next = [&]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return uint32_t(x & top); };
  for (uint32_t d = 1; d <= 4096; ++d) {
    const ssd::FastDiv f = ssd::make_fastdiv(d);
    for (uint32_t n = 0; n < 2 * d + 3; ++n) chk(n, d, f);
    for (uint32_t q : {7u, 1000u, top / d - 1}) {
      const uint64_t n0 = uint64_t(q) * d;
      for (int o = -1; o <= 1; ++o)
        if (int64_t(n0) + o >= 0 && int64_t(n0) + o <= int64_t(top)) chk(uint32_t(int64_t(n0) + o), d, f);
    }
    for (int t = 0; t < 64; ++t) chk(next(), d, f);
    chk(top, d, f);
  }
  for (int k = 0; k <= 31; ++k) {
    const uint32_t d = 1u << k;
    const ssd::FastDiv f = ssd::make_fastdiv(d);
    for (int t = 0; t < 256; ++t) chk(next(), d, f);
    chk(top, d, f);
    chk(d - 1, d, f);
    if (d <= top) chk(d, d, f);
  }
  for (int t = 0; t < 200000; ++t) {
    const uint32_t d = 1 + next();
    chk(next(), d, ssd::make_fastdiv(d));
  }
}

int main() {
  check_fastdiv();
  // fan-out: every budget, K and a range of (a_p, r) sums to the budget
  std::vector<int32_t> F(SSD_MAX_K + 1);
  for (int K = 1; K <= SSD_MAX_K; K += 7)
    for (int n = 0; n <= 300; n += 37)
      for (double ap : {0.05, 0.5, 0.8, 0.999})
        for (double r : {-0.9, 0.0, 1.0, 10.0}) {
          const int s = ssd_fanout(n, K, ap, r, F.data());
          EXPECT(s == n);
          long long tot = 0;
          for (int k = 0; k <= K; ++k) {
            EXPECT(F[k] >= 0);
            tot += F[k];
          }
          EXPECT(tot == n);
          EXPECT(ssd_fanout_uniform(n, K, F.data()) == n);
        }
  EXPECT(ssd_fanout(-1, 3, 0.5, 1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 0, 0.5, 1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 65, 0.5, 1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 3, 1.0, 1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 3, NAN, 1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 3, 0.5, -1.0, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 3, 0.5, INFINITY, F.data()) == SSD_EINVAL);
  EXPECT(ssd_fanout(10, 3, 0.5, 1.0, nullptr) == SSD_EINVAL);
  EXPECT(std::strlen(ssd_last_error()) > 0);

  double sp = 0.0;
  EXPECT(ssd_speedup(0.7, 3.0, 2.0, 0.5, 0.2, 4, &sp) == SSD_OK && std::isfinite(sp));
  EXPECT(ssd_speedup(1.5, 3.0, 2.0, 0.5, 0.2, 4, &sp) == SSD_EINVAL);
  EXPECT(ssd_speedup(0.5, 3.0, 2.0, 0.5, 0.2, 0, &sp) == SSD_EINVAL);

  // token-tree topologies: valid chains and stars, invalid parents
  std::vector<int32_t> parent(SSD_MAX_TREE);
  for (int N = 1; N <= SSD_MAX_TREE; N += 9) {
    for (int n = 0; n < N; ++n) parent[n] = n - 1;
    EXPECT(ssd_tree_rounds(parent.data(), N) == 1);
    for (int n = 1; n < N; ++n) parent[n] = 0;
    EXPECT(ssd_tree_rounds(parent.data(), N) == (N > 1 ? N - 1 : 1));
  }
  parent[0] = 0;
  EXPECT(ssd_tree_rounds(parent.data(), 3) == SSD_EINVAL);
  parent[0] = -1;
  parent[2] = 2;
  EXPECT(ssd_tree_rounds(parent.data(), 3) == SSD_EINVAL);
  EXPECT(ssd_tree_rounds(parent.data(), 65) == SSD_EINVAL);

  // workspace queries over many shapes, and each entry point with a valid
  // call (stub launches) and with bad arguments
  for (int B : {1, 7, 64, 4096})
    for (int K : {1, 5, 31, 64})
      for (int V : {1, 8191, 8192, 128256, 1 << 20})
        for (int dt : {SSD_F32, SSD_BF16}) {
          const size_t wv = ssd_verify_workspace_size(B, K, V, dt);
          const size_t wr = ssd_residual_workspace_size(B, K, V, dt);
          const size_t wc = ssd_build_cache_workspace_size(B, K, V, dt);
          const size_t wd = ssd_draft_sample_workspace_size(B, K, V, dt);
          const size_t wg = ssd_verify_greedy_workspace_size(B, K, V, dt);
          const size_t wo = ssd_verify_round_workspace_size(B, K, V, dt);
          EXPECT(wv > 0 && wr > 0 && wc > 0 && wd > 0 && wg > 0 && wo > 0);
          if (int64_t(B) * K * V > (int64_t(1) << 31)) continue;
          void* ws = fake(1 << 20);
          const int Fk = V < 64 ? V : 64;
          std::vector<int32_t> FF(K + 1, Fk > 3 ? 3 : Fk);
          EXPECT(ssd_verify(fake(1), V, fake(2), V, dt, B, K, V, 0.7f, (int32_t*)fake(3), (float*)fake(4),
                            (float*)fake(5), nullptr, (int32_t*)fake(6), (int32_t*)fake(7), nullptr, nullptr,
                            nullptr, ws, wv, nullptr) == SSD_OK);
          EXPECT(ssd_verify(fake(1), V, fake(2), V, dt, B, K, V, 0.7f, (int32_t*)fake(3), (float*)fake(4),
                            (float*)fake(5), nullptr, (int32_t*)fake(6), (int32_t*)fake(7), nullptr, nullptr,
                            nullptr, ws, wv - 1, nullptr) == SSD_EWORKSPACE);
          EXPECT(ssd_verify_round(fake(1), V, fake(2), V, dt, B, K, V, 0.7f, FF.data(), 0.5f, (int32_t*)fake(3),
                                  (float*)fake(4), (float*)fake(5), (int32_t*)fake(8), (ssd_rowkey*)fake(9),
                                  (double*)fake(10), (int32_t*)fake(6), (int32_t*)fake(7), (uint8_t*)fake(11),
                                  nullptr, ws, wo, nullptr) == SSD_OK);
          EXPECT(ssd_build_cache(fake(2), V, dt, B, K, V, 0.7f, FF.data(), (int32_t*)fake(8), (ssd_rowkey*)fake(9),
                                 (double*)fake(10), ws, wc, nullptr) == SSD_OK);
          EXPECT(ssd_residual_sample(fake(1), V, fake(2), V, dt, B, K, V, 0.7f, (int32_t*)fake(3), nullptr,
                                     (float*)fake(5), (int32_t*)fake(6), nullptr, ws, wr, nullptr) == SSD_OK);
          EXPECT(ssd_draft_sample(fake(2), V, dt, B, K, V, 0.7f, nullptr, (float*)fake(4), (int32_t*)fake(6), ws,
                                  wd, nullptr) == SSD_OK);
          EXPECT(ssd_verify_greedy(fake(1), V, dt, B, K, V, (int32_t*)fake(3), (int32_t*)fake(6),
                                   (int32_t*)fake(7), ws, wg, nullptr) == SSD_OK);
        }
  const size_t w = ssd_verify_workspace_size(4, 3, 100, SSD_BF16);
  void* ws = fake(1 << 20);
  auto verify = [&](int B, int K, int V, float tau, int dt, const void* t, const ssd_sigma* sg, void* wsp,
                    size_t wsz) {
    return ssd_verify(t, V, fake(2), V, dt, B, K, V, tau, (int32_t*)fake(3), (float*)fake(4), (float*)fake(5), sg,
                      (int32_t*)fake(6), (int32_t*)fake(7), nullptr, nullptr, nullptr, wsp, wsz, nullptr);
  };
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_OK);
  EXPECT(verify(0, 3, 100, 0.7f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 0, 100, 0.7f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 65, 100, 0.7f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 0, 0.7f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 100, 0.0f, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 100, NAN, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 100, INFINITY, SSD_BF16, fake(1), nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 100, 0.7f, 7, fake(1), nullptr, ws, w) == SSD_EDTYPE);
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, nullptr, nullptr, ws, w) == SSD_EINVAL);
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, fake(1), nullptr, nullptr, w) == SSD_EWORKSPACE);
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, fake(1), nullptr, (char*)ws + 8, w) == SSD_EWORKSPACE);
  ssd_sigma bad{1.5f, (ssd_rowkey*)fake(9), (double*)fake(10)};
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, fake(1), &bad, ws, w) == SSD_EINVAL);
  bad.C = 0.5f;
  bad.thr = nullptr;
  EXPECT(verify(4, 3, 100, 0.7f, SSD_BF16, fake(1), &bad, ws, w) == SSD_EINVAL);
  const int32_t Fbad[4] = {3, 65, 1, 1};
  EXPECT(ssd_build_cache(fake(2), 100, SSD_BF16, 4, 3, 100, 0.7f, Fbad, (int32_t*)fake(8), (ssd_rowkey*)fake(9),
                         (double*)fake(10), ws, ssd_build_cache_workspace_size(4, 3, 100, SSD_BF16),
                         nullptr) == SSD_EINVAL);
  const int32_t Fneg[4] = {3, -1, 1, 1};
  EXPECT(ssd_cache_lookup((int32_t*)fake(8), Fneg, 4, 3, (int32_t*)fake(6), (int32_t*)fake(7),
                          (uint8_t*)fake(11), nullptr, nullptr) == SSD_EINVAL);
  EXPECT(ssd_cache_stats(nullptr, (uint8_t*)fake(11), 4, 3, (uint32_t*)fake(12), nullptr) == SSD_EINVAL);
  EXPECT(ssd_cache_stats((int32_t*)fake(6), (uint8_t*)fake(11), 4, 3, (uint32_t*)fake(12), nullptr) == SSD_OK);
  const int32_t tpar[4] = {-1, 0, 0, 1};
  EXPECT(ssd_verify_tree(fake(1), 100 * 4, fake(2), 100 * 4, SSD_BF16, 4, 4, 100, 0.7f, tpar, (int32_t*)fake(3),
                         (float*)fake(4), (float*)fake(5), (int32_t*)fake(6), (int32_t*)fake(7), nullptr, ws,
                         ssd_verify_tree_workspace_size(4, 4, 100, SSD_BF16), nullptr) == SSD_OK);
  EXPECT(std::strlen(ssd_last_error()) == 0);
  std::printf("host ABI sanitizer driver: %d failures, %d stub launches\n", g_fail, ssd::g_launches);
  return g_fail == 0 ? 0 : 1;
}
