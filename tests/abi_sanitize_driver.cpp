// Host-side driver for the address / undefined-behaviour sanitizer run of the
// C ABI (built and run by tests/test_sanitize_host.py on a machine without a
// GPU).  Every call below either fails validation or has nothing to do, so no
// kernel is launched and no device memory is touched: the fake device
// pointers are never dereferenced.  The packing routines run for real on host
// arrays of random trajectories.  Prints each failed expectation and exits
// non-zero if there was one.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "bca.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    ++g_failures;
    std::printf("line %d: %s (last error: %s)\n", line, what, bca_last_error());
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never dereferenced
float* const FF = reinterpret_cast<float*>(F);
const int32_t* const FI = reinterpret_cast<const int32_t*>(F);

}  // namespace

int main() {
  // housekeeping
  EXPECT(bca_abi_version() == BCA_ABI_VERSION);
  for (int s = -3; s < 12; ++s) EXPECT(std::strlen(bca_status_string((bca_status_t)s)) > 0);
  // forward: every host-checked error, then nothing-to-do calls
  auto fwd = [](const void* q, int nseq, int ms, int total, int hq, int hkv, int d, int B, float sc,
                int dt) {
    return bca_staircase_fwd(q, F, F, F, FF, FI, nullptr, nseq, ms, total, hq, hkv, d, B, sc,
                             (bca_dtype_t)dt, nullptr);
  };
  EXPECT(fwd(F, 1, 64, 64, 32, 8, 96, 32, 0.1f, 1) == BCA_ERR_UNSUPPORTED);
  EXPECT(fwd(F, 1, 64, 64, 6, 4, 128, 32, 0.1f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 64, 64, 32, 0, 128, 32, 0.1f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 64, 64, 32, 8, 128, 0, 0.1f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, -1, 64, 64, 32, 8, 128, 32, 0.1f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 0, 64, 32, 8, 128, 32, 0.1f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 64, 64, 32, 8, 128, 32, -1.f, 1) == BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 64, 64, 32, 8, 128, 32, 0.1f, 7) == BCA_ERR_DTYPE);
  EXPECT(fwd(nullptr, 1, 64, 64, 32, 8, 128, 32, 0.1f, 1) == BCA_ERR_NULL);
  EXPECT(fwd(reinterpret_cast<char*>(F) + 8, 1, 64, 64, 32, 8, 128, 32, 0.1f, 1) ==
         BCA_ERR_SHAPE);
  EXPECT(fwd(F, 1, 64, 1 << 30, 1024, 8, 128, 32, 0.1f, 1) == BCA_ERR_SHAPE);  // too large
  EXPECT(fwd(nullptr, 0, 0, 0, 32, 8, 128, 32, 0.1f, 1) == BCA_OK);
  EXPECT(bca_fwd(F, F, F, F, FF, FI, 1, 64, 64, 32, 8, 100, 32, 0.1f, BCA_BF16, nullptr) ==
         BCA_ERR_UNSUPPORTED);
  EXPECT(bca_staircase_groups_fwd(F, F, F, F, FF, FI, nullptr, FI, FI, 1, 64, 64, 32, 8, 128, 32,
                                  0.1f, BCA_BF16, nullptr) == BCA_ERR_NULL);
  // backward and its stages
  const size_t need = bca_staircase_bwd_workspace(1000, 32, 8, 128);
  EXPECT(need >= 2 * 32 * 1000 * 4);
  EXPECT(bca_staircase_bwd_workspace(-1, 32, 8, 128) == 0);
  EXPECT(bca_staircase_bwd(F, F, F, F, FF, F, F, F, F, FI, nullptr, 1, 1000, 1000, 32, 8, 128, 32,
                           0.1f, BCA_BF16, F, need - 1, nullptr) == BCA_ERR_WORKSPACE);
  EXPECT(bca_staircase_bwd(F, F, F, F, FF, F, F, F, F, FI, nullptr, 1, 1000, 1000, 32, 8, 128, 32,
                           0.1f, BCA_F32, F, need, nullptr) == BCA_ERR_DTYPE);
  EXPECT(bca_staircase_bwd(F, F, F, F, FF, nullptr, F, F, F, FI, nullptr, 1, 1000, 1000, 32, 8,
                           128, 32, 0.1f, BCA_BF16, F, need, nullptr) == BCA_ERR_NULL);
  for (int st : {-1, 4, 1000})
    EXPECT(bca_staircase_bwd_stage(st, F, F, F, F, FF, F, F, F, F, FI, nullptr, 1, 1000, 1000, 32,
                                   8, 128, 32, 0.1f, BCA_BF16, F, need, nullptr) == BCA_ERR_SHAPE);
  for (int st = 0; st < 4; ++st)
    EXPECT(bca_staircase_bwd_stage(st, F, F, F, F, FF, F, F, F, F, FI, nullptr, 0, 0, 0, 32, 8, 128,
                                   32, 0.1f, BCA_BF16, nullptr, 0, nullptr) == BCA_OK);
  EXPECT(bca_staircase_groups_bwd(F, F, F, F, FF, F, F, F, F, FI, nullptr, FI, FI, 1, 64, 64, 32, 8,
                                  128, 32, 0.1f, BCA_BF16, F, need, nullptr) == BCA_ERR_NULL);
  // decode, FP8 decode, no-alloc decode, captured loop
  const size_t dneed = bca_decode_workspace(32, 1056, 32, 8, 128, 0);
  EXPECT(dneed > 0);
  EXPECT(bca_decode_workspace(32, 1056, 32, 8, 128, 1) == 0);
  EXPECT(bca_decode_workspace(0, 1056, 32, 8, 128, 0) == 0);
  EXPECT(bca_decode_workspace(32, 1 << 30, 32, 8, 128, 256) > 0);
  auto dec = [](int ql, int kvl, int hq, int d, float sc, int dt, int ns, void* ws, size_t wb) {
    return bca_decode(F, F, F, F, FF, ql, kvl, hq, 8, d, sc, (bca_dtype_t)dt, ns, ws, wb, nullptr);
  };
  EXPECT(dec(32, 1056, 32, 128, 0.1f, 1, 0, F, dneed - 1) == BCA_ERR_WORKSPACE);
  EXPECT(dec(32, 1056, 32, 128, 0.1f, 1, 0, nullptr, dneed) == BCA_ERR_WORKSPACE);
  EXPECT(dec(32, 16, 32, 128, 0.1f, 1, 0, F, dneed) == BCA_ERR_SHAPE);
  EXPECT(dec(32, 1056, 12, 128, 0.1f, 1, 0, F, dneed) == BCA_ERR_SHAPE);
  EXPECT(dec(32, 1056, 32, 32, 0.1f, 1, 0, F, dneed) == BCA_ERR_UNSUPPORTED);
  EXPECT(dec(32, 1056, 32, 128, 0.0f, 1, 0, F, dneed) == BCA_ERR_SHAPE);
  EXPECT(dec(32, 1056, 32, 128, 0.1f, 0, 0, F, dneed) == BCA_ERR_DTYPE);
  EXPECT(dec(32, 1056, 32, 128, 0.1f, 1, 257, F, dneed) == BCA_ERR_SHAPE);
  EXPECT(bca_decode_fp8(F, F, F, 0.f, 1.f, F, FF, 32, 1056, 32, 8, 128, 0.1f, 0, F, dneed,
                        nullptr) == BCA_ERR_SHAPE);
  EXPECT(bca_decode_noalloc(F, F, F, F, FF, 32, 8224, 32, 8, 128, 0.1f, BCA_BF16, 256, nullptr) ==
         BCA_ERR_WORKSPACE);
  EXPECT(bca_decode_noalloc(F, F, F, F, FF, 32, 8224, 32, 8, 128, 0.1f, BCA_F32, 0, nullptr) ==
         BCA_ERR_DTYPE);
  bca_decode_graph_t* g = reinterpret_cast<bca_decode_graph_t*>(F);
  EXPECT(bca_decode_graph_create(F, F, F, F, FF, 32, 1056, 32, 8, 128, 0.1f, BCA_BF16, 0, F, dneed,
                                 0, &g) == BCA_ERR_SHAPE);
  EXPECT(g == nullptr);
  EXPECT(bca_decode_graph_create(F, F, F, F, FF, 32, 1056, 32, 8, 128, 0.1f, BCA_BF16, 0, nullptr,
                                 dneed, 4, &g) == BCA_ERR_WORKSPACE);
  EXPECT(bca_decode_graph_create(F, F, F, F, FF, 32, 1056, 32, 8, 128, 0.1f, BCA_BF16, 0, F, dneed,
                                 4, nullptr) == BCA_ERR_NULL);
  EXPECT(bca_decode_graph_launch(nullptr, nullptr) == BCA_ERR_NULL);
  const int32_t* len_dev = reinterpret_cast<const int32_t*>(F);
  const int32_t* odd = reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(F) + 2);
  EXPECT(bca_decode_loop_create(F, F, F, F, FF, nullptr, nullptr, 32, 1056, 32, 8, 128, 0.1f,
                                BCA_BF16, 0, F, dneed, 4, &g) == BCA_ERR_NULL);
  EXPECT(g == nullptr);
  EXPECT(bca_decode_loop_create(F, F, F, F, FF, odd, nullptr, 32, 1056, 32, 8, 128, 0.1f,
                                BCA_BF16, 0, F, dneed, 4, &g) == BCA_ERR_SHAPE);
  EXPECT(bca_decode_loop_create(F, F, F, F, FF, len_dev, odd, 32, 1056, 32, 8, 128, 0.1f,
                                BCA_BF16, 0, F, dneed, 4, &g) == BCA_ERR_SHAPE);
  EXPECT(bca_decode_loop_create(F, F, F, F, FF, len_dev, nullptr, 32, 1056, 32, 8, 128, 0.1f,
                                BCA_BF16, 0, F, dneed, 0, &g) == BCA_ERR_SHAPE);
  EXPECT(bca_decode_loop_create(F, F, F, F, FF, len_dev, nullptr, 32, 16, 32, 8, 128, 0.1f,
                                BCA_BF16, 0, F, dneed, 4, &g) == BCA_ERR_SHAPE);
  bca_decode_graph_destroy(nullptr);
  // packing on random host trajectories, plain and with copy groups
  std::mt19937 rng(12345);
  for (int rep = 0; rep < 200; ++rep) {
    const int B = 1 + (int)(rng() % 64), n = (int)(rng() % 40), nbins = 1 + (int)(rng() % 9);
    std::vector<int32_t> len(n), cop(n), gstart(n + 1, 0), gpe, gcp;
    for (int t = 0; t < n; ++t) {
      const int nb = (int)(rng() % 50);
      cop[t] = (int)(rng() % 6);
      len[t] = nb * B + cop[t] * B + (cop[t] == 0 ? (int)(rng() % B) : 0);
      int pe = 0, left = cop[t], placed = 0;
      while (left > 0) {
        const int c = 1 + (int)(rng() % left);
        pe = pe + (int)(rng() % (nb - pe / B + 1)) * B;
        gpe.push_back(pe);
        gcp.push_back(c);
        left -= c;
        ++placed;
      }
      gstart[t + 1] = gstart[t] + placed;
    }
    std::vector<int32_t> bin_of(n), order(n), bin_start(nbins + 1);
    std::vector<int64_t> bin_cost(nbins);
    EXPECT(bca_pack_balanced(len.data(), cop.data(), n, B, nbins, bin_of.data(), bin_cost.data(),
                             order.data(), bin_start.data()) == BCA_OK);
    std::vector<int64_t> cost2(nbins);
    EXPECT(bca_pack_balanced_groups(len.data(), gstart.data(), gpe.data(), gcp.data(), n, B, nbins,
                                    bin_of.data(), cost2.data(), order.data(),
                                    bin_start.data()) == BCA_OK);
    int64_t sum = 0;
    for (int t = 0; t < n; ++t) sum += bca_trajectory_cost(len[t], cop[t], B);
    int64_t s1 = 0;
    for (int b = 0; b < nbins; ++b) s1 += bin_cost[b];
    EXPECT(s1 == sum);
    EXPECT(bin_start[nbins] == n);
  }
  EXPECT(bca_trajectory_cost(10, 3, 4) == -1);
  EXPECT(bca_trajectory_cost_groups(12, nullptr, nullptr, 1, 2) == -1);
  int32_t bo[1], ord[1], bs[3];
  int64_t bc[2];
  const int32_t bad_len[1] = {10}, bad_cop[1] = {3};
  EXPECT(bca_pack_balanced(bad_len, bad_cop, 1, 4, 2, bo, bc, ord, bs) == BCA_ERR_SHAPE);
  EXPECT(std::strlen(bca_pack_last_error()) > 0);
  EXPECT(bca_pack_balanced(bad_len, bad_cop, -1, 4, 2, bo, bc, ord, bs) == BCA_ERR_SHAPE);
  EXPECT(bca_pack_balanced(nullptr, nullptr, 1, 4, 2, bo, bc, ord, bs) == BCA_ERR_NULL);
  std::printf("%s: %d failed expectations\n", g_failures ? "FAIL" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
