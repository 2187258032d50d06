// Compute-balanced packing of staircase trajectories (host code).
//
// "On-Policy Residual Learning for Diffusion Language Models" (paper cards
// page, abstract and Figure 3 caption; thread page, Insight 3): captured
// trajectories are packed and balanced by compute across GPUs (or across the
// micro-batches of one GPU) before replay.  The cost of a trajectory is the
// number of (query, key) pairs its attention admits per query head, in closed
// form from its length L, copies S and block size B (P = L - S B):
//   prefix of n = P / B whole blocks and r = P % B tokens:
//     B^2 n (n + 1) / 2 + r (n B + r)
//   S copies of one block, each seeing the prefix and itself:  S B (P + B)
// and, for a general trajectory staircase whose copies come in groups (group
// g: c_g copies of the block that starts at clean position pe_g, each seeing
// the clean keys [0, pe_g) and itself), sum over groups of c_g B (pe_g + B)
// in place of the last term.
// Forward and backward FLOPs are both proportional to it.  Trajectories are
// assigned greedily in order of decreasing cost (ties: lower index first) to
// the bin with the least cost so far (ties: lower bin first) -- the
// longest-processing-time rule, whose largest bin is within 4/3 - 1/(3 nbins)
// of the best possible.
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/bca.h"

namespace {

thread_local char g_pack_error[256] = "";

bca_status_t pack_fail(bca_status_t st, const char* msg, long long a, long long b) {
  snprintf(g_pack_error, sizeof(g_pack_error), msg, a, b);
  return st;
}

}  // namespace

extern "C" {

int64_t bca_trajectory_cost(int32_t seqlen, int32_t s_copies, int32_t block_size) {
  if (seqlen < 0 || s_copies < 0 || block_size < 1) return -1;
  const int64_t L = seqlen, S = s_copies, B = block_size;
  const int64_t P = L - S * B;
  if (P < 0 || (S > 0 && P % B != 0)) return -1;
  const int64_t n = P / B, r = P % B;
  return B * B * n * (n + 1) / 2 + r * (n * B + r) + S * B * (P + B);
}

int64_t bca_trajectory_cost_groups(int32_t seqlen, const int32_t* group_pe,
                                   const int32_t* group_copies, int32_t ngroups,
                                   int32_t block_size) {
  if (seqlen < 0 || ngroups < 0 || block_size < 1) return -1;
  if (ngroups > 0 && (!group_pe || !group_copies)) return -1;
  const int64_t L = seqlen, B = block_size;
  int64_t S = 0;
  for (int32_t g = 0; g < ngroups; ++g) {
    if (group_copies[g] < 0) return -1;
    S += group_copies[g];
  }
  const int64_t P = L - S * B;
  if (P < 0 || (S > 0 && P % B != 0)) return -1;
  const int64_t n = P / B, r = P % B;
  int64_t cost = B * B * n * (n + 1) / 2 + r * (n * B + r);
  int64_t prev = 0;
  for (int32_t g = 0; g < ngroups; ++g) {
    const int64_t pe = group_pe[g];
    if (pe < prev || pe > P || pe % B != 0) return -1;
    prev = pe;
    cost += (int64_t)group_copies[g] * B * (pe + B);  // each copy sees [0, pe) and itself
  }
  return cost;
}

}  // extern "C"

namespace {

// Longest-processing-time assignment of items with the given costs (all
// >= 0) to nbins bins, with the conventions of bca_pack_balanced.
void lpt_assign(const std::vector<int64_t>& cost, int32_t nbins, int32_t* bin_of,
                int64_t* bin_cost, int32_t* order, int32_t* bin_start) {
  const int32_t ntraj = (int32_t)cost.size();
  std::vector<int32_t> by_cost(ntraj);
  std::iota(by_cost.begin(), by_cost.end(), 0);
  std::stable_sort(by_cost.begin(), by_cost.end(),
                   [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
  for (int32_t b = 0; b < nbins; ++b) bin_cost[b] = 0;
  std::vector<int32_t> count(nbins, 0);
  for (int32_t t : by_cost) {
    int32_t best = 0;
    for (int32_t b = 1; b < nbins; ++b)
      if (bin_cost[b] < bin_cost[best]) best = b;
    bin_of[t] = best;
    bin_cost[best] += cost[t];
    ++count[best];
  }
  // members of each bin, in assignment order (costliest first)
  bin_start[0] = 0;
  for (int32_t b = 0; b < nbins; ++b) bin_start[b + 1] = bin_start[b] + count[b];
  std::vector<int32_t> fill(bin_start, bin_start + nbins);
  for (int32_t t : by_cost) order[fill[bin_of[t]]++] = t;
}

// The packing entry points' bodies (their wrappers turn a failed host
// allocation into a status: no exception crosses the C ABI).
bca_status_t pack_balanced_impl(const int32_t* seqlens, const int32_t* s_copies, int32_t ntraj,
                                int32_t block_size, int32_t nbins, int32_t* bin_of,
                                int64_t* bin_cost, int32_t* order, int32_t* bin_start) {
  g_pack_error[0] = '\0';
  if (ntraj < 0 || nbins < 1 || block_size < 1)
    return pack_fail(BCA_ERR_SHAPE, "need ntraj >= 0 (%lld), nbins >= 1 (%lld), block_size >= 1",
                     ntraj, nbins);
  if (ntraj > 0 && (!seqlens || !bin_of || !order))
    return pack_fail(BCA_ERR_NULL, "a required pointer is NULL", 0, 0);
  if (!bin_cost || !bin_start) return pack_fail(BCA_ERR_NULL, "a required pointer is NULL", 0, 0);
  std::vector<int64_t> cost(ntraj);
  for (int32_t t = 0; t < ntraj; ++t) {
    const int32_t S = s_copies ? s_copies[t] : 0;
    cost[t] = bca_trajectory_cost(seqlens[t], S, block_size);
    if (cost[t] < 0)
      return pack_fail(BCA_ERR_SHAPE, "trajectory %lld: bad length %lld for its copies and block size",
                       t, seqlens[t]);
  }
  lpt_assign(cost, nbins, bin_of, bin_cost, order, bin_start);
  return BCA_OK;
}

bca_status_t pack_balanced_groups_impl(const int32_t* seqlens, const int32_t* group_start,
                                       const int32_t* group_pe, const int32_t* group_copies,
                                       int32_t ntraj, int32_t block_size, int32_t nbins,
                                       int32_t* bin_of, int64_t* bin_cost, int32_t* order,
                                       int32_t* bin_start) {
  g_pack_error[0] = '\0';
  if (ntraj < 0 || nbins < 1 || block_size < 1)
    return pack_fail(BCA_ERR_SHAPE, "need ntraj >= 0 (%lld), nbins >= 1 (%lld), block_size >= 1",
                     ntraj, nbins);
  if (ntraj > 0 && (!seqlens || !group_start || !bin_of || !order))
    return pack_fail(BCA_ERR_NULL, "a required pointer is NULL", 0, 0);
  if (!bin_cost || !bin_start) return pack_fail(BCA_ERR_NULL, "a required pointer is NULL", 0, 0);
  std::vector<int64_t> cost(ntraj);
  for (int32_t t = 0; t < ntraj; ++t) {
    const int32_t g0 = group_start[t], g1 = group_start[t + 1];
    if (g0 < 0 || g1 < g0)
      return pack_fail(BCA_ERR_SHAPE, "trajectory %lld: group_start does not increase (%lld)", t,
                       g1);
    if (g1 > g0 && (!group_pe || !group_copies))
      return pack_fail(BCA_ERR_NULL, "group_pe and group_copies are required", 0, 0);
    cost[t] = bca_trajectory_cost_groups(seqlens[t], g1 > g0 ? group_pe + g0 : nullptr,
                                         g1 > g0 ? group_copies + g0 : nullptr, g1 - g0,
                                         block_size);
    if (cost[t] < 0)
      return pack_fail(BCA_ERR_SHAPE, "trajectory %lld: length %lld does not fit its copy groups",
                       t, seqlens[t]);
  }
  lpt_assign(cost, nbins, bin_of, bin_cost, order, bin_start);
  return BCA_OK;
}

}  // namespace

extern "C" {

bca_status_t bca_pack_balanced(const int32_t* seqlens, const int32_t* s_copies, int32_t ntraj,
                               int32_t block_size, int32_t nbins, int32_t* bin_of,
                               int64_t* bin_cost, int32_t* order, int32_t* bin_start) {
  try {
    return pack_balanced_impl(seqlens, s_copies, ntraj, block_size, nbins, bin_of, bin_cost,
                              order, bin_start);
  } catch (const std::bad_alloc&) {
    return pack_fail(BCA_ERR_HOST_MEMORY, "no host memory for %lld trajectories in %lld bins",
                     ntraj, nbins);
  }
}

bca_status_t bca_pack_balanced_groups(const int32_t* seqlens, const int32_t* group_start,
                                      const int32_t* group_pe, const int32_t* group_copies,
                                      int32_t ntraj, int32_t block_size, int32_t nbins,
                                      int32_t* bin_of, int64_t* bin_cost, int32_t* order,
                                      int32_t* bin_start) {
  try {
    return pack_balanced_groups_impl(seqlens, group_start, group_pe, group_copies, ntraj,
                                     block_size, nbins, bin_of, bin_cost, order, bin_start);
  } catch (const std::bad_alloc&) {
    return pack_fail(BCA_ERR_HOST_MEMORY, "no host memory for %lld trajectories in %lld bins",
                     ntraj, nbins);
  }
}

const char* bca_pack_last_error(void) { return g_pack_error; }

}  // extern "C"
