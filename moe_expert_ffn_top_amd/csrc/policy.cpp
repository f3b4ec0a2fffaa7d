// Hot/cold swap planning on the host.
//
// [Strata] "哪些专家能长期留在显存？" (the passages on heat and candidate pairs):
// inside one layer the hottest experts outside the cache are paired with the
// coldest inside; a pair whose heat gap reaches the threshold is a swap
// candidate; the candidates go by gap, at most max_swaps a round.  Pairs are
// formed in heat order (ties to the lower expert index) and a layer stops at
// its first pair below the threshold; equal gaps go by (layer, pair index);
// the shared expert (column E) never swaps.  Heats are the device's fp32
// values and every comparison is taken in fp32.
#include <algorithm>
#include <vector>

#include "moe_common.hpp"

namespace moe {

int plan_swaps(const moe_dims& d, const float* heat, const int32_t* table, float threshold, int32_t max_swaps,
               int32_t* plan) {
  struct Cand {
    float gap;
    int layer, pair, hot, cold;
  };
  std::vector<Cand> cands;
  const int E = d.E, E1 = d.E + 1;
  std::vector<int> out, in;
  for (int l = 0; l < d.L; l++) {
    const float* h = heat + (int64_t)l * E;
    out.clear();
    in.clear();
    for (int e = 0; e < E; e++) (table[(int64_t)l * E1 + e] < 0 ? out : in).push_back(e);
    std::sort(out.begin(), out.end(), [&](int a, int b) { return h[a] != h[b] ? h[a] > h[b] : a < b; });
    std::sort(in.begin(), in.end(), [&](int a, int b) { return h[a] != h[b] ? h[a] < h[b] : a < b; });
    const size_t n = std::min(out.size(), in.size());
    for (size_t i = 0; i < n; i++) {
      const float gap = h[out[i]] - h[in[i]];
      if (!(gap >= threshold)) break;
      cands.push_back({gap, l, (int)i, out[i], in[i]});
    }
  }
  std::sort(cands.begin(), cands.end(), [](const Cand& a, const Cand& b) {
    if (a.gap != b.gap) return a.gap > b.gap;
    if (a.layer != b.layer) return a.layer < b.layer;
    return a.pair < b.pair;
  });
  const int n = (int)std::min<size_t>(cands.size(), (size_t)std::max(0, max_swaps));
  for (int i = 0; i < n; i++) {
    plan[3 * i] = cands[i].layer;
    plan[3 * i + 1] = cands[i].hot;
    plan[3 * i + 2] = cands[i].cold;
  }
  return n;
}

}  // namespace moe
