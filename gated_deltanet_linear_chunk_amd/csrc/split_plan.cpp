// split_plan.cpp -- host planning of segment splits for packed chunk-rule runs.
//
// The chunk scan is serial along a sequence, so a packed batch whose samples
// differ a lot in length is bounded by its longest sample.  When the offsets
// are known on the host, long samples are cut into chunk-aligned segments
// s_0 .. s_{n-1}.  Pass 1 runs s_0 forward from the sample's start state (its
// outputs, and its end state, which is the true start of s_1) and, beside it,
// the state-only scan of s_1 .. s_{n-2} on the augmented state [M | b] (each
// segment's affine map); an fp32 chain from s_1's start through those maps
// gives the true start of s_2 .. s_{n-1}; pass 2 runs every segment but the
// s_0 of split samples (the unsplit samples whole) from those starts.  This is
// the segment-wise state passing of the segmented entry point applied per
// sample, with the first segment of each chain run in pass 1, where the map
// blocks leave compute units free.  The cut length is chosen with a small
// list-scheduling model of the two passes on the device's compute units;
// nothing is split unless the model expects the run to be at least 15%
// shorter.
#include "split_plan.h"

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>

namespace gdn {

namespace {

// A run of `count` blocks of one duration, dispatched back to back.
struct Group {
  double d;
  int64_t count;
};

// Finish time of the groups' blocks dispatched in order, each block to the
// first free compute unit (one block per unit at a time).  The units are kept
// as (free-at time, number of units) classes, so a group costs one step per
// class it touches rather than one per block.
double makespan(const std::vector<Group>& groups, int cus) {
  std::map<double, int64_t> free_at{{0.0, (int64_t)cus}};
  double end = 0.0;
  for (const Group& g : groups) {
    int64_t left = g.count;
    while (left > 0) {
      auto it = free_at.begin();
      const double t = it->first;
      const int64_t take = std::min(left, it->second);
      if (take == it->second)
        free_at.erase(it);
      else
        it->second -= take;
      free_at[t + g.d] += take;
      end = std::max(end, t + g.d);
      left -= take;
    }
  }
  return end;
}

// The last plans, keyed by everything they depend on: repeated calls with the
// same offsets (a serving loop, a benchmark) skip the search.
struct PlanKey {
  std::vector<int32_t> cu;
  int32_t H_v, V;
  bool has_s0;
  int cus;
  bool operator==(const PlanKey& o) const {
    return H_v == o.H_v && V == o.V && has_s0 == o.has_s0 && cus == o.cus && cu == o.cu;
  }
};
struct CachedPlan {
  PlanKey key;
  bool split;
  SplitPlan plan;
};
constexpr size_t kCacheSize = 8;
std::mutex g_cache_mutex;
std::vector<CachedPlan> g_cache;  // most recent last

}  // namespace

// Upper bound on pass-1 segments: their blocks (K/128 + V/128 per head, the
// launch size of a forward and a map segment alike) fit twice on the
// compute units.
int max_prefix_segments(int32_t H_v, int32_t V, int cus) {
  const int tiles1 = 1 + V / 128;
  return std::max(0, 2 * cus / std::max(1, H_v * tiles1));
}

int64_t split_plan_ints_max(int n_seg, int n_prefix) {
  return 5 * (int64_t)n_seg + 1 + 5 * (int64_t)n_prefix;
}

static bool plan_split_uncached(const int32_t* cu, int32_t N, int32_t H_v, int32_t V, bool has_s0, int cus,
                                SplitPlan& out);

bool plan_split(const int32_t* cu, int32_t N, int32_t H_v, int32_t V, bool has_s0, int cus,
                SplitPlan& out) {
  PlanKey key{std::vector<int32_t>(cu, cu + N + 1), H_v, V, has_s0, cus};
  {
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    for (size_t i = 0; i < g_cache.size(); ++i)
      if (g_cache[i].key == key) {
        CachedPlan hit = g_cache[i];
        g_cache.erase(g_cache.begin() + (int64_t)i);
        g_cache.push_back(hit);
        out = hit.plan;
        return hit.split;
      }
  }
  SplitPlan plan;
  const bool split = plan_split_uncached(cu, N, H_v, V, has_s0, cus, plan);
  {
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    if (g_cache.size() >= kCacheSize) g_cache.erase(g_cache.begin());
    g_cache.push_back(CachedPlan{std::move(key), split, plan});
  }
  out = std::move(plan);
  return split;
}

static bool plan_split_uncached(const int32_t* cu, int32_t N, int32_t H_v, int32_t V, bool has_s0, int cus,
                                SplitPlan& out) {
  const int tiles2 = V / 128, tiles1 = 1 + V / 128;
  const int pmax = max_prefix_segments(H_v, V, cus);
  if (pmax == 0) return false;
  std::vector<int64_t> chunks(N);
  int64_t cmax = 0;
  for (int32_t n = 0; n < N; ++n) {
    chunks[n] = ((int64_t)cu[n + 1] - cu[n] + 63) / 64;
    cmax = std::max(cmax, chunks[n]);
  }
  // a forward pass over segments of these lengths, longest first
  auto forward = [&](std::vector<int64_t> lens) {
    std::sort(lens.begin(), lens.end(), std::greater<int64_t>());
    std::vector<Group> groups;
    for (int64_t c : lens) groups.push_back(Group{(double)c, (int64_t)H_v * tiles2});
    return makespan(groups, cus);
  };
  const double base = forward(chunks);
  // Every chunk runs forward once, and no schedule beats that work spread
  // evenly over the units: a run already within 15% of it is not split (and
  // the search below, costly for thousands of samples, is skipped).
  double work = 0.0;
  for (int64_t c : chunks) work += (double)c * H_v * tiles2;
  if (0.85 * base < work / cus) return false;
  // A sample of more than seg chunks is cut into a first segment of `first`
  // chunks (run forward in pass 1) and segments of seg chunks after it.
  auto n_segs = [](int64_t c, int64_t seg, int64_t first) -> int64_t {
    return c > seg ? 1 + (c - first + seg - 1) / seg : 1;
  };
  double best = base;
  int64_t best_seg = 0, best_first = 0;
  for (int parts = 2; parts <= 16; ++parts) {
    const int64_t even = (cmax + parts - 1) / parts;  // chunks per segment, all equal
    if (even < 4) break;
    // The first segment runs forward in pass 1 beside the maps, which cost
    // about 0.7 of a forward chunk each: a shorter first segment (the others
    // longer, so that the longest sample keeps `parts` segments) can end
    // pass 1 with the maps.
    for (const int64_t first : {even, (4 * even + 4) / 5, (3 * even + 3) / 4, (2 * even + 2) / 3}) {
      const int64_t seg = first == even ? even : (cmax - first + parts - 2) / (parts - 1);
      std::vector<int64_t> lens2, fwd1;
      int64_t n_maps = 0, longest_chain = 0;
      for (int32_t n = 0; n < N; ++n) {
        const int64_t s = n_segs(chunks[n], seg, first);
        if (s == 1) {
          lens2.push_back(chunks[n]);
          continue;
        }
        fwd1.push_back(first);
        n_maps += s - 2;
        longest_chain = std::max(longest_chain, s - 2);
        for (int64_t j = 1; j < s; ++j) lens2.push_back(std::min(seg, chunks[n] - first - (j - 1) * seg));
      }
      const int64_t n_pass1 = (int64_t)fwd1.size() + n_maps;
      if (n_pass1 == 0 || n_pass1 > pmax) continue;
      // pass 1: the forward segments first, then the maps; a map chunk skips
      // q, the output and P: about 0.7 of a forward chunk; a chain step costs
      // about one chunk
      std::vector<Group> p1;
      for (int64_t c : fwd1) p1.push_back(Group{(double)c, (int64_t)H_v * tiles2});
      p1.push_back(Group{0.7 * (double)seg, n_maps * H_v * tiles1});
      const double t = makespan(p1, cus) + (double)longest_chain + forward(lens2);
      if (t < best) {
        best = t;
        best_seg = seg;
        best_first = first;
      }
    }
  }
  if (best_seg == 0 || best > 0.85 * base) return false;

  // ---- the plan: a first segment of best_first chunks, then segments of best_seg --
  struct Seg {
    int32_t begin, end, n, j, s;
  };
  std::vector<Seg> segs;
  for (int32_t n = 0; n < N; ++n) {
    const int64_t s = n_segs(chunks[n], best_seg, best_first);
    // chunk where segment j starts: 0, first, first + seg, ...
    auto start = [&](int64_t j) { return j == 0 ? 0 : best_first + (j - 1) * best_seg; };
    for (int64_t j = 0; j < s; ++j) {
      const int32_t b = (int32_t)(cu[n] + 64 * start(j));
      const int32_t e = j + 1 < s ? (int32_t)(cu[n] + 64 * start(j + 1)) : cu[n + 1];
      segs.push_back({b, e, n, (int32_t)j, (int32_t)s});
    }
  }
  out.n_seg = (int)segs.size();
  out.n_prefix = 0;
  out.n_fwd = 0;
  out.n_chain = 0;
  for (const Seg& g : segs) {
    if (g.s > 1 && g.j + 1 < g.s) ++out.n_prefix;
    if (g.s > 1 && g.j == 0) ++out.n_fwd;
    if (g.s > 2 && g.j == 0) ++out.n_chain;
  }
  out.ints.assign((size_t)out.off_sample() + out.n_seg, 0);
  int32_t* I = out.ints.data();
  for (int i = 0; i < out.n_seg; ++i) I[i] = segs[i].begin;
  I[out.n_seg] = segs.back().end;
  // pass 2 longest first, then the segments pass 1 runs forward
  auto in_pass1 = [&](int32_t x) { return segs[x].s > 1 && segs[x].j == 0; };
  std::vector<int32_t> order(out.n_seg);
  for (int i = 0; i < out.n_seg; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    if (in_pass1(x) != in_pass1(y)) return in_pass1(y);
    return segs[x].end - segs[x].begin > segs[y].end - segs[y].begin;
  });
  std::copy(order.begin(), order.end(), I + out.off_order());
  int fwd = 0, map = 0, later = 0, chain = 0;
  for (int i = 0; i < out.n_seg; ++i) {
    const Seg& g = segs[i];
    if (g.j == 0 && g.s > 2) {  // the chain of this sample: from s_1's start through its maps
      int32_t* c = I + out.off_chains() + 4 * chain++;
      c[0] = later;
      c[1] = map;
      c[2] = g.s - 2;
      c[3] = later + 1;
    }
    I[out.off_s0ref() + i] = g.j == 0 ? (has_s0 ? -2 - g.n : -1) : later++;
    I[out.off_sfmap() + i] = g.j + 1 == g.s ? g.n : -1;
    I[out.off_sample() + i] = g.n;
    if (g.s > 1 && g.j == 0) I[out.off_pre() + fwd++] = i;
    if (g.j > 0 && g.j + 1 < g.s) I[out.off_pre() + out.n_fwd + map++] = i;
  }
  return true;
}


}  // namespace gdn
