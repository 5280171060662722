// split_plan.h -- host planning of segment splits for packed chunk-rule runs.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace gdn {

// A packed run cut into segments (see split_plan.cpp).  Index arrays, laid
// out as the device copy: seg_cu [n_seg + 1] | order [n_seg] | s0_ref [n_seg] |
// sf_map [n_seg] | pass1 [n_prefix] | chains [4 n_chain] | sample [n_seg]
// (the sample each segment cuts, whose chunk records it reads).  order lists
// the n_seg - n_fwd segments of pass 2 longest first, then the n_fwd first
// segments that pass 1 runs forward; pass1 lists those n_fwd segments, then
// the n_prefix - n_fwd segments whose affine maps pass 1 forms.
struct SplitPlan {
  int n_seg = 0, n_prefix = 0, n_fwd = 0, n_chain = 0;
  std::vector<int32_t> ints;
  int off_order() const { return n_seg + 1; }
  int off_s0ref() const { return off_order() + n_seg; }
  int off_sfmap() const { return off_s0ref() + n_seg; }
  int off_pre() const { return off_sfmap() + n_seg; }
  int off_chains() const { return off_pre() + n_prefix; }
  int off_sample() const { return off_chains() + 4 * n_chain; }
};

// Most pass-1 segments (forward and map) a plan uses for H_v heads of V
// columns on cus units.
int max_prefix_segments(int32_t H_v, int32_t V, int cus);
// Upper bound of SplitPlan::ints.size().
int64_t split_plan_ints_max(int n_seg, int n_prefix);
// Plans the split of the n samples at host offsets cu (cu[0] = 0, non-
// decreasing); false when running them unsplit is expected to be as fast.
bool plan_split(const int32_t* cu, int32_t n, int32_t H_v, int32_t V, bool has_s0, int cus,
                SplitPlan& out);

}  // namespace gdn
