// bf16 instances of the filter/sample kernel with logit processors applied in
// the kernel (their own translation unit: they build in parallel with the
// plain ones).
#include "qs_filter.hpp"

namespace qs {

hipError_t launch_filter_bf16_proc1(const FilterArgs& a, bool sample, int B, hipStream_t st);

// repetition and presence penalties alone take the instances that know it
// (qs_filter_bf16_proc1.hip); these instances also hold the sorted-subset
// switch
hipError_t launch_filter_bf16_proc(const FilterArgs& a, bool sample, int B, hipStream_t st) {
  if (a.p_freq == nullptr && a.p_bias_ids == nullptr && !(a.flags & QS_FLAG_SORT_SUBSET))
    return launch_filter_bf16_proc1(a, sample, B, st);
  return sample ? launch_dt<1, true, 2, true>(a, B, st) : launch_dt<1, false, 2, true>(a, B, st);
}

}  // namespace qs
