// fp32 instances of the filter/sample kernel with logit processors applied in
// the kernel (their own translation unit: they build in parallel with the
// plain ones).
#include "qs_filter.hpp"

namespace qs {

hipError_t launch_filter_f32_proc(const FilterArgs& a, bool sample, int B, hipStream_t st) {
  return sample ? launch_dt<0, true, 2, true>(a, B, st) : launch_dt<0, false, 2, true>(a, B, st);
}

}  // namespace qs
