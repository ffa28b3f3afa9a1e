// f32 instances of the filter/sample kernel that also write each row's top-n
// tokens (their own translation unit: the other instances hold none of that
// code).
#include "qs_filter.hpp"

namespace qs {

hipError_t launch_filter_f32_topn(const FilterArgs& a, bool sample, int B, hipStream_t st) {
  return sample ? launch_dt<0, true, 0, true, true>(a, B, st)
                : launch_dt<0, false, 0, true, true>(a, B, st);
}

}  // namespace qs
