// bf16 instances of the filter/sample and argmax kernels.
#include "qs_filter.hpp"

namespace qs {

hipError_t launch_filter_bf16_proc(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_filter_bf16_sort(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_filter_bf16_topn(const FilterArgs& a, bool sample, int B, hipStream_t st);

hipError_t launch_filter_bf16(const FilterArgs& a, bool sample, int B, hipStream_t st) {
  if (a.p_on) return launch_filter_bf16_proc(a, sample, B, st);
  if (a.top_n > 0) return launch_filter_bf16_topn(a, sample, B, st);
  if (a.flags & QS_FLAG_SORT_SUBSET) return launch_filter_bf16_sort(a, sample, B, st);
  return sample ? launch_dt<1, true, 0, false>(a, B, st) : launch_dt<1, false, 0, false>(a, B, st);
}

bool filter_row_resident(int dtype, int V) {
  return resident_steps(V) <= kResidentTier[dtype == 1 ? 1 : 0][1];
}

hipError_t launch_argmax_bf16(const ArgmaxArgs& a, int B, hipStream_t st) {
  return launch_argmax_dt<1>(a, B, st);
}

}  // namespace qs
