// fp32 instances of the filter/sample and argmax kernels, and the launchers
// that pick a dtype's instances.
#include "qs_filter.hpp"

namespace qs {

// Slice length of the streamed pass: V split in 16, rounded up to 32 tokens.
int seg_for(int V) {
  int s = (V + kWaves - 1) / kWaves;
  return (s + 31) & ~31;
}

hipError_t launch_filter_bf16(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_filter_f32_proc(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_filter_f32_sort(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_filter_f32_topn(const FilterArgs& a, bool sample, int B, hipStream_t st);
hipError_t launch_argmax_bf16(const ArgmaxArgs& a, int B, hipStream_t st);

hipError_t launch_filter(const FilterArgs& a, int dtype, bool sample, int B, hipStream_t st) {
  if (dtype == QS_F32) {
    if (a.p_on) return launch_filter_f32_proc(a, sample, B, st);
    if (a.top_n > 0) return launch_filter_f32_topn(a, sample, B, st);
    if (a.flags & QS_FLAG_SORT_SUBSET) return launch_filter_f32_sort(a, sample, B, st);
    return sample ? launch_dt<0, true, 0, false>(a, B, st) : launch_dt<0, false, 0, false>(a, B, st);
  }
  return launch_filter_bf16(a, sample, B, st);
}

hipError_t launch_argmax(const ArgmaxArgs& a, int dtype, int B, hipStream_t st) {
  if (dtype == QS_F32) return launch_argmax_dt<0>(a, B, st);
  return launch_argmax_bf16(a, B, st);
}

}  // namespace qs
