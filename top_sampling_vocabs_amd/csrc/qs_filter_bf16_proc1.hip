// bf16 instances of the filter/sample kernel with repetition and presence
// penalties alone applied in the kernel (no frequency penalty, no bias list:
// the edit needs no per-token table lookups).
#include "qs_filter.hpp"

namespace qs {

hipError_t launch_filter_bf16_proc1(const FilterArgs& a, bool sample, int B, hipStream_t st) {
  return sample ? launch_dt<1, true, 1, false>(a, B, st) : launch_dt<1, false, 1, false>(a, B, st);
}

}  // namespace qs
