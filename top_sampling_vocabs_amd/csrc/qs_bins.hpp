// Exact bf16 value bins shared by the value-histogram kernels: one bin per
// bf16 value of magnitude in [2^-24, 512) and sign, 16 bins below that range
// and one above it (magnitudes >= 512, infinities, NaN) per sign.
//
// Bin of a token with raw bits d: i = min(sat(mag - (kMagLo - 16)), kTop) with
// mag = d & 0x7FFF, plus kSide for a negative sign. Exact values are also
// ranked in descending order (rho = 0 is the largest, 511.x); a run of 16
// consecutive ranks lies in one binade, so its values are equally spaced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

namespace sel {
constexpr uint32_t kMagLo = 0x3380u;            // magnitude bits of 2^-24
constexpr uint32_t kExact = 33u * 128u;         // exact bins per sign: 33 binades
constexpr uint32_t kTop = 16u + kExact;         // bin of the magnitudes >= 512 (and inf, NaN)
constexpr uint32_t kSide = 4256u;               // bins per sign, a multiple of 16
constexpr int kBins = 2 * (int)kSide;           // 8512 bins
constexpr int kRho = 2 * (int)kExact;           // exact values in descending order
constexpr int kRuns = kRho / 16;                // 528 runs of 16 consecutive values
constexpr int kTab = 2048;                      // weights from the maximum to the boundary
constexpr uint32_t kNone = 0xFFFFFFFFu;
static_assert(kMagLo + kExact == 0x4400u, "the exact bins end at 512");
static_assert((kMagLo & 127u) == 0u && kSide % 16u == 0u, "runs of 16 stay in one binade");

// Value rank rho (0 = the largest exact value) of exact bin j of a side:
// positive j = 16 .. kTop-1 -> rho = kTop-1-j; negative -> kExact + j - 16.
// A run of 16 ranks starting at 16 t covers one aligned group of 16 bins.
__device__ __forceinline__ uint32_t run_bin0(int t) {
  return t < (int)(kExact / 16) ? kTop - 16u - 16u * (uint32_t)t
                                : kSide + 16u + 16u * (uint32_t)(t - (int)(kExact / 16));
}
// bf16 magnitude bits of rank rho, and its sign
__device__ __forceinline__ uint32_t rho_mag(uint32_t rho) {
  return rho < kExact ? kMagLo + kExact - 1u - rho : kMagLo + (rho - kExact);
}
__device__ __forceinline__ double rho_value(uint32_t rho) {
  const uint32_t bits = rho_mag(rho) | (rho < kExact ? 0u : 0x8000u);
  return (double)__uint_as_float(bits << 16);
}
}  // namespace sel

}  // namespace qs
