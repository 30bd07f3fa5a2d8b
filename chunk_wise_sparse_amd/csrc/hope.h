// HoPE rotation launcher (hope.hip), called by the C ABI in hils_api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

// Per-call constants: theta_i = base^(-2i/d) in fp64 and which pairs carry the rotation, both
// formed on the host (d / 2 <= 64 pairs).
struct HopeArgs {
  void* x;                  // [B, H, L, d], rotated in place
  const int32_t* positions; // [B] position of row 0 of each sequence, or NULL: pos0
  int B, H, L, pos0;
  uint64_t rotated;         // bit i: pair (2i, 2i+1) is rotated
  double theta[64];
};

template <typename T, int D>
hipError_t launch_hope_rotate(const HopeArgs& a, hipStream_t st);

}  // namespace hils
