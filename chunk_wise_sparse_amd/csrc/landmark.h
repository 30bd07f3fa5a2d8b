// Landmark of the chunk still being filled during decode (landmark.hip), called by the C ABI in
// hils_api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

struct PartialLmkArgs {
  const void* k_cache;     // [B, Hk, Lmax, d]
  void* lmk;               // [B, Hk, N, d], N = ceil(Lmax / C); row floor((kv_len - 1) / C) written
  const int32_t* kv_len;   // [B], clamped to [1, Lmax]
  int B, Hk, Lmax, N, C;
};

template <typename T, int D>
hipError_t launch_partial_landmark(const PartialLmkArgs& a, hipStream_t st);

}  // namespace hils
