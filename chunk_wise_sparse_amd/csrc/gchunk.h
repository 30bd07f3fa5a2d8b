// Chunk sizes other than 64 (gchunk.hip), called by the C ABI in hils_api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

constexpr int kGcMaxChunks = 8192;             // chunks per sequence (scores kept in LDS)

struct GcArgs {
  const void* q;             // [B, H, L, d]
  const void* key;           // [B, Hk, L, d]
  const void* val;           // [B, Hk, L, d]
  const void* lmk;           // [B, Hk, N, d], N = ceil(L / C)
  const void* w_up;          // [H * d, r] (r > 0)
  const float* tcode;        // Q-Cal code rows, tstride floats apart (r > 0)
  void* o;                   // like q; NULL: selection only (idx / w written, no attention)
  int32_t* idx;              // [B, H, L, k]
  float* w;                  // [B, H, L, k]
  int B, H, G, L, N, C, k, r, tstride, force_local;
  float scale;
};

template <typename T, int D>
hipError_t launch_gchunk(const GcArgs& a, hipStream_t st);

}  // namespace hils
