// Landmark of the chunk still being filled during decode.  A landmark token closes each chunk
// [HiLS Attention explainer (molayo1419.me), "Core idea: landmark tokens and hierarchical
// factorisation"], so the chunk that holds the newest key has none until it reaches C keys; its
// stand-in is the mean of its keys so far, recomputed from the cache at every step (no running
// state), and written into that chunk's landmark row.
//
// One workgroup per (sequence, key/value head): thread (g, v) owns 16-byte vector v of the row and
// sums, in fp32, the chunk's rows g, g + RG, ... (RG row groups, all rows' loads in flight
// together); the row groups' sums are then added in group order, divided by the key count and
// rounded once to the dtype.  The sum order is fixed, so results are bitwise reproducible.
#include "hils_device.h"
#include "landmark.h"

namespace hils {

template <typename T, int D>
__global__ __launch_bounds__(256) void partial_landmark_kernel(const PartialLmkArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector
  constexpr int VPR = D / VE;                  // vectors per row
  constexpr int RG = 256 / VPR;                // row groups
  constexpr int MAXI = (128 + RG - 1) / RG;    // rows per group for chunks of up to 128 keys
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float part[RG][D];
  const int pair = blockIdx.x, b = pair / a.Hk;
  const int tid = threadIdx.x, g = tid / VPR, v = tid % VPR;
  const int n_keys = min(max(a.kv_len[b], 1), a.Lmax);
  const int j = (n_keys - 1) / a.C, n = n_keys - j * a.C;    // 1 <= n <= C
  const T* rows = static_cast<const T*>(a.k_cache) + ((size_t)pair * a.Lmax + (size_t)j * a.C) * D + v * VE;
  vecT x[MAXI];
#pragma unroll
  for (int it = 0; it < MAXI; ++it) {
    const int r = g + RG * it;
    x[it] = *reinterpret_cast<const vecT*>(rows + (size_t)min(r, n - 1) * D);
  }
  float acc[VE];
#pragma unroll
  for (int z = 0; z < VE; ++z) acc[z] = 0.f;
#pragma unroll
  for (int it = 0; it < MAXI; ++it) {
    if (g + RG * it < n) {
#pragma unroll
      for (int z = 0; z < VE; ++z) acc[z] += to_f32(x[it][z]);
    }
  }
#pragma unroll
  for (int z = 0; z < VE; ++z) part[g][v * VE + z] = acc[z];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < RG; ++q) s += part[q][tid];
    T* out = static_cast<T*>(a.lmk) + ((size_t)pair * a.N + j) * D;
    out[tid] = from_f32<T>(s / (float)n);
  }
}

template <typename T, int D>
hipError_t launch_partial_landmark(const PartialLmkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((partial_landmark_kernel<T, D>), dim3(a.B * a.Hk), dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_partial_landmark<bf16, 64>(const PartialLmkArgs&, hipStream_t);
template hipError_t launch_partial_landmark<bf16, 128>(const PartialLmkArgs&, hipStream_t);
template hipError_t launch_partial_landmark<float, 64>(const PartialLmkArgs&, hipStream_t);
template hipError_t launch_partial_landmark<float, 128>(const PartialLmkArgs&, hipStream_t);

}  // namespace hils
