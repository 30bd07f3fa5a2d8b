// HoPE: the rotary position encoding on the dimensions inside the pre-training window, none on
// the others [HiLS Attention explainer (molayo1419.me), "Engineering details", hierarchical
// positional encoding].  Pair (2i, 2i+1) of a row at position p is turned by the angle
// p * theta_i, theta_i = base^(-2i/d), when its wavelength 2 pi / theta_i fits the pre-training
// window (which pairs, and theta, come from the host).
//
// A workgroup takes 16 (32 for bf16 at d = 64) consecutive positions of one sequence: it forms each (position, pair)
// cosine and sine once, the angle reduced modulo 2 pi in fp64 (positions reach millions of
// radians at the highest frequency), into LDS, then rotates those rows of every head with
// 16-byte loads and stores (four heads' loads in flight together), in fp32, rounding once to
// the dtype.
#include "hils_device.h"
#include "hope.h"

namespace hils {

// Positions per workgroup: 16, or more when a row has fewer than 16 16-byte vectors, so that
// the 256 threads cover the rows of one head with whole vectors.
template <typename T, int D>
constexpr int hope_rows() { return D * (int)sizeof(T) / 16 >= 16 ? 16 : 256 / (D * (int)sizeof(T) / 16); }

template <typename T, int D>
__global__ __launch_bounds__(256) void hope_rotate_kernel(const HopeArgs a) {
  constexpr int NP = D / 2;                      // pairs per row
  constexpr int VE = 16 / (int)sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = D / VE;                    // vectors per row
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  constexpr int kHopeRows = hope_rows<T, D>();
  __shared__ float2 cs[kHopeRows][NP];
  const int b = blockIdx.y, p0 = blockIdx.x * kHopeRows, tid = threadIdx.x;
  const int pos_b = a.positions ? a.positions[b] : a.pos0;
  for (int v = tid; v < kHopeRows * NP; v += 256) {
    const int r = v / NP, i = v % NP;
    float c = 1.f, s = 0.f;
    if ((a.rotated >> i) & 1ull) {
      const double ang = (double)(pos_b + p0 + r) * a.theta[i];
      const double red = ang - kTwoPi * rint(ang / kTwoPi);
      c = (float)cos(red);
      s = (float)sin(red);
    }
    cs[r][i] = make_float2(c, s);
  }
  __syncthreads();
  typedef T vecT __attribute__((ext_vector_type(VE)));
  constexpr int NVT = kHopeRows * VPR / 256;     // vectors per thread and head (1 or 2)
  constexpr int HU = 4;                          // heads per step: their loads go out together
  static_assert(NVT >= 1 && kHopeRows * VPR == 256 * NVT, "tile does not split over the threads");
  T* xs = static_cast<T*>(a.x);
  for (int h0 = 0; h0 < a.H; h0 += HU) {
    vecT e[HU][NVT];
#pragma unroll
    for (int u = 0; u < HU; ++u)
#pragma unroll
      for (int n = 0; n < NVT; ++n) {
        const int v = tid + 256 * n, r = v / VPR, pv = v % VPR;
        if (h0 + u < a.H && p0 + r < a.L)
          e[u][n] = *reinterpret_cast<const vecT*>(xs + (((size_t)b * a.H + h0 + u) * a.L + p0 + r) * D + pv * VE);
      }
#pragma unroll
    for (int u = 0; u < HU; ++u)
#pragma unroll
      for (int n = 0; n < NVT; ++n) {
        const int v = tid + 256 * n, r = v / VPR, pv = v % VPR;
        if (h0 + u < a.H && p0 + r < a.L) {
#pragma unroll
          for (int j = 0; j < VE / 2; ++j) {
            const float2 t = cs[r][pv * (VE / 2) + j];
            const float x0 = to_f32(e[u][n][2 * j]), y0 = to_f32(e[u][n][2 * j + 1]);
            e[u][n][2 * j] = from_f32<T>(x0 * t.x - y0 * t.y);
            e[u][n][2 * j + 1] = from_f32<T>(x0 * t.y + y0 * t.x);
          }
          *reinterpret_cast<vecT*>(xs + (((size_t)b * a.H + h0 + u) * a.L + p0 + r) * D + pv * VE) = e[u][n];
        }
      }
  }
}

template <typename T, int D>
hipError_t launch_hope_rotate(const HopeArgs& a, hipStream_t st) {
  constexpr int RB = hope_rows<T, D>();
  const dim3 grid((unsigned)((a.L + RB - 1) / RB), (unsigned)a.B);
  hipLaunchKernelGGL((hope_rotate_kernel<T, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_hope_rotate<bf16, 64>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<bf16, 128>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<float, 64>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<float, 128>(const HopeArgs&, hipStream_t);

}  // namespace hils
