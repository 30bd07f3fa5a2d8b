// HoPE: the rotary position encoding on the dimensions inside the pre-training window, none on
// the others [HiLS Attention explainer (molayo1419.me), "Engineering details", hierarchical
// positional encoding].  Pair (2i, 2i+1) of a row at position p is turned by the angle
// p * theta_i, theta_i = base^(-2i/d), when its wavelength 2 pi / theta_i fits the pre-training
// window (which pairs, and theta, come from the host).
//
// A workgroup takes 16 consecutive positions of one sequence: it forms each (position, pair)
// cosine and sine once, the angle reduced modulo 2 pi in fp64 (positions reach millions of
// radians at the highest frequency), into LDS, then rotates the 16 rows of every head with
// 16-byte loads and stores, in fp32, rounding once to the dtype.
#include "hils_device.h"
#include "hope.h"

namespace hils {

constexpr int kHopeRows = 16;

template <typename T, int D>
__global__ __launch_bounds__(256) void hope_rotate_kernel(const HopeArgs a) {
  constexpr int NP = D / 2;                      // pairs per row
  constexpr int VE = 16 / (int)sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = D / VE;                    // vectors per row
  constexpr double kTwoPi = 6.283185307179586476925286766559;
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
  T* xs = static_cast<T*>(a.x);
  for (int h = 0; h < a.H; ++h) {
    T* rows = xs + (((size_t)b * a.H + h) * a.L + p0) * D;
    for (int v = tid; v < kHopeRows * VPR; v += 256) {
      const int r = v / VPR, pv = v % VPR;
      if (p0 + r >= a.L) continue;
      vecT* ptr = reinterpret_cast<vecT*>(rows + (size_t)r * D + pv * VE);
      vecT e = *ptr;
#pragma unroll
      for (int j = 0; j < VE / 2; ++j) {
        const float2 t = cs[r][pv * (VE / 2) + j];
        const float x0 = to_f32(e[2 * j]), y0 = to_f32(e[2 * j + 1]);
        e[2 * j] = from_f32<T>(x0 * t.x - y0 * t.y);
        e[2 * j + 1] = from_f32<T>(x0 * t.y + y0 * t.x);
      }
      *ptr = e;
    }
  }
}

template <typename T, int D>
hipError_t launch_hope_rotate(const HopeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.L + kHopeRows - 1) / kHopeRows), (unsigned)a.B);
  hipLaunchKernelGGL((hope_rotate_kernel<T, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_hope_rotate<bf16, 64>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<bf16, 128>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<float, 64>(const HopeArgs&, hipStream_t);
template hipError_t launch_hope_rotate<float, 128>(const HopeArgs&, hipStream_t);

}  // namespace hils
