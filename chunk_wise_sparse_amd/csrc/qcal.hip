// Q-Cal, the low-rank query calibration delta_q = W_up (W_down h)
// [HiLS Attention explainer (molayo1419.me), "Engineering details", Q-Cal item].
//
// Prefill splits it in two: this file computes the rank-r code t = W_down h for every token
// (an HBM-bound pass over h, on MFMA), and the selection kernel applies W_up per head inside
// its query tile.  Decode does both halves here for one token per sequence.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// t[tok, a] = sum_D h[tok, D] * W_down[a, D], fp32.  One workgroup = 64 tokens, one wave = 16.
// A operand = h rows (tokens), B operand = W_down rows (code index a), contraction over D.
// Each lane owns a 64-byte run of its row per 256-byte block: k index within the block is
// g * (4 * VL) + e, the same for A and B.
template <typename T>
__global__ __launch_bounds__(256) void prefill_qcal_code_kernel(const T* __restrict__ h,
                                                                const T* __restrict__ w_down,
                                                                float* __restrict__ t_out,
                                                                int n_tok, int D, int r) {
  constexpr int VL = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int SUB = VL / KPL;             // MFMA steps per vector
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int tok0 = blockIdx.x * 64 + wave * 16;
  const int nb = (r + 15) >> 4;             // code blocks of 16
  const T* hrow = h + (size_t)(tok0 + m) * D + g * 4 * VL;

  f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
  for (int base = 0; base < D; base += 16 * VL) {
    typedef T vecT __attribute__((ext_vector_type(VL)));
    vecT av[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) av[u] = *reinterpret_cast<const vecT*>(hrow + base + u * VL);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (cb >= nb) break;
      const int a = cb * 16 + m;
      vecT bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (a < r) bv[u] = *reinterpret_cast<const vecT*>(w_down + (size_t)a * D + base + g * 4 * VL + u * VL);
        else bv[u] = vecT{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int e = 0; e < SUB; ++e) {
          typename Mfma<T>::frag fa, fb;
          if constexpr (KPL == 1) {
            fa = av[u][e];
            fb = bv[u][e];
          } else {
#pragma unroll
            for (int z = 0; z < KPL; ++z) { fa[z] = av[u][e * KPL + z]; fb[z] = bv[u][e * KPL + z]; }
          }
          acc[cb] = Mfma<T>::mma(fa, fb, acc[cb]);
        }
      }
    }
  }
  // D[tok][a]: lane holds column a = 16cb + m, rows (tokens) 4g + rr.
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if (cb >= nb) break;
    const int a = cb * 16 + m;
    if (a < r) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) t_out[(size_t)(tok0 + 4 * g + rr) * r + a] = acc[cb][rr];
    }
  }
}

template <typename T>
hipError_t launch_prefill_qcal_code(const T* h, const T* w_down, float* t_out, int n_tok, int D,
                                    int r, hipStream_t st) {
  hipLaunchKernelGGL(prefill_qcal_code_kernel<T>, dim3(n_tok / 64), dim3(256), 0, st, h, w_down,
                     t_out, n_tok, D, r);
  return hipGetLastError();
}

template hipError_t launch_prefill_qcal_code<bf16>(const bf16*, const bf16*, float*, int, int, int, hipStream_t);
template hipError_t launch_prefill_qcal_code<float>(const float*, const float*, float*, int, int, int, hipStream_t);

}  // namespace hils

